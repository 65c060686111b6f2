// C ABI of libloopq (declared in include/loopq.h): host-side validation,
// workspace planning and kernel dispatch on the caller's stream.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/loopq.h"
#include "loopq_internal.h"

using namespace loopq;

namespace {

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? LOOPQ_OK : LOOPQ_ERR_HIP; }

// ---------------------------------------------------------------------------
// Timing hooks: while enabled, each hot-path launch is bracketed by two HIP
// events recorded on its own stream; loopq_timing_read sums their elapsed
// times per kernel id.  Events are pooled and reused after a read or reset.
// ---------------------------------------------------------------------------
struct TimingRec {
  int kid;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimingRec> g_timing_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Set while loopq_w4a4_linear_noalloc runs on this thread: its launches take
// no timing records (a record may create HIP events, which allocate).
thread_local bool t_no_alloc = false;

struct TimingScope {
  bool on = false;
  TimingRec rec{};
  hipStream_t s;
  TimingScope(int kid, hipStream_t stream) : s(stream) {
    if (t_no_alloc) return;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (!g_timing_on) return;
    rec.kid = kid;
    rec.start = pooled_event();
    rec.stop = pooled_event();
    if (!rec.start || !rec.stop) return;
    on = hipEventRecord(rec.start, s) == hipSuccess;
  }
  ~TimingScope() {
    if (!on) return;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (hipEventRecord(rec.stop, s) == hipSuccess) g_timing_recs.push_back(rec);
  }
};

void recycle_locked() {
  for (auto& r : g_timing_recs) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_timing_recs.clear();
}

// The GEMM each activation width runs on: W4A4 on the fp6-operand kernel
// (e2m3 holds the codes -7..7 exactly), W4A8 on the INT8 kernel.
int code_format(int bits_a) { return bits_a == 4 ? kCodesTiledF6 : kCodesTiledI8; }

// Internal buffers of the quantize -> GEMM path, carved from the caller's
// workspace for `chunks` chunks of `rows` rows each:
//   codes  : chunks * padded(rows) rows in the tiled layout, row_bytes(K)
//            per row (enough for either tiled format)
//   scales : fp32 group-major, chunks * padded(rows) columns
//   wexp   : weights expanded to fp6 operands (W4A4 kernel only)
// The same region also holds all chunks * rows rows as one contiguous tiled
// matrix (padded(chunks * rows) <= chunks * padded(rows)).
struct ActBuffers {
  void* codes;
  float* scales;
  void* wexp;
  float* xt;  // x~ rows of the few-row path
  int ld;
};

int64_t row_bytes(int64_t K) {
  const int64_t f6 = group_pairs(K) * (kF6BlockBytes / 32);
  return K > f6 ? K : f6;
}
size_t codes_region(int64_t chunks, int64_t rows, int64_t K) {
  return align256((size_t)(chunks * padded_rows(rows) * row_bytes(K)));
}
size_t scales_region(int64_t chunks, int64_t rows, int64_t K) {
  return align256((size_t)((K / 32) * chunks * padded_rows(rows) * 4));
}
size_t wexp_region(int64_t K, int64_t N, int fmt) {
  return fmt == kCodesTiledF6 ? align256((size_t)(padded_cols(N) / 32 * group_pairs(K) * kF6BlockBytes)) : 0;
}
// x~ rows of the few-row (decode) path: one launch of all chunks * rows rows
// when they are few enough, else launches of `rows` rows
size_t xt_region(int64_t chunks, int64_t rows, int64_t K) {
  if (rows > kDecodeMaxRows) return 0;
  const int64_t r = chunks * rows <= kDecodeMaxRows ? chunks * rows : rows;
  return align256((size_t)(r * K * 4));
}
size_t act_bytes(int64_t chunks, int64_t rows, int64_t K, int64_t N, int fmt) {
  return codes_region(chunks, rows, K) + scales_region(chunks, rows, K) + wexp_region(K, N, fmt) +
         xt_region(chunks, rows, K);
}

// buffers of chunk c (rows rows each), or with all_rows > 0 the whole
// all_rows-row matrix starting at the region's base
ActBuffers carve(void* ws, int64_t chunks, int64_t rows, int64_t K, int64_t N, int64_t c,
                 int64_t all_rows) {
  ActBuffers b;
  char* base = reinterpret_cast<char*>(ws);
  const int64_t mp = padded_rows(rows);
  float* scales0 = reinterpret_cast<float*>(base + codes_region(chunks, rows, K));
  // regions: codes | scales | x~ rows (few-row path) | expanded weights
  b.xt = reinterpret_cast<float*>(base + codes_region(chunks, rows, K) + scales_region(chunks, rows, K));
  b.wexp = reinterpret_cast<char*>(b.xt) + xt_region(chunks, rows, K);
  if (all_rows > 0) {
    b.codes = base;
    b.scales = scales0;
    b.ld = (int)padded_rows(all_rows);
  } else {
    b.codes = base + (size_t)c * mp * row_bytes(K);
    b.scales = scales0 + (size_t)c * (K / 32) * mp;
    b.ld = (int)mp;
  }
  return b;
}

// the W4A4 kernel's weight operands, once per call (before its GEMMs, on the
// same stream)
hipError_t prepare_weights(const ActBuffers& b, int fmt, const void* w_codes, int K, int N, hipStream_t s) {
  if (fmt != kCodesTiledF6) return hipSuccess;
  return launch_expand_weights_f6(reinterpret_cast<const uint8_t*>(w_codes), K, N, b.wexp, s);
}

// GEMM stage on codes already in the internal layout `fmt`
hipError_t run_gemm(const ActBuffers& b, int fmt, int rows, int K, int N, const void* w_codes,
                    const void* w_scales, int gw, float* y, int32_t* dots, int mode, hipStream_t s,
                    const GemmSets* sets = nullptr) {
  const __half* wsc = reinterpret_cast<const __half*>(w_scales);
  if (fmt == kCodesTiledF6)
    return launch_gemm_f6(b.codes, b.scales, b.ld, rows, K, N, b.wexp, wsc, gw, y, dots, mode, s, sets);
  return launch_gemm(reinterpret_cast<const int8_t*>(b.codes), b.scales, b.ld, rows, K, N,
                     reinterpret_cast<const uint8_t*>(w_codes), wsc, gw, y, dots, mode, s, sets);
}

// ---------------------------------------------------------------------------
// Auxiliary stream (one per device, default priority) and events for the
// pipelined loop-sequential schedule: the quantizer of loop t + 1 runs on the
// auxiliary stream while the GEMM of loop t runs on the caller's stream.
// Enqueueing is serialized by a mutex; the caller's stream waits for every
// auxiliary launch it depends on, so stream order is preserved for the caller.
// ---------------------------------------------------------------------------
std::mutex g_launch_mu;
struct KernelState {
  int dev;
  const void* fn;
  int lds_set;
  std::vector<int> occ;  // (lds bytes, block, work-groups per CU) triples
};
std::vector<KernelState> g_kernels;
int g_ncu[64];

std::mutex g_pipe_mu;
struct DevicePipe {
  hipStream_t aux = nullptr;
  std::vector<hipEvent_t> events;
};
DevicePipe g_pipes[64];

hipError_t device_pipe(DevicePipe** out, int nevents) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  DevicePipe& p = g_pipes[dev];
  if (!p.aux) {
    e = hipStreamCreateWithFlags(&p.aux, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
  }
  while ((int)p.events.size() < nevents) {
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    p.events.push_back(ev);
  }
  *out = &p;
  return hipSuccess;
}

int32_t check_weights(int K, int N, int gw) {
  if (K <= 0 || N <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (K % 32 != 0) return LOOPQ_ERR_UNSUPPORTED;
  if (gw != 32 && gw != 128) return LOOPQ_ERR_UNSUPPORTED;
  return LOOPQ_OK;
}

int32_t check_transform(int K, const float* P1, int n1, const float* P2, int n2) {
  if ((P1 == nullptr) != (P2 == nullptr)) return LOOPQ_ERR_INVALID_ARG;
  if (P1 == nullptr) return LOOPQ_OK;
  if (n1 <= 0 || n2 <= 0) return LOOPQ_ERR_INVALID_ARG;
  if ((int64_t)n1 * n2 != K) return LOOPQ_ERR_UNSUPPORTED;
  if (n1 % 4 || n2 % 4 || n1 > 128 || n2 > 128) return LOOPQ_ERR_UNSUPPORTED;
  if (!aligned(P1, 4) || !aligned(P2, 4)) return LOOPQ_ERR_ALIGNMENT;
  if (!quant_plan_fits(K, n1, n2)) return LOOPQ_ERR_UNSUPPORTED;  // LDS of the fused kernel
  return LOOPQ_OK;
}

int32_t check_act(const void* x, int dtype, int M, int K, int bits_a) {
  if (M < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (K % 32 != 0) return LOOPQ_ERR_UNSUPPORTED;
  if (dtype != LOOPQ_F32 && dtype != LOOPQ_BF16) return LOOPQ_ERR_UNSUPPORTED;
  if (bits_a != 4 && bits_a != 8) return LOOPQ_ERR_UNSUPPORTED;
  if (M > 0 && x == nullptr) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(x, dtype == LOOPQ_F32 ? 16 : 8)) return LOOPQ_ERR_ALIGNMENT;
  return LOOPQ_OK;
}

// The GEMM addresses its operands with 32-bit buffer offsets: the step table
// of the activations (rows x K/32 fp32) and of the weights must stay below 2 GiB.
int32_t check_gemm_extent(int64_t rows, int K, int N, int gw) {
  const int64_t ga = K / 32;
  const int64_t gwn = (K + gw - 1) / gw;
  if (rows * ga * 4 >= ((int64_t)1 << 31)) return LOOPQ_ERR_UNSUPPORTED;
  if (padded_cols(N) * gwn * 2 >= ((int64_t)1 << 31)) return LOOPQ_ERR_UNSUPPORTED;
  return LOOPQ_OK;
}

bool clip_ok(float c) { return isfinite(c) && c > 0.0f; }

QuantArgs make_quant_args(const void* x, int dtype, int rows, int K, const float* P1, int n1,
                          const float* P2, int n2, int bits_a) {
  QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.rows = rows;
  a.K = K;
  a.bf16 = dtype == LOOPQ_BF16;
  a.P1 = P1;
  a.P2 = P2;
  a.n1 = n1;
  a.n2 = n2;
  a.rows_per_clip = rows > 0 ? rows : 1;
  a.qmax = bits_a == 4 ? 7 : 127;
  return a;
}

QuantArgs internal_quant_args(const void* x, int dtype, int rows, int K, const float* P1, int n1,
                              const float* P2, int n2, const ClipTable& clips, int rows_per_clip,
                              int bits_a, const ActBuffers& b) {
  QuantArgs a = make_quant_args(x, dtype, rows, K, P1, n1, P2, n2, bits_a);
  a.clips = clips;
  a.rows_per_clip = rows_per_clip;
  a.codes = reinterpret_cast<int8_t*>(b.codes);
  a.codes_fmt = code_format(bits_a);
  a.scales = b.scales;
  a.scales_gm = 1;
  a.scales_ld = b.ld;
  return a;
}

// Few rows (decode): the few-row kernel, in one launch where it can.
// x [rows][K] with row r taking clips.c[r / rows_per_clip].
hipError_t run_decode(const void* x, int dtype, int rows, int K, int N, const float* P1, int n1,
                      const float* P2, int n2, const ClipTable& clips, int rows_per_clip,
                      int bits_a, const void* w_codes, const void* w_scales, int gw, float* y,
                      const ActBuffers& b, hipStream_t s) {
  DecodeCall c;
  memset(&c, 0, sizeof(c));
  c.R = rows;
  c.K = K;
  c.N = N;
  c.clips = clips;
  c.rows_per_clip = rows_per_clip;
  c.qmax = bits_a == 4 ? 7 : 127;
  c.w = reinterpret_cast<const uint8_t*>(w_codes);
  c.sw = reinterpret_cast<const __half*>(w_scales);
  c.gw = gw;
  c.y = y;
  c.mode = 0;
  // one launch: a transform it repeats per work-group cheaply, or at most 4
  // rows quantized in place; otherwise the activations are quantized once
  // (transform items, then the plain quantizer, or the chunked quantizer for
  // a factor shape without items) and the kernel copies canonical codes
  const bool one = P1 != nullptr ? decode_transform_fused(rows, n1, n2) : rows <= 4;
  if (!one) {
    QuantArgs a = make_quant_args(x, dtype, rows, K, P1, n1, P2, n2, bits_a);
    a.clips = clips;
    a.rows_per_clip = rows_per_clip;
    a.codes = reinterpret_cast<int8_t*>(b.codes);
    a.codes_fmt = kCodesCanonical;
    a.scales = b.scales;
    a.scales_gm = 0;
    hipError_t e = hipSuccess;
    if (P1 != nullptr && decode_transform_items(n1, n2)) {
      {
        TimingScope ts(LOOPQ_KERNEL_QUANT_TRANSFORM, s);
        e = launch_decode_items(x, dtype == LOOPQ_BF16, P1, n1, P2, n2, rows, b.xt, s);
      }
      if (e != hipSuccess) return e;
      a.x = b.xt;
      a.bf16 = 0;
      a.P1 = a.P2 = nullptr;
      a.n1 = a.n2 = 0;
    }
    {
      TimingScope ts(a.P1 ? LOOPQ_KERNEL_QUANT_TRANSFORM : LOOPQ_KERNEL_QUANT_PLAIN, s);
      e = launch_quant_act(a, s);
    }
    if (e != hipSuccess) return e;
    c.a_codes = reinterpret_cast<const int8_t*>(b.codes);
    c.a_steps = b.scales;
  } else {
    c.x = x;
    c.bf16 = dtype == LOOPQ_BF16;
    c.P1 = P1;
    c.P2 = P2;
    c.n1 = n1;
    c.n2 = n2;
    // the codes the launch forms go to the workspace too (canonical), where
    // the other few-row form leaves them, for loopq_export_act_codes
    c.codes_out = reinterpret_cast<int8_t*>(b.codes);
    c.steps_out = b.scales;
  }
  TimingScope ts(LOOPQ_KERNEL_DECODE, s);
  return launch_decode(c, s);
}

// weight-stationary: quantize all `rows` rows, then one GEMM pass over the
// weights for all of them (few rows: the fused decode kernel)
int32_t linear_core(const void* x, int dtype, int rows, int K, int N, const float* P1, int n1,
                    const float* P2, int n2, const ClipTable& clips, int rows_per_clip, int bits_a,
                    const void* w_codes, const void* w_scales, int gw, float* y, void* ws,
                    int64_t ws_chunks, int64_t ws_rows, hipStream_t s, float* xt_out = nullptr) {
  ActBuffers b = carve(ws, ws_chunks, ws_rows, K, N, 0, rows);
  if (rows <= kDecodeMaxRows && !xt_out)
    return hip_status(run_decode(x, dtype, rows, K, N, P1, n1, P2, n2, clips, rows_per_clip, bits_a,
                                 w_codes, w_scales, gw, y, b, s));
  QuantArgs a = internal_quant_args(x, dtype, rows, K, P1, n1, P2, n2, clips, rows_per_clip,
                                    bits_a, b);
  a.xt_out = xt_out;
  const int fmt = code_format(bits_a);
  hipError_t e = prepare_weights(b, fmt, w_codes, K, N, s);
  if (e != hipSuccess) return LOOPQ_ERR_HIP;
  {
    TimingScope ts(P1 ? LOOPQ_KERNEL_QUANT_TRANSFORM : LOOPQ_KERNEL_QUANT_PLAIN, s);
    e = launch_quant_act(a, s);
  }
  if (e != hipSuccess) return LOOPQ_ERR_HIP;
  {
    TimingScope ts(LOOPQ_KERNEL_GEMM, s);
    e = run_gemm(b, fmt, rows, K, N, w_codes, w_scales, gw, y, nullptr, 0, s);
  }
  return hip_status(e);
}

// loop-sequential, pipelined: loop t's rows are quantized on the auxiliary
// stream and multiplied on the caller's stream as soon as they are ready, so
// the quantizer of loop t + 1 overlaps the GEMM of loop t
int32_t looped_pipelined(const void* x, int dtype, int T, int M, int K, int N, const float* P1,
                         int n1, const float* P2, int n2, const ClipTable& clips, int bits_a,
                         const void* w_codes, const void* w_scales, int gw, float* y, void* ws,
                         hipStream_t s, float* xt_out = nullptr) {
  const size_t esz = dtype == LOOPQ_F32 ? 4 : 2;
  if (M <= kDecodeMaxRows && !xt_out) {  // decode: one fused launch per loop, in loop order on `stream`
    for (int t = 0; t < T; ++t) {
      ClipTable one;
      memset(&one, 0, sizeof(one));
      one.c[0] = clips.c[t];
      const void* xt = reinterpret_cast<const char*>(x) + (size_t)t * M * K * esz;
      hipError_t e = run_decode(xt, dtype, M, K, N, P1, n1, P2, n2, one, M, bits_a, w_codes, w_scales,
                                gw, y + (size_t)t * M * N, carve(ws, T, M, K, N, t, 0), s);
      if (e != hipSuccess) return LOOPQ_ERR_HIP;
    }
    return LOOPQ_OK;
  }
  std::lock_guard<std::mutex> lk(g_pipe_mu);
  DevicePipe* p = nullptr;
  if (device_pipe(&p, T + 1) != hipSuccess) return LOOPQ_ERR_HIP;
  const int fmt = code_format(bits_a);
  // the auxiliary stream starts quantizing loop 0 while the caller's stream
  // expands the weights (separate workspace regions); the first GEMM waits
  // for both
  hipEvent_t start = p->events[T];
  if (hipEventRecord(start, s) != hipSuccess) return LOOPQ_ERR_HIP;
  if (hipStreamWaitEvent(p->aux, start, 0) != hipSuccess) return LOOPQ_ERR_HIP;
  if (prepare_weights(carve(ws, T, M, K, N, 0, 0), fmt, w_codes, K, N, s) != hipSuccess)
    return LOOPQ_ERR_HIP;
  for (int t = 0; t < T; ++t) {
    ClipTable one;
    memset(&one, 0, sizeof(one));
    one.c[0] = clips.c[t];
    ActBuffers b = carve(ws, T, M, K, N, t, 0);
    const void* xt = reinterpret_cast<const char*>(x) + (size_t)t * M * K * esz;
    QuantArgs a = internal_quant_args(xt, dtype, M, K, P1, n1, P2, n2, one, M, bits_a, b);
    if (xt_out) a.xt_out = xt_out + (size_t)t * M * K;
    hipError_t e;
    {
      TimingScope ts(P1 ? LOOPQ_KERNEL_QUANT_TRANSFORM : LOOPQ_KERNEL_QUANT_PLAIN, p->aux);
      e = launch_quant_act(a, p->aux);
    }
    if (e != hipSuccess) return LOOPQ_ERR_HIP;
    if (hipEventRecord(p->events[t], p->aux) != hipSuccess) return LOOPQ_ERR_HIP;
  }
  for (int t = 0; t < T; ++t) {
    if (hipStreamWaitEvent(s, p->events[t], 0) != hipSuccess) return LOOPQ_ERR_HIP;
    ActBuffers b = carve(ws, T, M, K, N, t, 0);
    hipError_t e;
    {
      TimingScope ts(LOOPQ_KERNEL_GEMM, s);
      e = run_gemm(b, fmt, M, K, N, w_codes, w_scales, gw, y + (size_t)t * M * N, nullptr, 0, s);
    }
    if (e != hipSuccess) return LOOPQ_ERR_HIP;
  }
  return LOOPQ_OK;
}

// Loop-dependent weight sets in one grouped GEMM (all loops at one bit width,
// M % 64 == 0): each maximal run of loops with one set is quantized with that
// set's transform into rows [t0 * M, t1 * M) of one activation buffer, every
// set in use has its W4A4 operands expanded once, and a single GEMM over all
// T * M rows takes loop t's weights for loop t's rows.  The workspace holds
// the activation buffers of T * M rows and one expansion region per set used.
hipError_t looped_grouped(const void* x, int dtype, int T, int M, int K, int N, const float* const* P1_sets,
                          int n1, const float* const* P2_sets, int n2, const void* const* w_codes_sets,
                          const void* const* w_scales_sets, int gw, const int32_t* sets, int bits_a,
                          const float* clips_host, float* y, void* ws, hipStream_t s) {
  const int fmt = code_format(bits_a);
  const int rows = T * M;
  const size_t esz = dtype == LOOPQ_F32 ? 4 : 2;
  ActBuffers b = carve(ws, T, M, K, N, 0, rows);
  const int64_t block_bytes = fmt == kCodesTiledF6 ? group_pairs(K) * kF6BlockBytes : (int64_t)(K / 32) * 1024;
  hipError_t e = hipSuccess;
  for (int t0 = 0; t0 < T;) {
    int t1 = t0 + 1;
    while (t1 < T && sets[t1] == sets[t0]) ++t1;
    const int set = sets[t0];
    ClipTable ct;
    memset(&ct, 0, sizeof(ct));
    for (int t = t0; t < t1; ++t) ct.c[t - t0] = clips_host[t];
    QuantArgs a = internal_quant_args(reinterpret_cast<const char*>(x) + (size_t)t0 * M * K * esz, dtype,
                                      (t1 - t0) * M, K, P1_sets ? P1_sets[set] : nullptr, n1,
                                      P2_sets ? P2_sets[set] : nullptr, n2, ct, M, bits_a, b);
    // rows t0 * M.. of the tiled codes (32-row blocks) and of the group-major steps
    a.codes = reinterpret_cast<int8_t*>(b.codes) + (int64_t)t0 * M / 32 * block_bytes;
    a.scales = b.scales + (int64_t)t0 * M;
    {
      TimingScope ts(a.P1 ? LOOPQ_KERNEL_QUANT_TRANSFORM : LOOPQ_KERNEL_QUANT_PLAIN, s);
      e = launch_quant_act(a, s);
    }
    if (e != hipSuccess) return e;
    t0 = t1;
  }
  GemmSets gs;
  gs.rows_per_set = M;
  gs.n = T;
  int slot_of[LOOPQ_MAX_LOOPS];
  int nslots = 0;
  for (int t = 0; t < T; ++t) {
    int slot = -1;
    for (int u = 0; u < t; ++u)
      if (sets[u] == sets[t]) slot = slot_of[u];
    if (slot < 0) {  // first loop of this set: expand its weights into a fresh region
      slot = nslots++;
      if (fmt == kCodesTiledF6) {
        ActBuffers bs = b;
        if (slot > 0)
          bs.wexp = reinterpret_cast<char*>(ws) + act_bytes(T, M, K, N, fmt) + (size_t)(slot - 1) * wexp_region(K, N, fmt);
        e = prepare_weights(bs, fmt, w_codes_sets[sets[t]], K, N, s);
        if (e != hipSuccess) return e;
      }
    }
    slot_of[t] = slot;
    gs.w[t] = fmt == kCodesTiledF6
                  ? (slot == 0 ? b.wexp
                               : reinterpret_cast<char*>(ws) + act_bytes(T, M, K, N, fmt) +
                                     (size_t)(slot - 1) * wexp_region(K, N, fmt))
                  : w_codes_sets[sets[t]];
    gs.sw[t] = reinterpret_cast<const __half*>(w_scales_sets[sets[t]]);
  }
  TimingScope ts(LOOPQ_KERNEL_GEMM, s);
  return run_gemm(b, fmt, rows, K, N, gs.w[0], gs.sw[0], gw, y, nullptr, 0, s, &gs);
}

// The per-token quantizer.  With a transform it runs inside the transform
// kernel, which holds whole x~ rows in LDS and takes each row's absmax there
// (one launch, no x~ round trip; x~ goes to a.xt_out only if the caller asked
// for it); without one, the row kernel quantizes x.  `a` carries the
// outputs; returns the first HIP error.
hipError_t per_token_quant(QuantArgs a, hipStream_t s) {
  if (a.P1 != nullptr) {
    a.per_token = 1;
    TimingScope ts(LOOPQ_KERNEL_QUANT_TRANSFORM, s);
    return launch_quant_act(a, s);
  }
  TimingScope ts(LOOPQ_KERNEL_QUANT_TOKEN, s);
  return launch_quant_token(a, s);
}

// ---------------------------------------------------------------------------
// Fixed scratch memory of loopq_w4a4_linear_noalloc, for callers that cannot
// allocate.  Every device the library runs on holds its own copy of the
// array until the process ends.  In host code the array's name is not a
// device address: the address is taken once per device with
// hipGetSymbolAddress (that device current) and only that address is used.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Host-side checks of loopq_looped_forward, before any HIP call.  Fills the
// clip table; *empty is set (with LOOPQ_OK) when there are no rows to run.
int32_t check_forward(const void* x, int dtype, int T, int M, int K, int N, const float* P1, int n1,
                      const float* P2, int n2, const float* clips_host, int bits_a, const void* w_codes,
                      const void* w_scales, int group_w, const float* y, int schedule, ClipTable* clips,
                      bool* empty) {
  *empty = false;
  if (T <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (T > LOOPQ_MAX_LOOPS) return LOOPQ_ERR_UNSUPPORTED;
  if ((int64_t)T * M > (int64_t)1 << 30) return LOOPQ_ERR_UNSUPPORTED;
  int32_t st = check_act(x, dtype, M, K, bits_a);
  if (st != LOOPQ_OK) return st;
  st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  st = check_gemm_extent((int64_t)T * padded_rows(M), K, N, group_w);
  if (st != LOOPQ_OK) return st;
  st = check_transform(K, P1, n1, P2, n2);
  if (st != LOOPQ_OK) return st;
  if (!clips_host) return LOOPQ_ERR_INVALID_ARG;
  memset(clips, 0, sizeof(*clips));
  for (int t = 0; t < T; ++t) {
    if (!clip_ok(clips_host[t])) return LOOPQ_ERR_INVALID_ARG;
    clips->c[t] = clips_host[t];
  }
  if (schedule < LOOPQ_SCHED_AUTO || schedule > LOOPQ_SCHED_WEIGHT_STATIONARY)
    return LOOPQ_ERR_INVALID_ARG;
  if (M == 0) {
    *empty = true;
    return LOOPQ_OK;
  }
  if (!w_codes || !w_scales || !y) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(w_codes, 16) || !aligned(w_scales, 16) || !aligned(y, 4)) return LOOPQ_ERR_ALIGNMENT;
  return LOOPQ_OK;
}

}  // namespace

extern "C" {

int32_t loopq_abi_version(void) { return LOOPQ_ABI_VERSION; }

const char* loopq_status_string(int32_t status) {
  switch (status) {
    case LOOPQ_OK: return "ok";
    case LOOPQ_ERR_INVALID_ARG: return "invalid argument";
    case LOOPQ_ERR_UNSUPPORTED: return "unsupported shape or option";
    case LOOPQ_ERR_ALIGNMENT: return "misaligned pointer";
    case LOOPQ_ERR_RANGE: return "weight step overflows fp16";
    case LOOPQ_ERR_HIP: return "HIP runtime error";
    case LOOPQ_ERR_WORKSPACE: return "workspace missing or too small";
    case LOOPQ_ERR_SINGULAR: return "singular transform factor";
    default: return "unknown status";
  }
}

int32_t loopq_packed_weight_bytes(int32_t K, int32_t N, int32_t group_w, size_t* codes_bytes,
                                  size_t* scales_bytes) {
  int32_t st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  if (!codes_bytes || !scales_bytes) return LOOPQ_ERR_INVALID_ARG;
  *codes_bytes = (size_t)padded_cols(N) * (size_t)K / 2;
  *scales_bytes = (size_t)padded_cols(N) * (size_t)weight_groups(K, group_w) * 2;
  return LOOPQ_OK;
}

int32_t loopq_workspace_bytes(int32_t op, int32_t T, int32_t M, int32_t K, int32_t N,
                              int32_t bits_a, size_t* bytes) {
  if (!bytes) return LOOPQ_ERR_INVALID_ARG;
  if ((op == LOOPQ_OP_LINEAR || op == LOOPQ_OP_LOOPED_FORWARD) && bits_a != 4 && bits_a != 8)
    return LOOPQ_ERR_UNSUPPORTED;
  switch (op) {
    case LOOPQ_OP_LINEAR:
      if (M < 0 || K <= 0 || K % 32) return M < 0 || K <= 0 ? LOOPQ_ERR_INVALID_ARG : LOOPQ_ERR_UNSUPPORTED;
      if (N <= 0) return LOOPQ_ERR_INVALID_ARG;
      *bytes = act_bytes(1, M, K, N, code_format(bits_a));
      return LOOPQ_OK;
    case LOOPQ_OP_LOOPED_FORWARD:
      if (T <= 0 || M < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (T > LOOPQ_MAX_LOOPS || K % 32) return LOOPQ_ERR_UNSUPPORTED;
      if (N <= 0) return LOOPQ_ERR_INVALID_ARG;
      *bytes = act_bytes(T, M, K, N, code_format(bits_a));
      return LOOPQ_OK;
    case LOOPQ_OP_LOOPED_FORWARD_EX: {
      if (T <= 0 || M < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (T > LOOPQ_MAX_LOOPS || K % 32) return LOOPQ_ERR_UNSUPPORTED;
      if (N <= 0) return LOOPQ_ERR_INVALID_ARG;
      // W4A4 with a weight set per loop: one fp6 expansion region per set
      const size_t a4 = act_bytes(T, M, K, N, code_format(4)) + (size_t)(T - 1) * wexp_region(K, N, code_format(4));
      const size_t a8 = act_bytes(T, M, K, N, code_format(8));
      *bytes = a4 > a8 ? a4 : a8;
      return LOOPQ_OK;
    }
    case LOOPQ_OP_QUANT_PER_TOKEN:  // the call needs no workspace
      if (M < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (K % 32) return LOOPQ_ERR_UNSUPPORTED;
      *bytes = 0;
      return LOOPQ_OK;
    case LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN: {
      if (bits_a != 4 && bits_a != 8) return LOOPQ_ERR_UNSUPPORTED;
      if (T <= 0 || M < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (T > LOOPQ_MAX_LOOPS || K % 32) return LOOPQ_ERR_UNSUPPORTED;
      if (N <= 0) return LOOPQ_ERR_INVALID_ARG;
      const int64_t rows = (int64_t)T * M;
      *bytes = act_bytes(1, rows, K, N, code_format(bits_a));
      return LOOPQ_OK;
    }
    case LOOPQ_OP_RECURRENT_ADAPTER:  // K = 2N is implied; the K argument is ignored
      if (bits_a != 4 && bits_a != 8) return LOOPQ_ERR_UNSUPPORTED;
      if (M < 0 || N <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (N % 16) return LOOPQ_ERR_UNSUPPORTED;
      *bytes = align256((size_t)M * 2 * N * 4) + act_bytes(1, M, 2 * (int64_t)N, N, code_format(bits_a));
      return LOOPQ_OK;
    case LOOPQ_OP_LOOPED_FORWARD_HESSIAN:  // the looped forward's region, x~ of all rows, the Hessian's
      if (T <= 0 || M < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (T > LOOPQ_MAX_LOOPS || K % 32 || K > kHessianMaxK || (int64_t)T * M > kHessianMaxRows)
        return LOOPQ_ERR_UNSUPPORTED;
      if (N <= 0) return LOOPQ_ERR_INVALID_ARG;
      *bytes = align256(act_bytes(T, M, K, N, code_format(bits_a))) + align256((size_t)T * M * K * 4) +
               align256(hessian_workspace_bytes(K));
      return LOOPQ_OK;
    case LOOPQ_OP_LOOPED_FORWARD_CTA:  // the looped forward's region, then the adapted loop inputs
      if (T <= 0 || M < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (T > LOOPQ_MAX_LOOPS || K % 32) return LOOPQ_ERR_UNSUPPORTED;
      if (N <= 0) return LOOPQ_ERR_INVALID_ARG;
      *bytes = align256(act_bytes(T, M, K, N, code_format(bits_a))) + align256((size_t)T * M * K * 4);
      return LOOPQ_OK;
    case LOOPQ_OP_HESSIAN:
      if (M < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (K % 32 || K > kHessianMaxK || M > kHessianMaxRows) return LOOPQ_ERR_UNSUPPORTED;
      *bytes = align256(hessian_workspace_bytes(K));
      return LOOPQ_OK;
    case LOOPQ_OP_FOLD:
      if (M <= 0 || N <= 0) return LOOPQ_ERR_INVALID_ARG;
      if (M > 128 || N > 128) return LOOPQ_ERR_UNSUPPORTED;
      *bytes = align256((size_t)(128 * 256 + M * M + N * N) * 8);
      return LOOPQ_OK;
    default:
      return LOOPQ_ERR_INVALID_ARG;
  }
}

int32_t loopq_fold_weights(const float* w, int32_t K, int32_t N, const float* P1, int32_t n1,
                           const float* P2, int32_t n2, float* w_folded, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!w || !w_folded || !P1 || !P2) return LOOPQ_ERR_INVALID_ARG;
  if (K <= 0 || N <= 0 || n1 <= 0 || n2 <= 0) return LOOPQ_ERR_INVALID_ARG;
  if ((int64_t)n1 * n2 != K || n1 > 128 || n2 > 128) return LOOPQ_ERR_UNSUPPORTED;
  if ((int64_t)K * 16 > 160 * 1024) return LOOPQ_ERR_UNSUPPORTED;  // fold kernel LDS
  if (!aligned(w, 4) || !aligned(w_folded, 4) || !aligned(P1, 4) || !aligned(P2, 4))
    return LOOPQ_ERR_ALIGNMENT;
  size_t need = 0;
  loopq_workspace_bytes(LOOPQ_OP_FOLD, 0, n1, K, n2, 0, &need);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  hipError_t e = reset_status(s);
  if (e == hipSuccess) e = launch_fold(w, K, N, P1, n1, P2, n2, w_folded, workspace, s);
  int flags = 0;
  if (e == hipSuccess) e = read_status(&flags, s);
  if (e != hipSuccess) return LOOPQ_ERR_HIP;
  return (flags & 2) ? LOOPQ_ERR_SINGULAR : LOOPQ_OK;
}

int32_t loopq_pack_weights(const float* w_folded, int32_t K, int32_t N, int32_t group_w,
                           void* w_codes, void* w_scales, void* stream) {
  int32_t st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  if (!w_folded || !w_codes || !w_scales) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(w_folded, 4) || !aligned(w_codes, 16) || !aligned(w_scales, 16))
    return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  hipError_t e = reset_status(s);
  if (e == hipSuccess)
    e = launch_pack_weights(w_folded, K, N, group_w, reinterpret_cast<uint8_t*>(w_codes),
                            reinterpret_cast<__half*>(w_scales), s);
  int flags = 0;
  if (e == hipSuccess) e = read_status(&flags, s);
  if (e != hipSuccess) return LOOPQ_ERR_HIP;
  return (flags & 1) ? LOOPQ_ERR_RANGE : LOOPQ_OK;
}

int32_t loopq_quant_act(const void* x, int32_t dtype, int32_t M, int32_t K, const float* P1,
                        int32_t n1, const float* P2, int32_t n2, float clip, int32_t bits_a,
                        int8_t* codes, float* scales, float* xt_out, void* stream) {
  int32_t st = check_act(x, dtype, M, K, bits_a);
  if (st != LOOPQ_OK) return st;
  st = check_transform(K, P1, n1, P2, n2);
  if (st != LOOPQ_OK) return st;
  if (!clip_ok(clip)) return LOOPQ_ERR_INVALID_ARG;
  if (M == 0) return LOOPQ_OK;
  if (!codes || !scales) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(codes, 4) || !aligned(scales, 4) || !aligned(xt_out, 16)) return LOOPQ_ERR_ALIGNMENT;
  QuantArgs a = make_quant_args(x, dtype, M, K, P1, n1, P2, n2, bits_a);
  a.clips.c[0] = clip;
  a.codes = codes;
  a.scales = scales;
  a.xt_out = xt_out;
  return hip_status(launch_quant_act(a, as_stream(stream)));
}

int32_t loopq_looped_forward(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                             int32_t N, const float* P1, int32_t n1, const float* P2, int32_t n2,
                             const float* clips_host, int32_t bits_a, const void* w_codes,
                             const void* w_scales, int32_t group_w, float* y, int32_t schedule,
                             void* workspace, size_t workspace_bytes, void* stream) {
  ClipTable clips;
  bool empty = false;
  int32_t st = check_forward(x, dtype, T, M, K, N, P1, n1, P2, n2, clips_host, bits_a, w_codes, w_scales,
                             group_w, y, schedule, &clips, &empty);
  if (st != LOOPQ_OK || empty) return st;
  size_t need = 0;
  loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, bits_a, &need);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  if (schedule == LOOPQ_SCHED_LOOP_SEQUENTIAL && T > 1)
    return looped_pipelined(x, dtype, T, M, K, N, P1, n1, P2, n2, clips, bits_a, w_codes, w_scales,
                            group_w, y, workspace, s);
  return linear_core(x, dtype, T * M, K, N, P1, n1, P2, n2, clips, M, bits_a, w_codes, w_scales,
                     group_w, y, workspace, T, M, s);
}

int32_t loopq_looped_forward_ex(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                                int32_t N, int32_t nsets, const float* const* P1_sets, int32_t n1,
                                const float* const* P2_sets, int32_t n2, const void* const* w_codes_sets,
                                const void* const* w_scales_sets, int32_t group_w,
                                const int32_t* sets_host, const int32_t* bits_host,
                                const float* clips_host, float* y, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (T <= 0 || nsets <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (T > LOOPQ_MAX_LOOPS) return LOOPQ_ERR_UNSUPPORTED;
  if ((int64_t)T * M > (int64_t)1 << 30) return LOOPQ_ERR_UNSUPPORTED;
  int32_t st = check_act(x, dtype, M, K, 4);
  if (st != LOOPQ_OK) return st;
  st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  st = check_gemm_extent((int64_t)T * padded_rows(M), K, N, group_w);
  if (st != LOOPQ_OK) return st;
  if (!sets_host || !bits_host || !clips_host || !w_codes_sets || !w_scales_sets) return LOOPQ_ERR_INVALID_ARG;
  if ((P1_sets == nullptr) != (P2_sets == nullptr)) return LOOPQ_ERR_INVALID_ARG;
  for (int s = 0; s < nsets; ++s) {
    const float* p1 = P1_sets ? P1_sets[s] : nullptr;
    const float* p2 = P2_sets ? P2_sets[s] : nullptr;
    if (P1_sets && (!p1 || !p2)) return LOOPQ_ERR_INVALID_ARG;
    st = check_transform(K, p1, n1, p2, n2);
    if (st != LOOPQ_OK) return st;
    if (!w_codes_sets[s] || !w_scales_sets[s]) return LOOPQ_ERR_INVALID_ARG;
    if (!aligned(w_codes_sets[s], 16) || !aligned(w_scales_sets[s], 16)) return LOOPQ_ERR_ALIGNMENT;
  }
  for (int t = 0; t < T; ++t) {
    if (sets_host[t] < 0 || sets_host[t] >= nsets) return LOOPQ_ERR_INVALID_ARG;
    if (bits_host[t] != 4 && bits_host[t] != 8) return LOOPQ_ERR_UNSUPPORTED;
    if (!clip_ok(clips_host[t])) return LOOPQ_ERR_INVALID_ARG;
  }
  if (M == 0) return LOOPQ_OK;
  if (!y) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(y, 4)) return LOOPQ_ERR_ALIGNMENT;
  size_t need = 0;
  loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD_EX, T, M, K, N, 0, &need);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  const size_t esz = dtype == LOOPQ_F32 ? 4 : 2;
  bool same_bits = true, one_run = true;
  for (int t = 1; t < T; ++t) {
    same_bits = same_bits && bits_host[t] == bits_host[0];
    one_run = one_run && sets_host[t] == sets_host[0] && bits_host[t] == bits_host[0];
  }
  if (!one_run && same_bits && M % 64 == 0 && (int64_t)T * M > kDecodeMaxRows)
    return hip_status(looped_grouped(x, dtype, T, M, K, N, P1_sets, n1, P2_sets, n2, w_codes_sets,
                                     w_scales_sets, group_w, sets_host, bits_host[0], clips_host, y,
                                     workspace, s));
  // maximal runs of consecutive loops with the same set and bit width, each
  // weight-stationary over its rows
  for (int t0 = 0; t0 < T;) {
    int t1 = t0 + 1;
    while (t1 < T && sets_host[t1] == sets_host[t0] && bits_host[t1] == bits_host[t0]) ++t1;
    const int set = sets_host[t0];
    ClipTable ct;
    memset(&ct, 0, sizeof(ct));
    for (int t = t0; t < t1; ++t) ct.c[t - t0] = clips_host[t];
    st = linear_core(reinterpret_cast<const char*>(x) + (size_t)t0 * M * K * esz, dtype, (t1 - t0) * M, K, N,
                     P1_sets ? P1_sets[set] : nullptr, n1, P2_sets ? P2_sets[set] : nullptr, n2, ct, M,
                     bits_host[t0], w_codes_sets[set], w_scales_sets[set], group_w, y + (size_t)t0 * M * N,
                     workspace, T, M, s);
    if (st != LOOPQ_OK) return st;
    t0 = t1;
  }
  return LOOPQ_OK;
}

int32_t loopq_w4a4_linear(const void* x, int32_t dtype, int32_t M, int32_t K, int32_t N,
                          const float* P1, int32_t n1, const float* P2, int32_t n2, float clip,
                          int32_t bits_a, const void* w_codes, const void* w_scales,
                          int32_t group_w, float* y, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return loopq_looped_forward(x, dtype, 1, M, K, N, P1, n1, P2, n2, &clip, bits_a, w_codes,
                              w_scales, group_w, y, LOOPQ_SCHED_WEIGHT_STATIONARY, workspace,
                              workspace_bytes, stream);
}

int32_t loopq_w4a4_linear_noalloc(const void* x, int32_t dtype, int32_t M, int32_t K, int32_t N,
                                  const float* P1, int32_t n1, const float* P2, int32_t n2, float clip,
                                  int32_t bits_a, const void* w_codes, const void* w_scales, int32_t group_w,
                                  float* y, void* stream) {
  ClipTable clips;
  bool empty = false;
  int32_t st = check_forward(x, dtype, 1, M, K, N, P1, n1, P2, n2, &clip, bits_a, w_codes, w_scales, group_w, y,
                             LOOPQ_SCHED_WEIGHT_STATIONARY, &clips, &empty);
  if (st != LOOPQ_OK || empty) return st;
  size_t need = 0;
  st = loopq_workspace_bytes(LOOPQ_OP_LINEAR, 1, M, K, N, bits_a, &need);
  if (st != LOOPQ_OK) return st;
  if (need > kScratchBytes) return LOOPQ_ERR_WORKSPACE;  // the call needs more than the fixed scratch
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return LOOPQ_ERR_HIP;
  t_no_alloc = true;
  // the kernels and workspace layout of loopq_w4a4_linear, on the scratch
  st = linear_core(x, dtype, M, K, N, P1, n1, P2, n2, clips, M, bits_a, w_codes, w_scales, group_w, y, ws, 1, M,
                   as_stream(stream));
  t_no_alloc = false;
  return st;
}

size_t loopq_noalloc_scratch_bytes(void) { return kScratchBytes; }

int32_t loopq_gemm_codes(const int8_t* a_codes, const float* a_scales, int32_t M, int32_t K,
                         int32_t N, const void* w_codes, const void* w_scales, int32_t group_w,
                         int32_t bits_a, float* y, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int32_t st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  if (bits_a != 4 && bits_a != 8) return LOOPQ_ERR_UNSUPPORTED;
  if (M < 0) return LOOPQ_ERR_INVALID_ARG;
  if (M == 0) return LOOPQ_OK;
  st = check_gemm_extent(padded_rows(M), K, N, group_w);
  if (st != LOOPQ_OK) return st;
  if (!a_codes || !a_scales || !w_codes || !w_scales || !y) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(a_codes, 4) || !aligned(a_scales, 4) || !aligned(w_codes, 16) ||
      !aligned(w_scales, 16) || !aligned(y, 4))
    return LOOPQ_ERR_ALIGNMENT;
  const int fmt = code_format(bits_a);
  const size_t need = act_bytes(1, M, K, N, fmt);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  ActBuffers b = carve(workspace, 1, M, K, N, 0, M);
  if (M <= kDecodeMaxRows) {  // decode: the fused kernel reads the canonical codes directly
    DecodeCall c;
    memset(&c, 0, sizeof(c));
    c.a_codes = a_codes;
    c.a_steps = a_scales;
    c.R = M;
    c.K = K;
    c.N = N;
    c.qmax = bits_a == 4 ? 7 : 127;
    c.w = reinterpret_cast<const uint8_t*>(w_codes);
    c.sw = reinterpret_cast<const __half*>(w_scales);
    c.gw = group_w;
    c.y = y;
    c.mode = 0;
    return hip_status(launch_decode(c, s));
  }
  hipError_t e = launch_tile_codes(a_codes, a_scales, M, K, b.codes, fmt, b.scales, b.ld, s);
  if (e == hipSuccess) e = prepare_weights(b, fmt, w_codes, K, N, s);
  if (e == hipSuccess) e = run_gemm(b, fmt, M, K, N, w_codes, w_scales, group_w, y, nullptr, 0, s);
  return hip_status(e);
}

int32_t loopq_export_weights(const void* w_codes, const void* w_scales, int32_t K, int32_t N,
                             int32_t group_w, int8_t* codes, uint16_t* scales, void* stream) {
  int32_t st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  if (!w_codes || !w_scales || !codes || !scales) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(w_codes, 16) || !aligned(w_scales, 16) || !aligned(scales, 2))
    return LOOPQ_ERR_ALIGNMENT;
  return hip_status(launch_export_weights(reinterpret_cast<const uint8_t*>(w_codes),
                                          reinterpret_cast<const __half*>(w_scales), K, N,
                                          group_w, codes, scales, as_stream(stream)));
}

int32_t loopq_group_dots(const int8_t* a_codes, int32_t M, int32_t K, int32_t N, int32_t bits_a,
                         const void* w_codes, int32_t* dots, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (M < 0 || K <= 0 || N <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (K % 32) return LOOPQ_ERR_UNSUPPORTED;
  if (bits_a != 4 && bits_a != 8) return LOOPQ_ERR_UNSUPPORTED;
  if (M == 0) return LOOPQ_OK;
  if (check_gemm_extent(padded_rows(M), K, N, 32) != LOOPQ_OK) return LOOPQ_ERR_UNSUPPORTED;
  if (!a_codes || !w_codes || !dots) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(a_codes, 4) || !aligned(w_codes, 16) || !aligned(dots, 4))
    return LOOPQ_ERR_ALIGNMENT;
  const int fmt = code_format(bits_a);
  const size_t need = act_bytes(1, M, K, N, fmt);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  ActBuffers b = carve(workspace, 1, M, K, N, 0, M);
  if (M <= kDecodeMaxRows) {  // the kernel the forward uses for this many rows
    DecodeCall c;
    memset(&c, 0, sizeof(c));
    c.a_codes = a_codes;
    c.R = M;
    c.K = K;
    c.N = N;
    c.qmax = bits_a == 4 ? 7 : 127;
    c.w = reinterpret_cast<const uint8_t*>(w_codes);
    c.gw = 32;
    c.dots = dots;
    c.mode = 1;
    return hip_status(launch_decode(c, s));
  }
  hipError_t e = launch_tile_codes(a_codes, nullptr, M, K, b.codes, fmt, nullptr, b.ld, s);
  if (e == hipSuccess) e = prepare_weights(b, fmt, w_codes, K, N, s);
  if (e == hipSuccess) e = run_gemm(b, fmt, M, K, N, w_codes, nullptr, 32, nullptr, dots, 1, s);
  return hip_status(e);
}

int32_t loopq_export_weight_codes(const void* w_codes, int32_t K, int32_t N, int32_t group_w, int8_t* codes,
                                  void* stream) {
  int32_t st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  if (!w_codes || !codes) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(w_codes, 16)) return LOOPQ_ERR_ALIGNMENT;
  return hip_status(launch_export_weights(reinterpret_cast<const uint8_t*>(w_codes), nullptr, K, N, group_w,
                                          codes, nullptr, as_stream(stream)));
}

int32_t loopq_export_act_codes(const void* workspace, size_t workspace_bytes, int32_t op, int32_t T, int32_t M,
                               int32_t K, int32_t N, int32_t bits_a, int32_t schedule, int8_t* codes,
                               float* scales, void* stream) {
  if (op == LOOPQ_OP_LINEAR) {
    if (T != 1) return LOOPQ_ERR_INVALID_ARG;
  } else if (op != LOOPQ_OP_LOOPED_FORWARD && op != LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN &&
             op != LOOPQ_OP_RECURRENT_ADAPTER) {
    return LOOPQ_ERR_INVALID_ARG;
  }
  if (op == LOOPQ_OP_RECURRENT_ADAPTER) {
    if (T != 1) return LOOPQ_ERR_INVALID_ARG;
    if (N <= 0 || N % 16) return N <= 0 ? LOOPQ_ERR_INVALID_ARG : LOOPQ_ERR_UNSUPPORTED;
    K = 2 * N;
  }
  if (T <= 0 || M < 0 || K <= 0 || N <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (T > LOOPQ_MAX_LOOPS || K % 32) return LOOPQ_ERR_UNSUPPORTED;
  if (bits_a != 4 && bits_a != 8) return LOOPQ_ERR_UNSUPPORTED;
  if (schedule < LOOPQ_SCHED_AUTO || schedule > LOOPQ_SCHED_WEIGHT_STATIONARY) return LOOPQ_ERR_INVALID_ARG;
  if ((int64_t)T * M > (int64_t)1 << 30) return LOOPQ_ERR_UNSUPPORTED;
  size_t need = 0;
  int32_t st = loopq_workspace_bytes(op, T, M, K, N, bits_a, &need);
  if (st != LOOPQ_OK) return st;
  if (M == 0) return LOOPQ_OK;
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  if (!codes || !scales) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(scales, 4)) return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  const int64_t rows = (int64_t)T * M;
  const int Ga = K / 32;
  void* wsp = const_cast<void*>(workspace);  // carve() only computes addresses; nothing is written
  // where each forward form leaves its codes (carve() as the call used it)
  auto one = [&](const ActBuffers& b, int64_t r, int64_t row0) -> hipError_t {
    const bool few = r <= kDecodeMaxRows;  // few-row path: canonical codes, row-major steps
    return launch_export_act(b.codes, b.scales, (int)r, K, few ? kCodesCanonical : code_format(bits_a), b.ld,
                             few ? 0 : 1, codes + row0 * K, scales + row0 * Ga, s);
  };
  if (op == LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN)
    return hip_status(one(carve(wsp, 1, rows, K, N, 0, rows), rows, 0));
  if (op == LOOPQ_OP_RECURRENT_ADAPTER) {
    void* ws = reinterpret_cast<char*>(wsp) + align256((size_t)M * K * 4);
    return hip_status(one(carve(ws, 1, M, K, N, 0, M), M, 0));
  }
  if (schedule == LOOPQ_SCHED_LOOP_SEQUENTIAL && T > 1) {
    for (int t = 0; t < T; ++t) {
      hipError_t e = one(carve(wsp, T, M, K, N, t, 0), M, (int64_t)t * M);
      if (e != hipSuccess) return LOOPQ_ERR_HIP;
    }
    return LOOPQ_OK;
  }
  return hip_status(one(carve(wsp, T, M, K, N, 0, rows), rows, 0));
}

int32_t loopq_quant_act_per_token(const void* x, int32_t dtype, int32_t M, int32_t K, const float* P1,
                                  int32_t n1, const float* P2, int32_t n2, float clip, int32_t bits_a,
                                  int8_t* codes, float* scales, float* xt_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  int32_t st = check_act(x, dtype, M, K, bits_a);
  if (st != LOOPQ_OK) return st;
  if ((int64_t)M * K > ((int64_t)1 << 40)) return LOOPQ_ERR_UNSUPPORTED;
  st = check_transform(K, P1, n1, P2, n2);
  if (st != LOOPQ_OK) return st;
  if (!clip_ok(clip)) return LOOPQ_ERR_INVALID_ARG;
  if (M == 0) return LOOPQ_OK;
  if (!codes || !scales) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(codes, 4) || !aligned(scales, 4) || !aligned(xt_out, 16)) return LOOPQ_ERR_ALIGNMENT;
  (void)workspace;  // accepted for compatibility; this call needs none
  (void)workspace_bytes;
  QuantArgs a = make_quant_args(x, dtype, M, K, P1, n1, P2, n2, bits_a);
  a.clips.c[0] = clip;
  a.codes = codes;
  a.scales = scales;
  a.xt_out = xt_out;
  return hip_status(per_token_quant(a, as_stream(stream)));
}

int32_t loopq_looped_forward_per_token(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                                       int32_t N, const float* P1, int32_t n1, const float* P2, int32_t n2,
                                       const float* clips_host, int32_t bits_a, const void* w_codes,
                                       const void* w_scales, int32_t group_w, float* y, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (T <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (T > LOOPQ_MAX_LOOPS) return LOOPQ_ERR_UNSUPPORTED;
  if ((int64_t)T * M > (int64_t)1 << 30) return LOOPQ_ERR_UNSUPPORTED;
  int32_t st = check_act(x, dtype, M, K, bits_a);
  if (st != LOOPQ_OK) return st;
  st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  st = check_gemm_extent(padded_rows((int64_t)T * M), K, N, group_w);
  if (st != LOOPQ_OK) return st;
  st = check_transform(K, P1, n1, P2, n2);
  if (st != LOOPQ_OK) return st;
  if (!clips_host) return LOOPQ_ERR_INVALID_ARG;
  ClipTable clips;
  memset(&clips, 0, sizeof(clips));
  for (int t = 0; t < T; ++t) {
    if (!clip_ok(clips_host[t])) return LOOPQ_ERR_INVALID_ARG;
    clips.c[t] = clips_host[t];
  }
  if (M == 0) return LOOPQ_OK;
  if (!w_codes || !w_scales || !y) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(w_codes, 16) || !aligned(w_scales, 16) || !aligned(y, 4)) return LOOPQ_ERR_ALIGNMENT;
  size_t need = 0;
  loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, T, M, K, N, bits_a, &need);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  const int rows = T * M;
  hipStream_t s = as_stream(stream);
  const int fmt = code_format(bits_a);
  ActBuffers b = carve(workspace, 1, rows, K, N, 0, rows);
  QuantArgs a = internal_quant_args(x, dtype, rows, K, P1, n1, P2, n2, clips, M, bits_a, b);
  const bool few = rows <= kDecodeMaxRows;
  if (few) {  // canonical codes and row-major steps for the few-row kernel
    a.codes_fmt = kCodesCanonical;
    a.scales_gm = 0;
  }
  hipError_t e = per_token_quant(a, s);
  if (e != hipSuccess) return LOOPQ_ERR_HIP;
  if (few) {
    DecodeCall c;
    memset(&c, 0, sizeof(c));
    c.a_codes = reinterpret_cast<const int8_t*>(b.codes);
    c.a_steps = b.scales;
    c.R = rows;
    c.K = K;
    c.N = N;
    c.qmax = bits_a == 4 ? 7 : 127;
    c.w = reinterpret_cast<const uint8_t*>(w_codes);
    c.sw = reinterpret_cast<const __half*>(w_scales);
    c.gw = group_w;
    c.y = y;
    c.mode = 0;
    TimingScope ts(LOOPQ_KERNEL_DECODE, s);
    return hip_status(launch_decode(c, s));
  }
  e = prepare_weights(b, fmt, w_codes, K, N, s);
  if (e != hipSuccess) return LOOPQ_ERR_HIP;
  TimingScope ts(LOOPQ_KERNEL_GEMM, s);
  return hip_status(run_gemm(b, fmt, rows, K, N, w_codes, w_scales, group_w, y, nullptr, 0, s));
}

int32_t loopq_looped_forward_hessian(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                                     int32_t N, const float* P1, int32_t n1, const float* P2, int32_t n2,
                                     const float* clips_host, int32_t bits_a, const void* w_codes,
                                     const void* w_scales, int32_t group_w, float* y, int32_t schedule,
                                     float* H, void* workspace, size_t workspace_bytes, void* stream) {
  ClipTable clips;
  bool empty = false;
  int32_t st = check_forward(x, dtype, T, M, K, N, P1, n1, P2, n2, clips_host, bits_a, w_codes, w_scales,
                             group_w, y, schedule, &clips, &empty);
  if (st != LOOPQ_OK) return st;
  if (K > kHessianMaxK || (int64_t)T * M > kHessianMaxRows) return LOOPQ_ERR_UNSUPPORTED;
  if (empty) return LOOPQ_OK;
  if (!H) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(H, 4)) return LOOPQ_ERR_ALIGNMENT;
  size_t need = 0, base = 0;
  loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD_HESSIAN, T, M, K, N, bits_a, &need);
  loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, bits_a, &base);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  unsigned char* w8 = static_cast<unsigned char*>(workspace);
  float* xt = reinterpret_cast<float*>(w8 + align256(base));
  float* part = reinterpret_cast<float*>(w8 + align256(base) + align256((size_t)T * M * K * 4));
  hipStream_t s = as_stream(stream);
  if (schedule == LOOPQ_SCHED_LOOP_SEQUENTIAL && T > 1)
    st = looped_pipelined(x, dtype, T, M, K, N, P1, n1, P2, n2, clips, bits_a, w_codes, w_scales, group_w, y,
                          workspace, s, xt);
  else
    st = linear_core(x, dtype, T * M, K, N, P1, n1, P2, n2, clips, M, bits_a, w_codes, w_scales, group_w, y,
                     workspace, T, M, s, xt);
  if (st != LOOPQ_OK) return st;
  TimingScope ts(LOOPQ_KERNEL_HESSIAN, s);
  return hip_status(launch_hessian(xt, T * M, K, H, part, s));
}

int32_t loopq_cta_apply(const void* h, int32_t dtype, int32_t M, int32_t K, const float* U,
                        const float* V, int32_t rank, const float* a, const float* b, float eta,
                        void* out, void* stream) {
  if (dtype != LOOPQ_F32 && dtype != LOOPQ_BF16) return LOOPQ_ERR_INVALID_ARG;
  if (M < 0 || K <= 0 || rank <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (K % 32 || rank > cta_max_rank()) return LOOPQ_ERR_UNSUPPORTED;
  if (!isfinite(eta)) return LOOPQ_ERR_INVALID_ARG;
  if (M == 0) return LOOPQ_OK;
  if (!h || !out || !U || !V || !a || !b) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(h, 16) || !aligned(out, 16) || !aligned(U, 4) || !aligned(V, 4) || !aligned(a, 4) ||
      !aligned(b, 4))
    return LOOPQ_ERR_ALIGNMENT;
  const size_t bytes = (size_t)M * K * (dtype == LOOPQ_BF16 ? 2 : 4);
  const uintptr_t hi = reinterpret_cast<uintptr_t>(h), oi = reinterpret_cast<uintptr_t>(out);
  if (hi != oi && hi < oi + bytes && oi < hi + bytes) return LOOPQ_ERR_INVALID_ARG;  // partial overlap
  hipStream_t s = as_stream(stream);
  TimingScope ts(LOOPQ_KERNEL_CTA, s);
  return hip_status(launch_cta(h, dtype == LOOPQ_BF16, M, K, U, V, rank, a, b, &eta, 1, M, 0, out, s));
}

int32_t loopq_looped_forward_cta(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                                 int32_t N, const float* P1, int32_t n1, const float* P2, int32_t n2,
                                 const float* clips_host, int32_t bits_a, const void* w_codes,
                                 const void* w_scales, int32_t group_w, float* y, int32_t schedule,
                                 const float* U, const float* V, int32_t rank, const float* a_sets,
                                 const float* b_sets, const float* eta_host, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  ClipTable clips;
  bool empty = false;
  int32_t st = check_forward(x, dtype, T, M, K, N, P1, n1, P2, n2, clips_host, bits_a, w_codes, w_scales,
                             group_w, y, schedule, &clips, &empty);
  if (st != LOOPQ_OK) return st;
  if (T > 1) {
    if (rank <= 0) return LOOPQ_ERR_INVALID_ARG;
    if (rank > cta_max_rank()) return LOOPQ_ERR_UNSUPPORTED;
    if (!U || !V || !a_sets || !b_sets || !eta_host) return LOOPQ_ERR_INVALID_ARG;
    if (!aligned(U, 4) || !aligned(V, 4) || !aligned(a_sets, 4) || !aligned(b_sets, 4)) return LOOPQ_ERR_ALIGNMENT;
    for (int t = 0; t + 1 < T; ++t)
      if (!isfinite(eta_host[t])) return LOOPQ_ERR_INVALID_ARG;
  }
  if (empty) return LOOPQ_OK;
  size_t need = 0, base = 0;
  loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD_CTA, T, M, K, N, bits_a, &need);
  loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, bits_a, &base);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  if (T == 1)  // no transition
    return loopq_looped_forward(x, dtype, T, M, K, N, P1, n1, P2, n2, clips_host, bits_a, w_codes, w_scales,
                                group_w, y, schedule, workspace, base, stream);
  void* xa = static_cast<unsigned char*>(workspace) + align256(base);
  hipStream_t s = as_stream(stream);
  {
    TimingScope ts(LOOPQ_KERNEL_CTA, s);
    if (launch_cta(x, dtype == LOOPQ_BF16, (int64_t)T * M, K, U, V, rank, a_sets, b_sets, eta_host, T - 1, M, -1,
                   xa, s) != hipSuccess)
      return LOOPQ_ERR_HIP;
  }
  return loopq_looped_forward(xa, dtype, T, M, K, N, P1, n1, P2, n2, clips_host, bits_a, w_codes, w_scales,
                              group_w, y, schedule, workspace, base, stream);
}

int32_t loopq_recurrent_adapter(const float* s0, const float* e, int32_t T, int32_t M, int32_t N,
                                const float* P1, int32_t n1, const float* P2, int32_t n2,
                                const float* clips_host, int32_t bits_a, const void* w_codes,
                                const void* w_scales, int32_t group_w, float* y, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (T <= 0 || M < 0 || N <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (T > LOOPQ_MAX_LOOPS || N % 16 || M > (1 << 30) / 2) return LOOPQ_ERR_UNSUPPORTED;
  const int K = 2 * N;
  int32_t st = check_act(s0, LOOPQ_F32, M, K, bits_a);
  if (st != LOOPQ_OK) return st;
  st = check_weights(K, N, group_w);
  if (st != LOOPQ_OK) return st;
  st = check_gemm_extent(padded_rows(M), K, N, group_w);
  if (st != LOOPQ_OK) return st;
  st = check_transform(K, P1, n1, P2, n2);
  if (st != LOOPQ_OK) return st;
  if (!clips_host) return LOOPQ_ERR_INVALID_ARG;
  for (int t = 0; t < T; ++t)
    if (!clip_ok(clips_host[t])) return LOOPQ_ERR_INVALID_ARG;
  if (M == 0) return LOOPQ_OK;
  if (!e || !w_codes || !w_scales || !y) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(e, 16) || !aligned(y, 16) || !aligned(w_codes, 16) || !aligned(w_scales, 16))
    return LOOPQ_ERR_ALIGNMENT;
  size_t need = 0;
  loopq_workspace_bytes(LOOPQ_OP_RECURRENT_ADAPTER, T, M, K, N, bits_a, &need);
  if (!workspace || workspace_bytes < need) return LOOPQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  float* x = reinterpret_cast<float*>(workspace);
  void* ws = reinterpret_cast<char*>(workspace) + align256((size_t)M * K * 4);
  for (int t = 0; t < T; ++t) {
    const float* state = t == 0 ? s0 : y + (size_t)(t - 1) * M * N;
    if (launch_concat_state(state, e, x, M, N, s) != hipSuccess) return LOOPQ_ERR_HIP;
    ClipTable clips;
    memset(&clips, 0, sizeof(clips));
    clips.c[0] = clips_host[t];
    st = linear_core(x, LOOPQ_F32, M, K, N, P1, n1, P2, n2, clips, M, bits_a, w_codes, w_scales, group_w,
                     y + (size_t)t * M * N, ws, 1, M, s);
    if (st != LOOPQ_OK) return st;
  }
  return LOOPQ_OK;
}

int32_t loopq_hessian_accumulate(const float* xt, int32_t rows, int32_t K, float* H, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (rows < 0 || K <= 0) return LOOPQ_ERR_INVALID_ARG;
  if (K % 32 || K > kHessianMaxK || rows > kHessianMaxRows) return LOOPQ_ERR_UNSUPPORTED;
  if (rows == 0) return LOOPQ_OK;  // nothing to read or add
  if (!xt || !H) return LOOPQ_ERR_INVALID_ARG;
  if (!aligned(xt, 16) || !aligned(H, 4)) return LOOPQ_ERR_ALIGNMENT;
  const size_t need = hessian_workspace_bytes(K);
  if (need && (!workspace || workspace_bytes < need)) return LOOPQ_ERR_WORKSPACE;
  if (need && !aligned(workspace, 256)) return LOOPQ_ERR_ALIGNMENT;
  hipStream_t s = as_stream(stream);
  TimingScope ts(LOOPQ_KERNEL_HESSIAN, s);
  return hip_status(launch_hessian(xt, rows, K, H, reinterpret_cast<float*>(workspace), s));
}

int32_t loopq_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on = on != 0;
  return LOOPQ_OK;
}

int32_t loopq_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (auto& r : g_timing_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return LOOPQ_ERR_HIP;
  }
  recycle_locked();
  return LOOPQ_OK;
}

int32_t loopq_timing_read(int32_t n, double* ms_host, int64_t* launches_host) {
  if (n <= 0 || !ms_host || !launches_host) return LOOPQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (int k = 0; k < n; ++k) {
    ms_host[k] = 0.0;
    launches_host[k] = 0;
  }
  for (auto& r : g_timing_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return LOOPQ_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return LOOPQ_ERR_HIP;
    if (r.kid < n) {
      ms_host[r.kid] += ms;
      launches_host[r.kid] += 1;
    }
  }
  recycle_locked();
  return LOOPQ_OK;
}

}  // extern "C"

namespace loopq {

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(g_launch_mu);
  if (g_ncu[dev] <= 0) {
    int n = 0;
    g_ncu[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return g_ncu[dev];
}

hipError_t prepare_launch(const void* fn, int lds_bytes, int block, int* per_cu, int* ncu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_launch_mu);
  KernelState* st = nullptr;
  for (KernelState& k : g_kernels)
    if (k.dev == dev && k.fn == fn) st = &k;
  if (!st) {
    g_kernels.push_back(KernelState{dev, fn, 0, {}});
    st = &g_kernels.back();
  }
  if (lds_bytes > st->lds_set) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    st->lds_set = lds_bytes;
  }
  if (ncu) {
    if (g_ncu[dev] <= 0) {
      int n = 0;
      g_ncu[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
    }
    *ncu = g_ncu[dev];
  }
  if (per_cu) {
    int found = -1;
    for (size_t i = 0; i + 2 < st->occ.size(); i += 3)
      if (st->occ[i] == lds_bytes && st->occ[i + 1] == block) found = st->occ[i + 2];
    if (found < 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&found, fn, block, lds_bytes) != hipSuccess || found < 1)
        found = 1;
      st->occ.insert(st->occ.end(), {lds_bytes, block, found});
    }
    *per_cu = found;
  }
  return hipSuccess;
}

}  // namespace loopq
