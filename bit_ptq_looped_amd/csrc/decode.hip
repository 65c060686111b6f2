// Few-row (decode) form of the quantized linear (gfx950): for at most 16
// token rows, the Kronecker transform, the Eq.(4) group quantizer with the
// loop's LAS clip, and the integer product with per-group rescale
//
//   y[m][n] = sum_j s_a[m][j] * s_w[n][32j / group_w] * d[m][n][j],
//   d[m][n][j] = sum_{k in group j} q_a[m][k] * q_w[n][k]   (exact int32)
//
// in one launch.  Method: Eq.(4) ("paper_specification.yaml",
// lq1_quantization), LAS (loopq_components.las, lq2), the shared Kronecker
// transform (lq3); the product is the integer form of the reproduction's
// simulated quantize-dequantize linear (README of the LoopQ reproduction,
// "Protocol").
//
// With a handful of rows the call is bound by streaming the packed INT4
// weights once and by latency.  Each work-group owns one block of 32 output
// columns over all of K and needs no other work-group: it issues the loads of
// its first weight slice (64 groups) into registers, forms the rows' codes
// while they arrive, then dots, with the next slice's loads in flight.
//   * Transform instances compute x~ of every row themselves (the same
//     operands and MFMA order as the chunked transform kernel, so the same x~
//     bit for bit), quantize each row into LDS with the quantizer the other
//     kernels use, and keep all rows' codes in LDS.  Every work-group repeats
//     the transform; the host takes this form only while that costs about as
//     much as the weight fetch it overlaps.
//   * Other instances quantize x (no transform) or copy canonical codes for
//     all rows and all of K into LDS (one weight slice at a time if that does
//     not fit), with every thread's loads of the next round in flight while
//     it quantizes the current one.
// Group dots: thread (column c, lane group gq) takes groups gq, gq + 8, ...
// of each slice, unpacks the column's 32 nibbles and dots them with every
// row's codes on V_DOT4_I32_I8 (exact), folding with fl32(s_w * s_a); the
// eight partial sums of a column are added in a fixed order through LDS, so y
// is deterministic.
#include "loopq_internal.h"
#include "quant_core.h"

#include <cstring>
#include <type_traits>

namespace loopq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSlice = 64;        // groups per weight slice
constexpr int kPer = kSlice / 8;  // groups of a slice per thread
constexpr int kLdsBudget = 160 * 1024;

struct DecodeArgs {
  const void* x;          // [R][K] fp32 or bf16 (in_codes == 0)
  int bf16;
  const int8_t* a_codes;  // canonical codes [R][K] (in_codes == 1)
  const float* a_steps;   // row-major steps [R][K/32] (in_codes == 1, mode 0)
  int in_codes;
  const float* P1;        // factors (transform instances)
  const float* P2;
  int R, K, N;
  ClipTable clips;
  int rows_per_clip;
  int qmax;
  const uint8_t* w;       // packed nibbles
  const __half* sw;       // packed steps [Npad/32][Gw][32] (mode 0)
  int gshift;
  float* y;               // [R][N] (mode 0)
  int32_t* dots;          // [R][N][K/32] (mode 1)
  int whole;              // non-transform instances: all codes fit LDS at once
  int wide_codes;         // canonical codes 16-byte aligned (copied 16 at a time)
};

// 8 biased nibbles (q + 8) per dword -> 16 int8 codes, in K order
__device__ __forceinline__ v4i unpack16(uint2 p) {
  v4i r;
  r[0] = (int)(((p.x & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[1] = (int)((((p.x >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[2] = (int)(((p.y & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[3] = (int)((((p.y >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  return r;
}

// The weights of one slice held by one thread: groups sl * kSlice + gq + 8 i.
struct WSlice {
  uint2 lo[kPer], hi[kPer];
  float s[kPer];
};

// Load a thread's part of slice `sl`; groups past Ga re-read group Ga - 1
// and are not used.
template <int MODE>
__device__ __forceinline__ void load_slice(const DecodeArgs& g, int cb, int sl, int c, int gq,
                                           WSlice& ws) {
  const int Ga = g.K >> 5;
  const int Gw = (Ga + (1 << g.gshift) - 1) >> g.gshift;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = min(sl * kSlice + gq + 8 * i, Ga - 1);
    const uint8_t* blk = g.w + ((int64_t)cb * Ga + j) * kBlockBytes + c * 8;
    ws.lo[i] = *reinterpret_cast<const uint2*>(blk);        // K 32 j + 0..15
    ws.hi[i] = *reinterpret_cast<const uint2*>(blk + 256);  // K 32 j + 16..31
    ws.s[i] = MODE == 0 ? __half2float(g.sw[((int64_t)cb * Gw + (j >> g.gshift)) * 32 + step_slot(c)]) : 0.0f;
  }
}

// Dots of the thread's groups of slice `sl` that lie in [jlo, jhi) with every
// row's codes: codes of group j of row m at sA + m * a_ld + (j - a_j0) * 32
// (bytes), its step at sS[m * s_ld + j - a_j0].
template <int RM, int MODE>
__device__ __forceinline__ void dot_slice(const DecodeArgs& g, int cb, int sl, int c, int gq,
                                          const WSlice& ws, int jlo, int jhi, const int8_t* sA,
                                          int a_ld, int a_j0, const float* sS, int s_ld,
                                          float (&acc)[RM]) {
  const int Ga = g.K >> 5;
  const int n = cb * 32 + c;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = sl * kSlice + gq + 8 * i;
    if (j >= jlo && j < jhi && j < Ga) {
      const v4i w0 = unpack16(ws.lo[i]);
      const v4i w1 = unpack16(ws.hi[i]);
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        if (m < g.R) {
          const v4i* ap = reinterpret_cast<const v4i*>(sA + m * a_ld + (j - a_j0) * 32);
          const v4i a0 = ap[0], a1 = ap[1];
          int d = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) d = __builtin_amdgcn_sdot4(a0[e], w0[e], d, false);
#pragma unroll
          for (int e = 0; e < 4; ++e) d = __builtin_amdgcn_sdot4(a1[e], w1[e], d, false);
          if (MODE == 0) {
            const float coef = ws.s[i] * sS[m * s_ld + j - a_j0];  // fl32(s_w * s_a)
            acc[m] = __builtin_fmaf((float)d, coef, acc[m]);
          } else if (n < g.N) {
            g.dots[((int64_t)m * g.N + n) * Ga + j] = d;
          }
        }
      }
    }
  }
}

// ---- MFMA form of the dots (up to 16 rows): V_MFMA_I32_16X16X32_I8 takes
// 16 rows (activation codes, rows >= R zero) x one 32-element group x 16
// weight columns and returns the 256 exact int32 dots.  Operand lanes: A row
// l % 16 and B column l % 16 hold K 8 (l / 16) .. + 7 of the group as 8 bytes;
// result element e of lane l is row 4 (l / 16) + e, column l % 16.  A wave
// takes groups wave, wave + 4, ... of a slice and both 16-column halves of
// the block; its nibbles for one (half, group) are one dword of the packed
// layout (K-half (l / 16) / 2, run (l / 16) % 2).

// The weights of one slice held by one lane: groups sl * kSlice + wave + 4 i.
constexpr int kMPer = kSlice / 4;
struct MSlice {
  uint32_t w[kMPer][2];  // packed nibbles, [group][column half]
  float s[kMPer][2];     // fp16 steps of the lane's column
};

template <int MODE>
__device__ __forceinline__ void load_mslice(const DecodeArgs& g, int cb, int sl, MSlice& ms) {
  const int Ga = g.K >> 5;
  const int Gw = (Ga + (1 << g.gshift) - 1) >> g.gshift;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4;
#pragma unroll
  for (int i = 0; i < kMPer; ++i) {
    const int j = min(sl * kSlice + wave + 4 * i, Ga - 1);  // past Ga: re-read, unused
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int c = tt * 16 + (lane & 15);
      ms.w[i][tt] = *reinterpret_cast<const uint32_t*>(g.w + ((int64_t)cb * Ga + j) * kBlockBytes + (q >> 1) * 256 +
                                                        c * 8 + (q & 1) * 4);
      ms.s[i][tt] = MODE == 0 ? __half2float(g.sw[((int64_t)cb * Gw + (j >> g.gshift)) * 32 + step_slot(c)]) : 0.0f;
    }
  }
}

// 8 biased nibbles (q + 8) of one dword -> 8 int8 codes in K order (low
// nibbles first), as the 64-bit MFMA operand
__device__ __forceinline__ long unpack8(uint32_t p) {
  const uint32_t lo = ((p & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
  const uint32_t hi = (((p >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
  return (long)(((uint64_t)hi << 32) | lo);
}

// Dots of the wave's groups of slice `sl` lying in [jlo, jhi), codes and
// steps addressed as in dot_slice; acc[half][e] is row 4 (l / 16) + e of
// column half * 16 + l % 16.
template <int MODE>
__device__ __forceinline__ void mfma_slice(const DecodeArgs& g, int cb, int sl, const MSlice& ms, int jlo,
                                           int jhi, const int8_t* sA, int a_ld, int a_j0, const float* sS,
                                           int s_ld, float (&acc)[2][4]) {
  typedef int v4i_t __attribute__((ext_vector_type(4)));
  const int Ga = g.K >> 5;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int ra = lane & 15;           // A row of the lane
  const int rac = min(ra, g.R - 1);   // rows past R read row R - 1, then zeroed
#pragma unroll
  for (int i = 0; i < kMPer; ++i) {
    const int j = sl * kSlice + wave + 4 * i;
    if (j >= jlo && j < jhi && j < Ga) {  // wave-uniform
      long a = *reinterpret_cast<const long*>(sA + rac * a_ld + (j - a_j0) * 32 + q * 8);
      if (ra >= g.R) a = 0;
      float sa[4];
      if (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sa[e] = sS[min(4 * q + e, g.R - 1) * s_ld + j - a_j0];
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const v4i_t d = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, unpack8(ms.w[i][tt]), v4i_t{0, 0, 0, 0}, 0, 0, 0);
        if (MODE == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[tt][e] = __builtin_fmaf((float)d[e], ms.s[i][tt] * sa[e], acc[tt][e]);  // coef fl32(s_w * s_a)
        } else {
          const int n = cb * 32 + tt * 16 + (lane & 15);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 4 * q + e;
            if (m < g.R && n < g.N) g.dots[((int64_t)m * g.N + n) * Ga + j] = d[e];
          }
        }
      }
    }
  }
}

// Copy an NN x NN fp32 matrix into LDS rows of stride SP.  All of a
// thread's loads are issued before any store, so the copy costs one memory
// round trip rather than one per element.
template <int NN, int SP>
__device__ __forceinline__ void stage_matrix(const float* __restrict__ src, float* dst) {
  constexpr int T = (NN * NN + 255) / 256;
  float v[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const int idx = threadIdx.x + 256 * i;
    v[i] = idx < NN * NN ? src[idx] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const int idx = threadIdx.x + 256 * i;
    if (idx < NN * NN) dst[(idx / NN) * SP + idx % NN] = v[i];
  }
}

// Row r of x (K elements, bf16 or fp32) into LDS as the n1 x n2 grid with
// row stride SX, loads first as above.
template <int K, int N2, int SX>
__device__ __forceinline__ void stage_x_row(const DecodeArgs& g, int r, float* sX) {
  constexpr int T = (K / 4 + 255) / 256;
  auto put = [&](int q, const float4& v) {
    const int k = q * 4;
    float* dst = sX + (k / N2) * SX + k % N2;
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  };
  if (g.bf16) {
    const uint2* src = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.x) + (int64_t)r * K);
    uint2 u[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int q = threadIdx.x + 256 * i;
      u[i] = q < K / 4 ? src[q] : uint2{0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int q = threadIdx.x + 256 * i;
      if (q < K / 4)
        put(q, float4{bf16_bits_to_float(u[i].x & 0xffffu), bf16_bits_to_float(u[i].x >> 16),
                      bf16_bits_to_float(u[i].y & 0xffffu), bf16_bits_to_float(u[i].y >> 16)});
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(g.x) + (int64_t)r * K);
    float4 v[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int q = threadIdx.x + 256 * i;
      v[i] = q < K / 4 ? src[q] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int q = threadIdx.x + 256 * i;
      if (q < K / 4) put(q, v[i]);
    }
  }
}

// LDS plan of the transform instances (bytes): P1 and P2 with bank-spread
// strides, the X row (later the x~ row), T = X * P2 for all column tiles,
// all rows' codes and steps, and the partial sums.
template <int N1, int N2>
struct XPlan {
  static constexpr int K = N1 * N2;
  static constexpr int sp1 = XStrides<N1, N2>::sp1, sp2 = XStrides<N1, N2>::sp2, sx = XStrides<N1, N2>::sx;
  static constexpr int njt = (N2 + 15) / 16;
  static constexpr int st = njt * 16;  // T row stride
  static constexpr int off_p2 = (N1 * sp1 * 4 + 15) / 16 * 16;
  static constexpr int off_x = off_p2 + (N2 * sp2 * 4 + 15) / 16 * 16;
  static constexpr int x_bytes = N1 * sx * 4 > K * 4 ? N1 * sx * 4 : K * 4;
  static constexpr int off_t = off_x + (x_bytes + 15) / 16 * 16;
  static constexpr int off_codes = off_t + N1 * st * 4;
  static constexpr int codes_bytes(int R) { return (R * K + 15) / 16 * 16; }
  static constexpr int lds(int R, int RM) { return off_codes + codes_bytes(R) + R * (K / 32) * 4 + 8 * RM * 32 * 4; }
};

// ---- transform work items (rows the one-launch form does not take): one
// work-group per (row r, 16-column tile jt of the n1 x n2 grid) writes that
// tile of x~ to xt[r][K] (fp32); the decode kernel then quantizes xt as
// plain input.  Wave w computes the stage-1 tile T[16 w ..][tile] with the
// full reduction over b, stores it in LDS, and after a barrier the stage-2
// tile x~[16 w ..][tile]; operands and MFMA order are those of the chunked
// kernel, so x~ is bitwise the same.
template <int N1, int N2>
struct ItemPlan {
  static constexpr int sp1 = XStrides<N1, N2>::sp1, sx = XStrides<N1, N2>::sx;
  static constexpr int off_p2 = (N1 * sp1 * 4 + 15) / 16 * 16;
  static constexpr int off_x = off_p2 + N2 * 16 * 4;
  static constexpr int off_t = (off_x + N1 * sx * 4 + 15) / 16 * 16;
  static constexpr int lds = off_t + N1 * 16 * 4;
};

template <int NRT, int N1, int N2>
__global__ __launch_bounds__(256) void xform_items_kernel(DecodeArgs g, float* __restrict__ xt) {
  extern __shared__ __align__(16) unsigned char lds[];
  using P = ItemPlan<N1, N2>;
  constexpr int n1 = N1, n2 = N2, K = N1 * N2;
  constexpr int njt = (N2 + 15) / 16;
  float* sP1 = reinterpret_cast<float*>(lds);
  float* sP2 = reinterpret_cast<float*>(lds + P::off_p2);
  float* sX = reinterpret_cast<float*>(lds + P::off_x);
  float* sT = reinterpret_cast<float*>(lds + P::off_t);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;
  const int lk = lane >> 4;
  const int r = blockIdx.x / njt;
  const int jt = blockIdx.x - r * njt;

  stage_matrix<N1, P::sp1>(g.P1, sP1);
  {  // the tile's P2 columns [n2][16] (zero past n2), loads first
    constexpr int T = (N2 * 16 + 255) / 256;
    float v[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int idx = tid + 256 * i;
      const int b = idx >> 4, j = jt * 16 + (idx & 15);
      v[i] = (idx < N2 * 16 && j < n2) ? g.P2[b * n2 + j] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int idx = tid + 256 * i;
      if (idx < N2 * 16) sP2[idx] = v[i];
    }
  }
  stage_x_row<K, N2, P::sx>(g, r, sX);
  __syncthreads();

  // stage 1: T[rt] = X_r * P2[:, tile], steps of b in order (as the chunked kernel)
  for (int rt = wave; rt < NRT; rt += 4) {
    v4f T = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* xa = sX + min(rt * 16 + li, n1 - 1) * P::sx;
    const uint32_t mrow = (rt * 16 + li < n1) ? 0xffffffffu : 0u;
#pragma unroll
    for (int st = 0; st < N2 / 4; ++st) {
      const int b = 4 * st + lk;
      T = __builtin_amdgcn_mfma_f32_16x16x4f32(masked(xa[b], mrow), sP2[b * 16 + li], T, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // element e of lane l: row 16 rt + 4 (l / 16) + e
      const int row = rt * 16 + 4 * lk + e;
      if (row < n1) sT[row * 16 + li] = T[e];
    }
  }
  __syncthreads();

  // stage 2: x~[it][tile] = sum_a P1[a][it] T[a][tile], a in the chunked kernel's order
  for (int it = wave; it < NRT; it += 4) {
    v4f o = {0.0f, 0.0f, 0.0f, 0.0f};
    const int i = it * 16 + li;
    const uint32_t mi = i < n1 ? 0xffffffffu : 0u;
#pragma unroll
    for (int st = 0; st < 4 * NRT; ++st) {
      const int ar = 16 * (st >> 2) + 4 * lk + (st & 3);
      const int ac = min(ar, n1 - 1);
      o = __builtin_amdgcn_mfma_f32_16x16x4f32(masked(sP1[ac * P::sp1 + min(i, n1 - 1)], ar < n1 ? mi : 0u),
                                               sT[ac * 16 + li], o, 0, 0, 0);
    }
    const int j = jt * 16 + li;
    if (j < n2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int io = it * 16 + 4 * lk + e;
        if (io < n1) xt[(int64_t)r * K + io * n2 + j] = o[e];
      }
    }
  }
}

// x~ of row r (bitwise the chunked kernel's) into the X region, then its codes
// and steps into sC / sS.  Ends with a barrier.
template <int NRT, int N1, int N2>
__device__ __forceinline__ void transform_row(const DecodeArgs& g, int r, unsigned char* lds,
                                              int8_t* sC, float* sS) {
  using P = XPlan<N1, N2>;
  constexpr int n1 = N1, n2 = N2, K = P::K, Ga = K / 32;
  const float* sP1 = reinterpret_cast<const float*>(lds);
  const float* sP2 = reinterpret_cast<const float*>(lds + P::off_p2);
  float* sX = reinterpret_cast<float*>(lds + P::off_x);
  float* sT = reinterpret_cast<float*>(lds + P::off_t);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;
  const int lk = lane >> 4;

  stage_x_row<K, N2, P::sx>(g, r, sX);
  __syncthreads();

  // stage 1: tile (rt, jt) of T = X[16 rt .., :] * P2[:, 16 jt ..], steps of b
  // in order.  Wave w takes tiles w, w + 4, ... (task t: rt = t % NRT, jt =
  // t / NRT), all at once as independent accumulators; the operands of step
  // s + 1 are read before step s multiplies.
  constexpr int ntask = NRT * P::njt;
  constexpr int NT = (ntask + 3) / 4;  // tiles per wave
  int rt[NT], jc[NT];
  bool has[NT];
  uint32_t mrow[NT], mj[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int t0 = wave + 4 * u;
    has[u] = t0 < ntask;
    const int t = min(t0, ntask - 1);
    rt[u] = t % NRT;
    jc[u] = (t / NRT) * 16 + li;
    mrow[u] = rt[u] * 16 + li < n1 ? 0xffffffffu : 0u;
    mj[u] = jc[u] < n2 ? 0xffffffffu : 0u;
  }
  {
    v4f acc[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float av[2][NT], bv[2][NT];
    auto fetch1 = [&](int s, float (&a)[NT], float (&bb)[NT]) {
      const int b = 4 * s + lk;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        a[u] = masked(sX[min(rt[u] * 16 + li, n1 - 1) * P::sx + b], mrow[u]);
        bb[u] = masked(sP2[b * P::sp2 + min(jc[u], n2 - 1)], mj[u]);
      }
    };
    fetch1(0, av[0], bv[0]);
#pragma unroll
    for (int s = 0; s < N2 / 4; ++s) {
      if (s + 1 < N2 / 4) fetch1(s + 1, av[(s + 1) & 1], bv[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NT; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s & 1][u], bv[s & 1][u], acc[u], 0, 0, 0);
    }
    // element e of lane l: row 16 rt + 4 (l / 16) + e, column jc
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (has[u]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rt[u] * 16 + 4 * lk + e;
          if (row < n1) sT[row * P::st + jc[u]] = acc[u][e];
        }
      }
    }
  }
  __syncthreads();

  // stage 2: tile (it, jt) of x~ = sum_a P1[a][i] T[a][j], the same tiles per
  // wave (it = t % NRT), over a in the chunked kernel's order (a = 16 (s / 4)
  // + 4 (l / 16) + s % 4, rows >= n1 masked), into the flat x~ row in the X
  // region (no longer read)
  float* sXt = sX;
  {
    v4f acc[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float av[2][NT], bv[2][NT];
    auto fetch2 = [&](int s, float (&a)[NT], float (&bb)[NT]) {
      const int ar = 16 * (s >> 2) + 4 * lk + (s & 3);
      const int ac = min(ar, n1 - 1);
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int i = rt[u] * 16 + li;
        a[u] = masked(sP1[ac * P::sp1 + min(i, n1 - 1)], (ar < n1 && i < n1) ? 0xffffffffu : 0u);
        bb[u] = sT[ac * P::st + jc[u]];
      }
    };
    fetch2(0, av[0], bv[0]);
#pragma unroll
    for (int s = 0; s < 4 * NRT; ++s) {
      if (s + 1 < 4 * NRT) fetch2(s + 1, av[(s + 1) & 1], bv[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NT; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s & 1][u], bv[s & 1][u], acc[u], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (has[u] && jc[u] < n2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int io = rt[u] * 16 + 4 * lk + e;
          if (io < n1) sXt[io * n2 + jc[u]] = acc[u][e];
        }
      }
    }
  }
  __syncthreads();

  // quantize row r: 8 lanes per group
  const float qmaxf = (float)g.qmax;
  const float rq = 1.0f / qmaxf;
  const float clip = g.clips.c[r / g.rows_per_clip];
  for (int base = 0; base < Ga * 8; base += 256) {
    const int q = base + tid;
    const bool valid = q < Ga * 8;
    const int qc = valid ? q : base;  // keep the group's shuffle partners active
    const int j = qc >> 3, l8 = qc & 7;
    const float4 v = *reinterpret_cast<const float4*>(sXt + j * 32 + l8 * 4);
    float s;
    const uint32_t packed = quantize4(v, clip, qmaxf, rq, &s);
    if (valid) {
      *reinterpret_cast<uint32_t*>(sC + r * K + j * 32 + l8 * 4) = packed;
      if (l8 == 0) sS[r * Ga + j] = s;
    }
  }
  __syncthreads();
}

// Canonical codes (16-byte aligned rows) and steps of every row for groups
// [j0, j0 + G) into LDS as make_codes lays them out, 16 codes per load, all
// of a round's loads (8 per thread) issued before its stores.
template <int MODE>
__device__ __forceinline__ void copy_codes(const DecodeArgs& g, int j0, int G, int8_t* sA, int a_ld,
                                           float* sS, int s_ld) {
  const int K = g.K, Ga = K >> 5;
  const int nch = g.R * G * 2;  // 16-code chunks
  for (int base = 0; base < nch; base += 256 * 8) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = base + (int)threadIdx.x + 256 * i;
      if (t < nch) {
        const int m = t / (2 * G), rem = t - m * 2 * G;
        v[i] = *reinterpret_cast<const uint4*>(g.a_codes + (int64_t)m * K + (j0 + (rem >> 1)) * 32 + (rem & 1) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = base + (int)threadIdx.x + 256 * i;
      if (t < nch) {
        const int m = t / (2 * G), rem = t - m * 2 * G;
        *reinterpret_cast<uint4*>(sA + m * a_ld + (rem >> 1) * 32 + (rem & 1) * 16) = v[i];
      }
    }
  }
  if (MODE == 0) {
    const int ns = g.R * G;
    for (int base = 0; base < ns; base += 256 * 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = base + (int)threadIdx.x + 256 * i;
        if (t < ns) {
          const int m = t / G;
          v[i] = g.a_steps[(int64_t)m * Ga + j0 + (t - m * G)];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = base + (int)threadIdx.x + 256 * i;
        if (t < ns) {
          const int m = t / G;
          sS[m * s_ld + t - m * G] = v[i];
        }
      }
    }
  }
}

// Codes and steps of every row for groups [j0, j0 + G) into LDS: codes of
// group j0 + gi of row m at sA + m * a_ld + gi * 32, its step at
// sS[m * s_ld + gi].  Task t = 8 (m G + gi) + l8 covers 4 elements; thread
// tid takes tasks tid + 256 i, kU per round, and the loads of round q + 1
// are issued before round q is quantized.  A group's 8 lanes are consecutive
// and aligned, and R G 8 is a multiple of 8, so a group is wholly valid or
// wholly past the end (then it quantizes a copy of the round's first task
// and stores nothing).
constexpr int kU = 4;
struct CodeRaw {
  uint4 v[kU];  // fp32: 4 elements; bf16: 4 elements in .x .y; codes: .x codes, .y step bits
};
template <int MODE>
__device__ __forceinline__ void make_codes(const DecodeArgs& g, int j0, int G, int8_t* sA, int a_ld,
                                           float* sS, int s_ld) {
  const int K = g.K, Ga = K >> 5;
  const int ntask = g.R * G * 8;
  const int per_round = 256 * kU;
  const int nround = (ntask + per_round - 1) / per_round;
  const float qmaxf = (float)g.qmax;
  const float rq = 1.0f / qmaxf;
  auto task_of = [&](int q, int i, int* m, int* gi, int* l8) {
    const int base = q * per_round + 256 * i;
    const int t = base + (int)threadIdx.x < ntask ? base + (int)threadIdx.x : base;
    const int grp = t >> 3;
    *l8 = t & 7;
    *m = grp / G;
    *gi = grp - *m * G;
  };
  auto issue = [&](int q, CodeRaw& raw) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      int m, gi, l8;
      task_of(q, i, &m, &gi, &l8);
      const int64_t e = (int64_t)m * K + (j0 + gi) * 32 + l8 * 4;
      if (q * per_round + 256 * i >= ntask) {  // uniform: nothing of this pass exists
        raw.v[i] = uint4{0u, 0u, 0u, 0u};
      } else if (g.in_codes) {
        raw.v[i].x = *reinterpret_cast<const uint32_t*>(g.a_codes + e);
        raw.v[i].y = MODE == 0 ? __float_as_uint(g.a_steps[(int64_t)m * Ga + j0 + gi]) : 0u;
      } else if (g.bf16) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.x) + e);
        raw.v[i].x = u.x;
        raw.v[i].y = u.y;
      } else {
        raw.v[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(g.x) + e);
      }
    }
  };
  auto process = [&](int q, const CodeRaw& raw) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int base = q * per_round + 256 * i;
      if (base >= ntask) continue;  // uniform
      int m, gi, l8;
      task_of(q, i, &m, &gi, &l8);
      uint32_t packed;
      float st;
      if (g.in_codes) {
        packed = raw.v[i].x;
        st = __uint_as_float(raw.v[i].y);
      } else {
        float4 v;
        if (g.bf16)
          v = float4{bf16_bits_to_float(raw.v[i].x & 0xffffu), bf16_bits_to_float(raw.v[i].x >> 16),
                     bf16_bits_to_float(raw.v[i].y & 0xffffu), bf16_bits_to_float(raw.v[i].y >> 16)};
        else
          v = float4{__uint_as_float(raw.v[i].x), __uint_as_float(raw.v[i].y),
                     __uint_as_float(raw.v[i].z), __uint_as_float(raw.v[i].w)};
        packed = quantize4(v, g.clips.c[m / g.rows_per_clip], qmaxf, rq, &st);
      }
      if (base + (int)threadIdx.x < ntask) {
        *reinterpret_cast<uint32_t*>(sA + m * a_ld + gi * 32 + l8 * 4) = packed;
        if (l8 == 0) sS[m * s_ld + gi] = st;
      }
    }
  };
  CodeRaw ra, rb;
  issue(0, ra);
  for (int q = 0; q < nround; q += 2) {  // two register buffers, unrolled by two
    if (q + 1 < nround) issue(q + 1, rb);
    process(q, ra);
    if (q + 1 < nround) {
      if (q + 2 < nround) issue(q + 2, ra);
      process(q + 1, rb);
    }
  }
}

// N1 = N2 = 0: no transform (x quantized as it is, or codes given).
// RM: rows bound (4 or 16).  MODE 0: y; MODE 1: int32 group dots.
template <int NRT, int N1, int N2, int RM, int MODE>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs g) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x;
  const int cb = blockIdx.x;  // column block
  const int c = tid & 31;     // column of the block
  const int gq = tid >> 5;    // lane group: groups gq + 8 i of each slice
  const int K = g.K;
  const int Ga = K >> 5;
  const int R = g.R;
  const int nsl = (Ga + kSlice - 1) / kSlice;

  // the first weight slice is in flight while the codes are formed (the
  // second follows once they are: both would crowd the transform's registers)
  constexpr bool kMfma = RM > 4;  // up to 16 rows: MFMA dots; up to 4: VALU dots
  typedef typename std::conditional<kMfma, MSlice, WSlice>::type Slice;
  Slice wa, wb;
  auto load = [&](int sl, Slice& buf) {
    if constexpr (kMfma) load_mslice<MODE>(g, cb, sl, buf);
    else load_slice<MODE>(g, cb, sl, c, gq, buf);
  };
  float acc[RM];
  float accm[2][4];
#pragma unroll
  for (int m = 0; m < RM; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int e = 0; e < 4; ++e) accm[tt][e] = 0.0f;
  auto dots = [&](int sl, const Slice& buf, int jlo, int jhi, const int8_t* sA, int a_ld, int a_j0,
                  const float* sS, int s_ld) {
    if constexpr (kMfma) mfma_slice<MODE>(g, cb, sl, buf, jlo, jhi, sA, a_ld, a_j0, sS, s_ld, accm);
    else dot_slice<RM, MODE>(g, cb, sl, c, gq, buf, jlo, jhi, sA, a_ld, a_j0, sS, s_ld, acc);
  };
  // slices alternate between the two register buffers (unrolled by two so
  // each buffer stays in registers); `body(sl, buf)` consumes slice sl
  auto sweep = [&](auto body) {
    for (int sl = 0; sl < nsl; sl += 2) {
      body(sl, wa);
      if (sl + 2 < nsl) load(sl + 2, wa);
      if (sl + 1 < nsl) {
        body(sl + 1, wb);
        if (sl + 3 < nsl) load(sl + 3, wb);
      }
    }
  };
  load(0, wa);
  float* red;

  if constexpr (N1 > 0) {
    using P = XPlan<N1, N2>;
    float* sP1 = reinterpret_cast<float*>(lds);
    float* sP2 = reinterpret_cast<float*>(lds + P::off_p2);
    int8_t* sC = reinterpret_cast<int8_t*>(lds + P::off_codes);
    float* sS = reinterpret_cast<float*>(lds + P::off_codes + P::codes_bytes(R));
    red = sS + R * (P::K / 32);
    stage_matrix<N1, P::sp1>(g.P1, sP1);
    stage_matrix<N2, P::sp2>(g.P2, sP2);
    // (transform_row's barrier after the X staging orders these stores too)
    for (int r = 0; r < R; ++r) transform_row<NRT, N1, N2>(g, r, lds, sC, sS);
    if (nsl > 1) load(1, wb);
    sweep([&](int sl, const Slice& buf) { dots(sl, buf, 0, Ga, sC, K, 0, sS, Ga); });
  } else if (g.whole) {
    // every row's codes for all of K in LDS, then the dots of every slice
    int8_t* sA = reinterpret_cast<int8_t*>(lds);                                    // [R][K]
    float* sSt = reinterpret_cast<float*>(lds + ((R * K + 15) & ~15));            // [R][Ga]
    red = sSt + R * Ga;
    if (nsl > 1) load(1, wb);
    if (g.in_codes && g.wide_codes)
      copy_codes<MODE>(g, 0, Ga, sA, K, sSt, Ga);
    else
      make_codes<MODE>(g, 0, Ga, sA, K, sSt, Ga);
    __syncthreads();
    sweep([&](int sl, const Slice& buf) { dots(sl, buf, 0, Ga, sA, K, 0, sSt, Ga); });
  } else {
    // too many codes for LDS: one weight slice of codes at a time
    int8_t* sA = reinterpret_cast<int8_t*>(lds);                          // [RM][kSlice * 32]
    float* sSt = reinterpret_cast<float*>(lds + RM * kSlice * 32);       // [RM][kSlice]
    red = sSt + RM * kSlice;
    if (nsl > 1) load(1, wb);
    sweep([&](int sl, const Slice& buf) {
      const int j0 = sl * kSlice;
      const int GS = min(kSlice, Ga - j0);
      __syncthreads();  // the previous slice's codes are no longer read
      if (g.in_codes && g.wide_codes)
        copy_codes<MODE>(g, j0, GS, sA, kSlice * 32, sSt, kSlice);
      else
        make_codes<MODE>(g, j0, GS, sA, kSlice * 32, sSt, kSlice);
      __syncthreads();
      dots(sl, buf, j0, j0 + GS, sA, kSlice * 32, j0, sSt, kSlice);
    });
  }
  if (MODE != 0) return;

  // partial sums of each (row, column) added in a fixed order through LDS
  if constexpr (kMfma) {
    // the four waves' sums: red[((wave * 2 + half) * 4 + e) * 64 + lane]
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave * 2 + tt) * 4 + e) * 64 + lane] = accm[tt][e];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = tid + 256 * i;  // row o / 32, column o % 32
      const int m = o >> 5, col = o & 31;
      const int n = cb * 32 + col;
      if (m < R && n < g.N) {
        const int ln = (m >> 2) * 16 + (col & 15);
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) tot += red[((w * 2 + (col >> 4)) * 4 + (m & 3)) * 64 + ln];
        g.y[(int64_t)m * g.N + n] = tot;
      }
    }
  } else {
    // the eight lane groups' sums
#pragma unroll
    for (int m = 0; m < RM; ++m) red[(gq * RM + m) * 32 + c] = acc[m];
    __syncthreads();
    const int n = cb * 32 + c;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = tid + 256 * i;  // row o / 32, column c
      if (o < R * 32 && n < g.N) {
        float tot = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) tot += red[(q * RM + (o >> 5)) * 32 + c];
        g.y[(int64_t)(o >> 5) * g.N + n] = tot;
      }
    }
  }
}

template <int RM, int MODE>
const void* plain_kernel() {
  return reinterpret_cast<const void*>(decode_kernel<1, 0, 0, RM, MODE>);
}

// LDS of the non-transform instances: all rows' codes and steps, or one
// weight slice of them; then the partial sums
int whole_lds(int R, int K, int RM) { return ((R * K + 15) & ~15) + R * (K / 32) * 4 + 8 * RM * 32 * 4; }
int slice_lds(int RM) { return RM * kSlice * 32 + RM * kSlice * 4 + 8 * RM * 32 * 4; }

}  // namespace

bool decode_transform_fused(int R, int n1, int n2) {
  // every work-group repeats the transform of all rows; keep that near the
  // time of the weight fetch it overlaps: at most 1.25M multiply-adds
  if (R <= 0 || R > kDecodeMaxRows) return false;
  if ((int64_t)R * n1 * n2 * (n1 + n2) > 1250000) return false;
  const int RM = R <= 4 ? 4 : kDecodeMaxRows;
#define LOOPQ_DECODE_FITS(n1_, n2_, rs_, nim_) \
  if (n1 == n1_ && n2 == n2_) return XPlan<n1_, n2_>::lds(R, RM) <= kLdsBudget;
  LOOPQ_SHAPES(LOOPQ_DECODE_FITS)
#undef LOOPQ_DECODE_FITS
  return false;
}

bool decode_transform_items(int n1, int n2) {
#define LOOPQ_ITEM_SHAPE(n1_, n2_, rs_, nim_) \
  if (n1 == n1_ && n2 == n2_) return true;
  LOOPQ_SHAPES(LOOPQ_ITEM_SHAPE)
#undef LOOPQ_ITEM_SHAPE
  return false;
}

hipError_t launch_decode(const DecodeCall& c, hipStream_t s) {
  if (c.R <= 0) return hipSuccess;
  if (c.R > kDecodeMaxRows || c.K % 32 != 0) return hipErrorInvalidValue;
  const bool xform = c.P1 != nullptr;
  if (xform && (c.a_codes != nullptr || c.mode != 0)) return hipErrorInvalidValue;
  if (xform && !decode_transform_fused(c.R, c.n1, c.n2)) return hipErrorInvalidValue;
  DecodeArgs g;
  memset(&g, 0, sizeof(g));
  g.x = c.x;
  g.bf16 = c.bf16;
  g.a_codes = c.a_codes;
  g.a_steps = c.a_steps;
  g.in_codes = c.a_codes != nullptr;
  g.P1 = c.P1;
  g.P2 = c.P2;
  g.R = c.R;
  g.K = c.K;
  g.N = c.N;
  g.clips = c.clips;
  g.rows_per_clip = c.rows_per_clip > 0 ? c.rows_per_clip : 1;
  g.qmax = c.qmax;
  g.w = c.w;
  g.sw = c.sw;
  g.gshift = c.gw == 128 ? 2 : 0;
  g.y = c.y;
  g.dots = c.dots;
  g.wide_codes = c.a_codes != nullptr && (reinterpret_cast<uintptr_t>(c.a_codes) & 15) == 0 && (c.K & 15) == 0;
  const void* fn = nullptr;
  int lds = 0;
  const bool small = c.R <= 4;
  const int RM = small ? 4 : kDecodeMaxRows;
  if (xform) {
#define LOOPQ_DECODE_KERNEL(n1_, n2_, rs_, nim_)                                                   \
    if (c.n1 == n1_ && c.n2 == n2_) {                                                              \
      constexpr int nrt = (n1_ + 15) / 16;                                                         \
      fn = small ? reinterpret_cast<const void*>(decode_kernel<nrt, n1_, n2_, 4, 0>)               \
                 : reinterpret_cast<const void*>(decode_kernel<nrt, n1_, n2_, kDecodeMaxRows, 0>); \
      lds = XPlan<n1_, n2_>::lds(c.R, RM);                                                         \
    }
    LOOPQ_SHAPES(LOOPQ_DECODE_KERNEL)
#undef LOOPQ_DECODE_KERNEL
  } else {
    fn = small ? (c.mode == 0 ? plain_kernel<4, 0>() : plain_kernel<4, 1>())
               : (c.mode == 0 ? plain_kernel<kDecodeMaxRows, 0>() : plain_kernel<kDecodeMaxRows, 1>());
    g.whole = whole_lds(c.R, c.K, RM) <= kLdsBudget;
    lds = g.whole ? whole_lds(c.R, c.K, RM) : slice_lds(RM);
  }
  if (fn == nullptr || lds > kLdsBudget) return hipErrorInvalidValue;
  hipError_t e = prepare_launch(fn, lds, 256);
  if (e != hipSuccess) return e;
  void* args[] = {&g};
  e = hipLaunchKernel(fn, dim3((unsigned)(padded_cols(c.N) / 32)), dim3(256), args, lds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_decode_items(const void* x, int bf16, const float* P1, int n1, const float* P2, int n2,
                               int R, float* xt, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (!decode_transform_items(n1, n2)) return hipErrorInvalidValue;
  DecodeArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.x = x;
  ga.bf16 = bf16;
  ga.P1 = P1;
  ga.P2 = P2;
  const void* fi = nullptr;
  int ilds = 0, items = 0;
#define LOOPQ_ITEM_KERNEL(n1_, n2_, rs_, nim_)                                                \
  if (n1 == n1_ && n2 == n2_) {                                                               \
    fi = reinterpret_cast<const void*>(xform_items_kernel<(n1_ + 15) / 16, n1_, n2_>);       \
    ilds = ItemPlan<n1_, n2_>::lds;                                                           \
    items = R * ((n2_ + 15) / 16);                                                            \
  }
  LOOPQ_SHAPES(LOOPQ_ITEM_KERNEL)
#undef LOOPQ_ITEM_KERNEL
  hipError_t e = prepare_launch(fi, ilds, 256);
  if (e != hipSuccess) return e;
  void* iargs[] = {&ga, &xt};
  e = hipLaunchKernel(fi, dim3((unsigned)items), dim3(256), iargs, ilds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace loopq
