// Trajectory Hessian accumulation H += X~^T X~ over the transformed inputs
// x~ of every loop of a looped linear.
//
// "Quantizing Looped Transformers: Feedback Exposure and Calibration
// Blindness" calibrates GPTQ on a Hessian summed over the recurrence steps,
// H = sum_t X_t^T X_t (its N-step calibration, Tables 19 and 25; Table 1
// reports the rank of such Hessians), one fp32 [K][K] matrix per linear (the
// GPTQ memory note of the same page set).  Stacking the rows of every loop,
// the sum is one symmetric rank-k update of H by all rows.
//
// The contraction runs on the bf16 matrix cores (V_MFMA_F32_32X32X16_BF16):
// every fp32 x~ value is split into three bf16 planes whose sum is the value
// exactly (hi = the value truncated to bf16, mid = the remainder truncated,
// lo = the rest), and each product x~_ri x~_rj is taken as the six plane
// products of order <= 2 (mid mid, lo hi, hi lo, mid hi, hi mid, hi hi per
// step of 16 rows, in that order), each exact in fp32; the dropped mid lo,
// lo mid and lo lo are below 2^-20 of |x~_ri x~_rj|.  Accumulation is fp32.
// Six bf16 products take 6 x 32 cycles per 32 x 32 block and 16 rows against
// 8 x 64 for the fp32 MFMA (V_MFMA_F32_32X32X2_F32).
//   - H is cut into 128 x 128 tiles; only tiles on or above the diagonal are
//     computed, and each tile's sum is added to H at its place and, mirrored,
//     below the diagonal, so H stays exactly symmetric.
//   - A work group (4 waves) owns one tile at a time and stages 32 rows of
//     both 128-column strips at a time in LDS (double buffered, float4 loads
//     from global memory); each wave keeps a 64 x 64 quadrant of the tile in
//     a fp32 accumulator (2 x 2 MFMA blocks) over all rows.
//   - MFMA operands: lane l reads columns 2(l % 32) and 2(l % 32) + 1 of its
//     64-column half strip for rows 8 (l / 32) .. + 7 of a 16-row step and
//     splits them into the planes, so MFMA block p (0, 1) holds the columns
//     of parity p.
//   - Work balance: the grid is a fixed number of work groups (kGroups, two
//     per compute unit of a 256-CU part).  Whole tiles are dealt out round
//     robin; the tiles left over (fewer than kGroups) are cut into 64-row
//     units and the units split evenly, in tile order, across all work
//     groups.  A leftover tile one work group covers entirely is added
//     directly; the pieces of one split across several are written to the
//     workspace and a second kernel adds them up in work-group order.  The
//     summation order depends only on (rows, K), so results are
//     deterministic.
#include <math.h>

#include "loopq_internal.h"
#include "quant_core.h"

namespace loopq {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kGroups = 512;     // work groups of the tile kernel (fixed: the partition sets the summation order)
constexpr int kTile = 128;       // H tile edge
constexpr int kUnitRows = 64;    // rows per work unit
constexpr int kStep = 32;        // rows per LDS stage
constexpr int kStrip = kStep * kTile;  // floats of one staged strip
constexpr int kStage = 2 * kStrip;     // A and B strips of one stage
constexpr int kLds = 65;         // LDS row stride of a 64 x 64 quadrant (conflict-free column reads)
constexpr int kQuadLds = 64 * kLds;
constexpr int kThreads = 256;

struct HPlan {
  const float* x;
  float* H;
  float* part;       // [kGroups][2][128 * 128] pieces of split tiles
  int rows, K;
  int nc;            // units per tile: ceil(rows / 64)
  int q;             // whole tiles per work group
  int r;             // leftover tiles (split by units)
  long long wr;      // leftover units r * nc
};

// column-major order over the upper triangle: u = tj (tj + 1) / 2 + ti, ti <= tj
__device__ __forceinline__ void tile_of(int u, int* ti, int* tj) {
  int t = (int)((sqrtf(8.0f * (float)u + 1.0f) - 1.0f) * 0.5f);
  while ((t + 1) * (t + 2) / 2 <= u) ++t;
  while (t * (t + 1) / 2 > u) --t;
  *tj = t;
  *ti = u - t * (t + 1) / 2;
}

__device__ __forceinline__ long long unit_start(int g, long long wr) { return (long long)g * wr / kGroups; }

// first work group whose unit range holds unit v (its range is not empty)
__device__ __forceinline__ int unit_owner(long long v, long long wr) {
  return (int)(((v + 1) * kGroups + wr - 1) / wr) - 1;
}

// Rows [row0, row0 + kStep) of the 128-column strips at i0 (A) and j0 (B)
// into registers, kLoads float4 per thread and strip.  Columns past K are clamped to
// K - 4 (their outputs are never stored); RAGGED clamps rows past the end to
// the last row and zeroes their A side, so they add nothing.
constexpr int kLoads = kStrip / (4 * kThreads);  // float4 per thread and strip

struct StageRegs {
  float4 a[kLoads], b[kLoads];
};

template <bool RAGGED, bool DIAG>
__device__ __forceinline__ float4 stage_elem(const HPlan& p, int row0, int i0, int j0, int e, float4* bv) {
  const int c = 4 * (e & 31);
  int row = row0 + (e >> 5);
  const bool ok = !RAGGED || row < p.rows;
  if (RAGGED && !ok) row = p.rows - 1;
  const float* src = p.x + (size_t)row * p.K;
  const float4 a = *reinterpret_cast<const float4*>(src + min(i0 + c, p.K - 4));
  if (!DIAG) *bv = *reinterpret_cast<const float4*>(src + min(j0 + c, p.K - 4));
  return ok ? a : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

template <bool RAGGED, bool DIAG>
__device__ __forceinline__ StageRegs stage_load(const HPlan& p, int row0, int i0, int j0) {
  StageRegs r;
#pragma unroll
  for (int h = 0; h < kLoads; ++h) {
    r.b[h] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    r.a[h] = stage_elem<RAGGED, DIAG>(p, row0, i0, j0, threadIdx.x + kThreads * h, &r.b[h]);
  }
  return r;
}

// registers -> one LDS stage ([kStep][128] A, then [kStep][128] B; a
// diagonal tile keeps only A)
template <bool DIAG>
__device__ __forceinline__ void stage_store(float* stage, const StageRegs& r) {
#pragma unroll
  for (int h = 0; h < kLoads; ++h) {
    const int e = threadIdx.x + kThreads * h;
    *reinterpret_cast<float4*>(stage + 4 * e) = r.a[h];
    if (!DIAG) *reinterpret_cast<float4*>(stage + kStrip + 4 * e) = r.b[h];
  }
}

// The three bf16 planes (hi + mid + lo = v exactly: hi = v truncated to
// bf16, mid = the remainder truncated, lo = the rest, as split3_bf16) of 8
// consecutive staged rows of two adjacent columns (P, row stride kTile): the
// MFMA operand of the column of parity p with the 8 rows as its K slots,
// pl[p][plane].  A plane value is the upper half of an fp32 word (v, then
// r1 = v - hi, then r2 = r1 - mid, each difference exact), so each pair of
// K slots is one byte permute of two such words (top_halves).
__device__ __forceinline__ void planes_rows8(const float* P, v4u (&pl)[2][3]) {
  float2 v[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = *reinterpret_cast<const float2*>(P + t * kTile);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float e0 = v[2 * k].x, e1 = v[2 * k + 1].x, o0 = v[2 * k].y, o1 = v[2 * k + 1].y;
    const float e0m = minus_top(e0), e1m = minus_top(e1), o0m = minus_top(o0), o1m = minus_top(o1);
    pl[0][0][k] = top_halves(e0, e1);
    pl[0][1][k] = top_halves(e0m, e1m);
    pl[0][2][k] = top_halves(minus_top(e0m), minus_top(e1m));
    pl[1][0][k] = top_halves(o0, o1);
    pl[1][1][k] = top_halves(o0m, o1m);
    pl[1][2][k] = top_halves(minus_top(o0m), minus_top(o1m));
  }
}

__device__ __forceinline__ v16f mm16(const v4u& a, const v4u& b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// this wave's quadrant (qa, qb) over the staged rows, 16 rows per step on the
// bf16 MFMA: both operands as three exact bf16 planes and the six plane
// products of order <= 2, smallest first (mid mid, lo hi, hi lo, mid hi,
// hi mid, hi hi), into one fp32 accumulator per block.  Lane l takes columns
// 2 (l % 32) and 2 (l % 32) + 1 of its half strip (block (pa, pb) holds the
// columns of parities pa and pb) and rows 8 (l / 32) .. + 7 of the step.
template <bool DIAG>
__device__ __forceinline__ void stage_mfma(v16f acc[4], const float* stage, int qa, int qb, int lane) {
  const int lo = (lane >> 5) * 8 * kTile + 2 * (lane & 31);
  const float* A = stage + 64 * qa + lo;
  const float* B = stage + (DIAG ? 0 : kStrip) + 64 * qb + lo;
  constexpr int pa_of[6] = {1, 2, 0, 1, 0, 0};
  constexpr int pb_of[6] = {1, 0, 2, 0, 1, 0};
#pragma unroll
  for (int k = 0; k < kStep / 16; ++k) {
    v4u a[2][3], b[2][3];
    planes_rows8(A + 16 * k * kTile, a);
    planes_rows8(B + 16 * k * kTile, b);
#pragma unroll
    for (int q = 0; q < 6; ++q)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
        acc[blk] = mm16(a[blk >> 1][pa_of[q]], b[blk & 1][pb_of[q]], acc[blk]);
  }
}

// Units [c0, c1) of tile (ti, tj): the stage after the current one is loaded
// into registers while the current one is multiplied, then stored to the
// other LDS buffer; one barrier per stage.  On a diagonal tile quadrant
// (1, 0) is the transpose of (0, 1) and is never read, so wave 2 idles.
template <bool DIAG>
__device__ void run_units_t(v16f acc[4], float* lds, const HPlan& p, int ti, int tj, int c0, int c1, int wave,
                            int lane) {
  const int i0 = ti * kTile, j0 = tj * kTile;
  const int qa = wave >> 1, qb = wave & 1;
  const bool idle = DIAG && wave == 2;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.0f;
  const int s0 = c0 * (kUnitRows / kStep), s1 = c1 * (kUnitRows / kStep);
  __syncthreads();  // the previous tile's LDS readers are done
  {
    const int row0 = s0 * kStep;
    const StageRegs r = row0 + kStep > p.rows ? stage_load<true, DIAG>(p, row0, i0, j0)
                                              : stage_load<false, DIAG>(p, row0, i0, j0);
    stage_store<DIAG>(lds, r);
  }
  __syncthreads();
  for (int st = s0; st < s1; ++st) {
    float* cur = lds + ((st - s0) & 1) * kStage;
    float* nxt = lds + (((st - s0) & 1) ^ 1) * kStage;
    const bool more = st + 1 < s1;
    const int row0 = (st + 1) * kStep;
    StageRegs r;
    if (more)
      r = row0 + kStep > p.rows ? stage_load<true, DIAG>(p, row0, i0, j0) : stage_load<false, DIAG>(p, row0, i0, j0);
    if (!idle) stage_mfma<DIAG>(acc, cur, qa, qb, lane);
    if (more) stage_store<DIAG>(nxt, r);
    __syncthreads();
  }
}

__device__ __forceinline__ void run_units(v16f acc[4], float* lds, const HPlan& p, int ti, int tj, int c0, int c1,
                                          int wave, int lane) {
  if (ti == tj)
    run_units_t<true>(acc, lds, p, ti, tj, c0, c1, wave, lane);
  else
    run_units_t<false>(acc, lds, p, ti, tj, c0, c1, wave, lane);
}

// This wave's accumulator -> its quadrant of S (four 64 x 65 quadrants in
// LDS).  Element e of MFMA block (pa, pb) in lane l is quadrant element
// (2 i + pa, 2 j + pb) with i = 8 (e / 4) + 4 (l / 32) + e % 4, j = l % 32.
__device__ void write_quadrant(const v16f acc[4], float* S, int wave, int lane) {
  float* Q = S + wave * kQuadLds;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int pa = blk >> 1, pb = blk & 1;
    const int b = 2 * (lane & 31) + pb;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      Q[(2 * i + pa) * kLds + b] = acc[blk][e];
    }
  }
}

// Quadrant w = (qa, qb) of tile (ti, tj), held in LDS as Q[64][65], added
// to H: H[i0 + a][j0 + b] += Q[a][b] (mirror = false) or H[j0 + b][i0 + a]
// += Q[a][b] (mirror = true), (i0, j0) the quadrant's origin.  On the
// diagonal of H (ti == tj and qa == qb) the upper half takes a <= b and the
// mirror a < b, so both halves come from the same values; quadrant (1, 0) of
// a diagonal tile is the mirror of (0, 1) and is skipped.  Each thread takes
// 16 elements, with 64 consecutive lanes along the contiguous index of H; the
// H values of a batch of 8 are all loaded before any is stored.
__device__ void add_quadrant_pass(const HPlan& p, const float* Q, int ti, int tj, int w, bool mirror) {
  const int qa = w >> 1, qb = w & 1;
  const bool dq = ti == tj && qa == qb;
  const int i0 = ti * kTile + 64 * qa, j0 = tj * kTile + 64 * qb, K = p.K, t = threadIdx.x;
  const int lo = t & 63, hi = t >> 6;
  auto elem = [&](int k, int* a, int* b, size_t* off) {
    *a = mirror ? lo : hi + 4 * k;
    *b = mirror ? hi + 4 * k : lo;
    const int i = i0 + *a, j = j0 + *b;
    *off = mirror ? (size_t)j * K + i : (size_t)i * K + j;
    return i < K && j < K && (!dq || (mirror ? *a < *b : *a <= *b));
  };
#pragma unroll
  for (int k0 = 0; k0 < 16; k0 += 8) {
    float h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int a, b;
      size_t off;
      h[k] = elem(k0 + k, &a, &b, &off) ? p.H[off] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int a, b;
      size_t off;
      if (elem(k0 + k, &a, &b, &off)) p.H[off] = h[k] + Q[a * kLds + b];
    }
  }
}

__device__ void add_quadrant(const HPlan& p, const float* Q, int ti, int tj, int w) {
  if (ti == tj && w == 2) return;
  add_quadrant_pass(p, Q, ti, tj, w, false);
  add_quadrant_pass(p, Q, ti, tj, w, true);
}

// Units [c0, c1) of tile u.  A whole tile is added to H here; a piece of a
// split one goes to `piece` in the accumulator layout
// [wave][block][element][lane], straight from the registers.
__device__ void run_segment(v16f acc[4], float* lds, const HPlan& p, int u, int c0, int c1, float* piece, int wave,
                            int lane) {
  int ti, tj;
  tile_of(u, &ti, &tj);
  run_units(acc, lds, p, ti, tj, c0, c1, wave, lane);
  if (c0 == 0 && c1 == p.nc) {  // the last stage's barrier has retired every staging read
    write_quadrant(acc, lds, wave, lane);
    __syncthreads();
#pragma unroll 1
    for (int w = 0; w < 4; ++w) add_quadrant(p, lds + w * kQuadLds, ti, tj, w);
  } else {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) piece[((wave * 4 + blk) * 16 + e) * 64 + lane] = acc[blk][e];
  }
}

__global__ __launch_bounds__(kThreads, 2) void hessian_tiles_kernel(HPlan p) {
  extern __shared__ float lds[];  // max(2 stages, 4 quadrants) floats
  // Logical work group g: the hardware dispatches consecutive work groups to
  // the 8 XCDs in turn, so g = 64 * (XCD) + (slot) gives each XCD a run of
  // 64 consecutive logical groups -- neighbouring tiles, which share column
  // strips of the same rows, then read them through one L2.  The partition
  // (and so the summation order) is that of g alone.
  const int g = (int)(blockIdx.x & 7) * (kGroups / 8) + (int)(blockIdx.x >> 3);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  v16f acc[4];
  // whole tiles round robin (k < q), then this work group's contiguous range
  // of units of the leftover tiles; one call site keeps one copy of the loop
  const long long v_end = p.r ? unit_start(g + 1, p.wr) : 0;
  long long v = p.r ? unit_start(g, p.wr) : 0;
  int k = 0;
  bool first = true;
  for (;;) {
    int u, c0, c1;
    float* piece = nullptr;
    if (k < p.q) {
      u = g + kGroups * k++;
      c0 = 0;
      c1 = p.nc;
    } else {
      if (v >= v_end) break;
      const int t = (int)(v / p.nc);
      c0 = (int)(v - (long long)t * p.nc);
      const long long tile_end = (long long)(t + 1) * p.nc;
      c1 = (int)((v_end < tile_end ? v_end : tile_end) - (long long)t * p.nc);
      u = p.q * kGroups + t;
      // slot 0 for this work group's first range, 1 for its last
      piece = p.part + ((size_t)g * 2 + (first ? 0 : 1)) * (kTile * kTile);
      first = false;
      v = (long long)t * p.nc + c1;
    }
    run_segment(acc, lds, p, u, c0, c1, piece, wave, lane);
  }
}

// Adds up the pieces of each leftover tile that was split across work
// groups, in work-group order, and adds the sum to H.  Block (t, w) takes
// quadrant w of leftover tile t: in the piece layout [wave][block][element]
// [lane] that is the contiguous block of wave w, 16 elements per thread.
__global__ __launch_bounds__(kThreads) void hessian_pieces_kernel(HPlan p) {
  __shared__ float Q[kQuadLds];
  const int t = blockIdx.x, w = blockIdx.y;
  const long long v0 = (long long)t * p.nc, v1 = v0 + p.nc;
  const int gf = unit_owner(v0, p.wr), gl = unit_owner(v1 - 1, p.wr);
  if (gf == gl) return;  // covered by one work group, added there
  int ti, tj;
  tile_of(p.q * kGroups + t, &ti, &tj);
  if (ti == tj && w == 2) return;  // the mirror of quadrant (0, 1)
  float sum[16];
  bool have = false;
  for (int g = gf; g <= gl; ++g) {
    const long long st = unit_start(g, p.wr);
    if (st == unit_start(g + 1, p.wr)) continue;  // empty ranges hold no piece
    const float* src = p.part + ((size_t)g * 2 + (st >= v0 ? 0 : 1)) * (kTile * kTile) + w * 4096;
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = src[threadIdx.x + kThreads * k];
#pragma unroll
    for (int k = 0; k < 16; ++k) sum[k] = have ? sum[k] + v[k] : v[k];
    have = true;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {  // element ((block * 16) + el) * 64 + lane of the quadrant
    const int e = threadIdx.x + kThreads * k;
    const int lane = e & 63, el = (e >> 6) & 15, blk = e >> 10;
    const int i = 8 * (el >> 2) + 4 * (lane >> 5) + (el & 3);
    Q[(2 * i + (blk >> 1)) * kLds + 2 * (lane & 31) + (blk & 1)] = sum[k];
  }
  __syncthreads();
  add_quadrant(p, Q, ti, tj, w);
}

int tiles_of(int K) {
  const int nt = (K + kTile - 1) / kTile;
  return nt * (nt + 1) / 2;
}

HPlan make_plan(const float* x, int rows, int K, float* H, float* part) {
  HPlan p{};
  p.x = x;
  p.H = H;
  p.part = part;
  p.rows = rows;
  p.K = K;
  const int ntiles = tiles_of(K);
  p.nc = (rows + kUnitRows - 1) / kUnitRows;
  p.q = ntiles / kGroups;
  p.r = ntiles % kGroups;
  p.wr = (long long)p.r * p.nc;
  return p;
}

constexpr size_t kLdsBytes = (4 * kQuadLds > 2 * kStage ? 4 * kQuadLds : 2 * kStage) * sizeof(float);

}  // namespace

size_t hessian_workspace_bytes(int K) {
  return tiles_of(K) % kGroups ? (size_t)kGroups * 2 * kTile * kTile * sizeof(float) : 0;
}

hipError_t launch_hessian(const float* x, int rows, int K, float* H, float* part, hipStream_t s) {
  const HPlan p = make_plan(x, rows, K, H, part);
  hipError_t e = prepare_launch(reinterpret_cast<const void*>(hessian_tiles_kernel), (int)kLdsBytes, kThreads);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hessian_tiles_kernel, dim3(kGroups), dim3(kThreads), kLdsBytes, s, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.r == 0) return e;
  hipLaunchKernelGGL(hessian_pieces_kernel, dim3(p.r, 4), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace loopq
