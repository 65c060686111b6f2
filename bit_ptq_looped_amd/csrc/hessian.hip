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
// The contraction runs on the fp32 matrix cores (V_MFMA_F32_32X32X2_F32):
//   - H is cut into square tiles (64 or 128 wide); only tiles on or above the
//     diagonal are computed, and each tile's sum is added to H at its place
//     and, mirrored, below the diagonal, so H stays exactly symmetric.
//   - MFMA operands: lane l of a wave covers columns 2(l % 32) and
//     2(l % 32) + 1 of a 64-column strip and row l / 32 of a row pair, so
//     MFMA block p (0, 1) holds the columns of parity p; a wave keeps a
//     64 x 64 fp32 accumulator (2 x 2 blocks).
//   - 64-wide tiles (small K): a work group (4 waves) owns one tile at a
//     time; each wave takes 16 of every 64 rows, reads its operands straight
//     from global memory, and the 4 partial tiles are summed in LDS in a fixed
//     order.
//   - 128-wide tiles (K of 4000 and more, enough tiles to fill the chip):
//     each wave owns a 64 x 64 quadrant over all rows; the work group stages
//     16 rows of both 128-column strips at a time in LDS (double buffered,
//     loaded with float4), which halves the cache-to-CU traffic per flop and
//     cuts the load instructions by four.
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

namespace loopq {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kGroups = 512;     // work groups of the tile kernel (fixed: the partition sets the summation order)
constexpr int kTile = 64;        // H tile edge
constexpr int kUnitRows = 64;    // rows per work unit (16 per wave)
constexpr int kPairs = 8;        // row pairs per wave per unit
constexpr int kLds = 65;         // LDS row stride of a tile (conflict-free column reads)
constexpr int kTileLds = kTile * kLds;
constexpr int kThreads = 256;

struct HPlan {
  const float* x;
  float* H;
  float* part;       // [kGroups][2][tile * tile] pieces of split tiles
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

struct Operands {
  float2 a[kPairs], b[kPairs];
};

// This wave's 16 rows of unit c: strip i0 (A side) and strip j0 (B side).
// Columns past K (the last strip when K % 64 == 32) are clamped to K - 2:
// they only feed H elements past K, which are never stored.  RAGGED (the last
// unit when rows % 64 != 0): rows past the end are clamped to the last row
// and their A side is zeroed, so they add nothing.
template <bool RAGGED, bool DIAG>
__device__ __forceinline__ void load_unit(Operands& o, const HPlan& p, int c, int i0, int j0, int wave,
                                          int lane) {
  const int col = 2 * (lane & 31);
  const int ca = min(i0 + col, p.K - 2), cb = min(j0 + col, p.K - 2);
  const int row0 = c * kUnitRows + 16 * wave;  // wave-uniform
  const float* base = p.x + (size_t)row0 * p.K;
  if (!RAGGED) {
    const int la = (lane >> 5) * p.K + ca, lb = (lane >> 5) * p.K + cb;
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const float* bk = base + (size_t)(2 * k) * p.K;
      o.a[k] = *reinterpret_cast<const float2*>(bk + la);
      if (!DIAG) o.b[k] = *reinterpret_cast<const float2*>(bk + lb);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int r = row0 + 2 * k + (lane >> 5);
      const bool ok = r < p.rows;
      const size_t ro = (size_t)(ok ? r : p.rows - 1) * p.K;
      const float2 a = *reinterpret_cast<const float2*>(p.x + ro + ca);
      o.a[k] = ok ? a : make_float2(0.0f, 0.0f);
      if (!DIAG) o.b[k] = *reinterpret_cast<const float2*>(p.x + ro + cb);
    }
  }
}

template <bool DIAG>
__device__ __forceinline__ void mfma_unit(v16f acc[4], const Operands& o) {
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const float2 a = o.a[k];
    const float2 b = DIAG ? a : o.b[k];
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.y, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.x, acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc[3], 0, 0, 0);
  }
}

// Sum of units [c0, c1) of tile (ti, tj) into this wave's accumulator.  Two
// operand sets alternate: the loads of the next unit are in flight while the
// MFMAs of the current one run.
template <bool DIAG>
__device__ void run_units_t(v16f acc[4], const HPlan& p, int ti, int tj, int c0, int c1, int wave, int lane) {
  const int i0 = ti * kTile, j0 = tj * kTile;
  const int ragged = p.rows % kUnitRows ? p.nc - 1 : -1;  // the unit with rows past the end
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.0f;
  auto load = [&](Operands& o, int c) {
    if (c == ragged)
      load_unit<true, DIAG>(o, p, c, i0, j0, wave, lane);
    else
      load_unit<false, DIAG>(o, p, c, i0, j0, wave, lane);
  };
  Operands u0, u1;
  load(u0, c0);
  int c = c0;
  for (; c + 1 < c1; c += 2) {
    load(u1, c + 1);
    mfma_unit<DIAG>(acc, u0);
    if (c + 2 < c1) load(u0, c + 2);
    mfma_unit<DIAG>(acc, u1);
  }
  if (c < c1) mfma_unit<DIAG>(acc, u0);
}

__device__ __forceinline__ void run_units(v16f acc[4], const HPlan& p, int ti, int tj, int c0, int c1, int wave,
                                          int lane) {
  if (ti == tj)
    run_units_t<true>(acc, p, ti, tj, c0, c1, wave, lane);
  else
    run_units_t<false>(acc, p, ti, tj, c0, c1, wave, lane);
}

// The 4 waves' accumulators -> one 64 x 64 tile sum in lds[0 .. kTileLds).
// Result element (i, j) of MFMA block (pa, pb) is H[i0 + 2i + pa][j0 + 2j + pb];
// lane l, element e holds i = 8 (e / 4) + 4 (l / 32) + e % 4, j = l % 32.
__device__ void reduce_waves(const v16f acc[4], float* lds, int wave, int lane) {
  __syncthreads();  // the previous tile's readers are done
  float* P = lds + wave * kTileLds;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int pa = blk >> 1, pb = blk & 1;
    const int b = 2 * (lane & 31) + pb;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      P[(2 * i + pa) * kLds + b] = acc[blk][e];
    }
  }
  __syncthreads();
  for (int k = 0; k < 16; ++k) {
    const int e = threadIdx.x + kThreads * k;
    const int o = (e >> 6) * kLds + (e & 63);
    lds[o] = (lds[o] + lds[kTileLds + o]) + (lds[2 * kTileLds + o] + lds[3 * kTileLds + o]);
  }
  __syncthreads();
}

// H[i0 + a][j0 + b] += S[a][b] and, mirrored, H[j0 + b][i0 + a] += S[a][b];
// a diagonal tile takes a <= b from S for the upper half and a < b for the
// lower, so both halves come from the same values.  Each thread handles E
// elements of a pass with its W-wide lane group; the H values of a batch of
// 16 are all loaded before any is stored, so the loads overlap.
template <int W, typename At>
__device__ __forceinline__ void add_tile_pass(const HPlan& p, At at, int i0, int j0, bool diag, bool mirror) {
  constexpr int E = W * W / kThreads, R = kThreads / W;
  const int K = p.K, t = threadIdx.x;
  const int lo = t % W, hi = t / W;
  // element k of this thread: (a, b), its H offset, and whether it is stored
  auto elem = [&](int k, int* a, int* b, size_t* off) {
    *a = mirror ? lo : hi + R * k;
    *b = mirror ? hi + R * k : lo;
    const int i = i0 + *a, j = j0 + *b;
    *off = mirror ? (size_t)j * K + i : (size_t)i * K + j;
    return i < K && j < K && (!diag || (mirror ? *a < *b : *a <= *b));
  };
#pragma unroll 1
  for (int k0 = 0; k0 < E; k0 += 16) {
    float h[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      int a, b;
      size_t off;
      h[k] = elem(k0 + k, &a, &b, &off) ? p.H[off] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      int a, b;
      size_t off;
      if (elem(k0 + k, &a, &b, &off)) p.H[off] = h[k] + at(a, b);
    }
  }
}

__device__ void add_tile(const HPlan& p, const float* S, int ti, int tj) {
  auto at = [S](int a, int b) { return S[a * kLds + b]; };
  const bool diag = ti == tj;
  add_tile_pass<kTile>(p, at, ti * kTile, tj * kTile, diag, false);
  add_tile_pass<kTile>(p, at, ti * kTile, tj * kTile, diag, true);
}

// ---------------------------------------------------------------------------
// 128-wide tiles: LDS-staged operands, one 64 x 64 quadrant per wave
// ---------------------------------------------------------------------------
constexpr int kBig = 128;
constexpr int kStep = 16;                    // rows per LDS stage
constexpr int kStrip = kStep * kBig;         // floats of one staged strip
constexpr int kStage = 2 * kStrip;           // A and B strips of one stage

// Rows [row0, row0 + 16) of the 128-column strips at i0 (A) and j0 (B) into
// registers, two float4 per thread and strip.  Columns past K are clamped to
// K - 4 (their outputs are never stored); RAGGED clamps rows past the end to
// the last row and zeroes their A side.
struct StageRegs {
  float4 a0, a1, b0, b1;
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
  r.b0 = r.b1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  r.a0 = stage_elem<RAGGED, DIAG>(p, row0, i0, j0, threadIdx.x, &r.b0);
  r.a1 = stage_elem<RAGGED, DIAG>(p, row0, i0, j0, threadIdx.x + kThreads, &r.b1);
  return r;
}

// registers -> one LDS stage ([16][128] A, then [16][128] B; a diagonal tile
// keeps only A)
template <bool DIAG>
__device__ __forceinline__ void stage_store(float* stage, const StageRegs& r) {
  const int e = threadIdx.x;
  *reinterpret_cast<float4*>(stage + 4 * e) = r.a0;
  *reinterpret_cast<float4*>(stage + 4 * (e + kThreads)) = r.a1;
  if (!DIAG) {
    *reinterpret_cast<float4*>(stage + kStrip + 4 * e) = r.b0;
    *reinterpret_cast<float4*>(stage + kStrip + 4 * (e + kThreads)) = r.b1;
  }
}

// this wave's quadrant (qa, qb) over the 16 staged rows
template <bool DIAG>
__device__ __forceinline__ void stage_mfma(v16f acc[4], const float* stage, int qa, int qb, int lane) {
  const int lo = (lane >> 5) * kBig + 2 * (lane & 31);
  const float* A = stage + 64 * qa + lo;
  const float* B = stage + (DIAG ? 0 : kStrip) + 64 * qb + lo;
#pragma unroll
  for (int k = 0; k < kStep / 2; ++k) {
    const float2 a = *reinterpret_cast<const float2*>(A + 2 * k * kBig);
    const float2 b = *reinterpret_cast<const float2*>(B + 2 * k * kBig);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.y, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.x, acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc[3], 0, 0, 0);
  }
}

// Units [c0, c1) of tile (ti, tj): the stage after the current one is loaded
// into registers while the current one is multiplied, then stored to the
// other LDS buffer; one barrier per stage.  On a diagonal tile quadrant
// (1, 0) is the transpose of (0, 1) and is never read, so wave 2 idles.
template <bool DIAG>
__device__ void run_units_big_t(v16f acc[4], float* lds, const HPlan& p, int ti, int tj, int c0, int c1, int wave,
                                int lane) {
  const int i0 = ti * kBig, j0 = tj * kBig;
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

__device__ __forceinline__ void run_units_big(v16f acc[4], float* lds, const HPlan& p, int ti, int tj, int c0,
                                              int c1, int wave, int lane) {
  if (ti == tj)
    run_units_big_t<true>(acc, lds, p, ti, tj, c0, c1, wave, lane);
  else
    run_units_big_t<false>(acc, lds, p, ti, tj, c0, c1, wave, lane);
}

// S(a, b) of a 128-wide tile held as four 64 x 65 quadrants in LDS
__device__ __forceinline__ float big_at(const float* S, int a, int b) {
  return S[((a >> 6) * 2 + (b >> 6)) * kTileLds + (a & 63) * kLds + (b & 63)];
}

// this wave's accumulator -> its quadrant of S (element mapping as in reduce_waves)
__device__ void write_quadrant(const v16f acc[4], float* Q, int lane) {
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

// add_tile for a 128-wide tile
__device__ void add_tile_big(const HPlan& p, const float* S, int ti, int tj) {
  auto at = [S](int a, int b) { return big_at(S, a, b); };
  const bool diag = ti == tj;
  add_tile_pass<kBig>(p, at, ti * kBig, tj * kBig, diag, false);
  add_tile_pass<kBig>(p, at, ti * kBig, tj * kBig, diag, true);
}

// ---------------------------------------------------------------------------
// partition and pieces, shared by both tile sizes
// ---------------------------------------------------------------------------

// A piece of a 64-wide tile is stored row-major [64][64]; one of a 128-wide
// tile in the accumulator layout [wave][block][element][lane], written
// straight from the registers.
template <int TILE>
__device__ void run_segment(v16f acc[4], float* lds, const HPlan& p, int u, int c0, int c1, float* piece, int wave,
                            int lane) {
  int ti, tj;
  tile_of(u, &ti, &tj);
  const bool whole = c0 == 0 && c1 == p.nc;
  if (TILE == kTile) {
    run_units(acc, p, ti, tj, c0, c1, wave, lane);
    reduce_waves(acc, lds, wave, lane);
    if (whole) {
      add_tile(p, lds, ti, tj);
    } else {
      for (int k = 0; k < 16; ++k) {
        const int e = threadIdx.x + kThreads * k;
        piece[e] = lds[(e >> 6) * kLds + (e & 63)];
      }
    }
  } else {
    run_units_big(acc, lds, p, ti, tj, c0, c1, wave, lane);
    if (whole) {  // the last stage's barrier has retired every staging read
      write_quadrant(acc, lds + wave * kTileLds, lane);
      __syncthreads();
      add_tile_big(p, lds, ti, tj);
    } else {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int e = 0; e < 16; ++e) piece[((wave * 4 + blk) * 16 + e) * 64 + lane] = acc[blk][e];
    }
  }
}

template <int TILE>
__global__ __launch_bounds__(kThreads) void hessian_tiles_kernel(HPlan p) {
  extern __shared__ float lds[];  // 4 * kTileLds floats
  const int g = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  v16f acc[4];
  // whole tiles, round robin
  for (int k = 0; k < p.q; ++k) run_segment<TILE>(acc, lds, p, g + kGroups * k, 0, p.nc, nullptr, wave, lane);
  if (p.r == 0) return;
  // leftover tiles: this work group's contiguous range of units
  const long long v_end = unit_start(g + 1, p.wr);
  long long v = unit_start(g, p.wr);
  bool first = true;
  while (v < v_end) {
    const int t = (int)(v / p.nc);
    const int c0 = (int)(v - (long long)t * p.nc);
    const long long tile_end = (long long)(t + 1) * p.nc;
    const int c1 = (int)((v_end < tile_end ? v_end : tile_end) - (long long)t * p.nc);
    // slot 0 for this work group's first range, 1 for its last
    float* piece = p.part + ((size_t)g * 2 + (first ? 0 : 1)) * (TILE * TILE);
    run_segment<TILE>(acc, lds, p, p.q * kGroups + t, c0, c1, piece, wave, lane);
    first = false;
    v = (long long)t * p.nc + c1;
  }
}

// Adds up the pieces of each leftover tile that was split across work
// groups, in work-group order, and adds the sum to H.  Block (t, y) takes 256
// elements of leftover tile t (in the piece layout), one per thread, with up
// to 8 piece loads in flight.
template <int TILE>
__global__ __launch_bounds__(kThreads) void hessian_pieces_kernel(HPlan p) {
  const int t = blockIdx.x;
  const int e = blockIdx.y * kThreads + threadIdx.x;
  const long long v0 = (long long)t * p.nc, v1 = v0 + p.nc;
  const int gf = unit_owner(v0, p.wr), gl = unit_owner(v1 - 1, p.wr);
  if (gf == gl) return;  // covered by one work group, added there
  float sum = 0.0f;
  bool have = false;
  for (int g0 = gf; g0 <= gl; g0 += 8) {
    float v[8];
    bool use[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int g = g0 + k;
      const long long st = unit_start(g, p.wr);
      use[k] = g <= gl && st < unit_start(g + 1, p.wr);  // empty ranges hold no piece
      const float* src = p.part + ((size_t)g * 2 + (st >= v0 ? 0 : 1)) * (TILE * TILE);
      v[k] = use[k] ? src[e] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (use[k]) {
        sum = have ? sum + v[k] : v[k];
        have = true;
      }
    }
  }
  int a, b;
  if (TILE == kTile) {  // row-major [64][64]
    a = e >> 6;
    b = e & 63;
  } else {  // e = ((wave * 4 + block) * 16 + element) * 64 + lane
    const int lane = e & 63, el = (e >> 6) & 15, blk = (e >> 10) & 3, w = e >> 12;
    a = 64 * (w >> 1) + 2 * (8 * (el >> 2) + 4 * (lane >> 5) + (el & 3)) + (blk >> 1);
    b = 64 * (w & 1) + 2 * (lane & 31) + (blk & 1);
  }
  int ti, tj;
  tile_of(p.q * kGroups + t, &ti, &tj);
  const bool diag = ti == tj;
  const int i = ti * TILE + a, j = tj * TILE + b, K = p.K;
  if (i >= K || j >= K) return;
  if (!diag || a <= b) p.H[(size_t)i * K + j] += sum;
  if (!diag || a < b) p.H[(size_t)j * K + i] += sum;
}

int tiles_of(int K, int tile) {
  const int nt = (K + tile - 1) / tile;
  return nt * (nt + 1) / 2;
}

// 128-wide tiles once there are enough of them for every work group
int tile_for(int K) { return tiles_of(K, kBig) >= kGroups ? kBig : kTile; }

HPlan make_plan(const float* x, int rows, int K, float* H, float* part, int tile) {
  HPlan p{};
  p.x = x;
  p.H = H;
  p.part = part;
  p.rows = rows;
  p.K = K;
  const int ntiles = tiles_of(K, tile);
  p.nc = (rows + kUnitRows - 1) / kUnitRows;
  p.q = ntiles / kGroups;
  p.r = ntiles % kGroups;
  p.wr = (long long)p.r * p.nc;
  return p;
}

template <int TILE>
hipError_t launch_tiles(const HPlan& p, hipStream_t s) {
  const size_t lds = (size_t)4 * kTileLds * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(hessian_tiles_kernel<TILE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hessian_tiles_kernel<TILE>, dim3(kGroups), dim3(kThreads), lds, s, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.r == 0) return e;
  hipLaunchKernelGGL(hessian_pieces_kernel<TILE>, dim3(p.r, TILE * TILE / kThreads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

size_t hessian_workspace_bytes(int K) {
  const int tile = tile_for(K);
  return tiles_of(K, tile) % kGroups ? (size_t)kGroups * 2 * tile * tile * sizeof(float) : 0;
}

hipError_t launch_hessian(const float* x, int rows, int K, float* H, float* part, hipStream_t s) {
  const int tile = tile_for(K);
  const HPlan p = make_plan(x, rows, K, H, part, tile);
  return tile == kBig ? launch_tiles<kBig>(p, s) : launch_tiles<kTile>(p, s);
}

}  // namespace loopq
