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
//   - H is cut into 64 x 64 tiles; only tiles on or above the diagonal are
//     computed, and each tile's sum is added to H at its place and, mirrored,
//     below the diagonal, so H stays exactly symmetric.
//   - A work group (4 waves) owns one tile at a time; each wave takes 16 of
//     every 64 rows and holds a full 64 x 64 fp32 accumulator (2 x 2 MFMA
//     blocks).  Operands are read straight from global memory as float2:
//     lane l of a wave covers columns 2(l % 32) and 2(l % 32) + 1 of the
//     strip and row l / 32 of the row pair, so MFMA block p (0, 1) holds the
//     columns of parity p.  The 4 partial tiles are summed in LDS in a fixed
//     order.
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
  float* part;       // [kGroups][2][64 * 64] pieces of split tiles
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

__device__ __forceinline__ float2 load_pair(const float* x, int rows, int K, int row, int col) {
  const bool ok = row < rows && col < K;
  const float2 v = *reinterpret_cast<const float2*>(x + (ok ? (size_t)row * K + col : 0));
  return ok ? v : make_float2(0.0f, 0.0f);
}

struct Operands {
  float2 a[kPairs], b[kPairs];
};

// this wave's 16 rows of unit c: strip i0 (A side) and strip j0 (B side)
__device__ __forceinline__ void load_unit(Operands& o, const HPlan& p, int c, int i0, int j0, bool diag,
                                          int wave, int lane) {
  const int col = 2 * (lane & 31);
  const int row = c * kUnitRows + 16 * wave + (lane >> 5);
#pragma unroll
  for (int k = 0; k < kPairs; ++k) o.a[k] = load_pair(p.x, p.rows, p.K, row + 2 * k, i0 + col);
  if (!diag) {
#pragma unroll
    for (int k = 0; k < kPairs; ++k) o.b[k] = load_pair(p.x, p.rows, p.K, row + 2 * k, j0 + col);
  }
}

__device__ __forceinline__ void mfma_unit(v16f acc[4], const Operands& o, bool diag) {
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const float2 a = o.a[k];
    const float2 b = diag ? a : o.b[k];
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.y, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.x, acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc[3], 0, 0, 0);
  }
}

// Sum of units [c0, c1) of tile (ti, tj) into this wave's accumulator.
__device__ void run_units(v16f acc[4], const HPlan& p, int ti, int tj, int c0, int c1, int wave, int lane) {
  const bool diag = ti == tj;
  const int i0 = ti * kTile, j0 = tj * kTile;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.0f;
  Operands cur, nxt;
  load_unit(cur, p, c0, i0, j0, diag, wave, lane);
  for (int c = c0; c < c1; ++c) {
    // the next unit's loads are in flight during this unit's MFMAs (the last
    // iteration reloads its own unit, which stays in bounds)
    load_unit(nxt, p, c + 1 < c1 ? c + 1 : c, i0, j0, diag, wave, lane);
    mfma_unit(acc, cur, diag);
    cur = nxt;
  }
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
// lower, so both halves come from the same values.
__device__ void add_tile(const HPlan& p, const float* S, int ti, int tj) {
  const bool diag = ti == tj;
  const int i0 = ti * kTile, j0 = tj * kTile, K = p.K;
  const int t = threadIdx.x;
  {
    const int b = t & 63, j = j0 + b;
    for (int k = 0; k < 16; ++k) {
      const int a = (t >> 6) + 4 * k, i = i0 + a;
      if (i < K && j < K && (!diag || a <= b)) p.H[(size_t)i * K + j] += S[a * kLds + b];
    }
  }
  {
    const int a = t & 63, i = i0 + a;
    for (int k = 0; k < 16; ++k) {
      const int b = (t >> 6) + 4 * k, j = j0 + b;
      if (i < K && j < K && (!diag || a < b)) p.H[(size_t)j * K + i] += S[a * kLds + b];
    }
  }
}

__global__ __launch_bounds__(kThreads) void hessian_tiles_kernel(HPlan p) {
  extern __shared__ float lds[];  // 4 * kTileLds floats
  const int g = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v16f acc[4];
  // whole tiles, round robin
  for (int k = 0; k < p.q; ++k) {
    int ti, tj;
    tile_of(g + kGroups * k, &ti, &tj);
    run_units(acc, p, ti, tj, 0, p.nc, wave, lane);
    reduce_waves(acc, lds, wave, lane);
    add_tile(p, lds, ti, tj);
  }
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
    int ti, tj;
    tile_of(p.q * kGroups + t, &ti, &tj);
    run_units(acc, p, ti, tj, c0, c1, wave, lane);
    reduce_waves(acc, lds, wave, lane);
    if (c0 == 0 && c1 == p.nc) {
      add_tile(p, lds, ti, tj);
    } else {  // a piece: slot 0 for this work group's first range, 1 for its last
      float* dst = p.part + ((size_t)g * 2 + (first ? 0 : 1)) * (kTile * kTile);
      for (int k = 0; k < 16; ++k) {
        const int e = threadIdx.x + kThreads * k;
        dst[e] = lds[(e >> 6) * kLds + (e & 63)];
      }
    }
    first = false;
    v = (long long)t * p.nc + c1;
  }
}

// One work group per leftover tile: adds the pieces of a tile that was split
// across work groups, in work-group order, then adds the sum to H.
__global__ __launch_bounds__(kThreads) void hessian_pieces_kernel(HPlan p) {
  __shared__ float S[kTileLds];
  const int t = blockIdx.x;
  const long long v0 = (long long)t * p.nc, v1 = v0 + p.nc;
  const int gf = unit_owner(v0, p.wr), gl = unit_owner(v1 - 1, p.wr);
  if (gf == gl) return;  // covered by one work group, added there
  float s[16];
  bool have = false;
  for (int g = gf; g <= gl; ++g) {
    const long long st = unit_start(g, p.wr);
    if (st == unit_start(g + 1, p.wr)) continue;  // empty range
    const float* src = p.part + ((size_t)g * 2 + (st >= v0 ? 0 : 1)) * (kTile * kTile);
    for (int k = 0; k < 16; ++k) {
      const float v = src[threadIdx.x + kThreads * k];
      s[k] = have ? s[k] + v : v;
    }
    have = true;
  }
  for (int k = 0; k < 16; ++k) {
    const int e = threadIdx.x + kThreads * k;
    S[(e >> 6) * kLds + (e & 63)] = s[k];
  }
  __syncthreads();
  int ti, tj;
  tile_of(p.q * kGroups + t, &ti, &tj);
  add_tile(p, S, ti, tj);
}

HPlan make_plan(const float* x, int rows, int K, float* H, float* part) {
  HPlan p{};
  p.x = x;
  p.H = H;
  p.part = part;
  p.rows = rows;
  p.K = K;
  const int nt = (K + kTile - 1) / kTile;
  const int ntiles = nt * (nt + 1) / 2;
  p.nc = (rows + kUnitRows - 1) / kUnitRows;
  p.q = ntiles / kGroups;
  p.r = ntiles % kGroups;
  p.wr = (long long)p.r * p.nc;
  return p;
}

}  // namespace

size_t hessian_workspace_bytes(int K) {
  const int nt = (K + kTile - 1) / kTile;
  const int ntiles = nt * (nt + 1) / 2;
  return ntiles % kGroups ? (size_t)kGroups * 2 * kTile * kTile * sizeof(float) : 0;
}

hipError_t launch_hessian(const float* x, int rows, int K, float* H, float* part, hipStream_t s) {
  const HPlan p = make_plan(x, rows, K, H, part);
  const size_t lds = (size_t)4 * kTileLds * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(hessian_tiles_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hessian_tiles_kernel, dim3(kGroups), dim3(kThreads), lds, s, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.r == 0) return e;
  hipLaunchKernelGGL(hessian_pieces_kernel, dim3(p.r), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace loopq
