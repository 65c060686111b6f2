// Device helpers shared by the two GEMM kernels (INT8 and fp6 operands):
// argument block, buffer resources, the XCD-aware work-group -> tile map and
// the fp32 output store.  Both kernels compute 128x128 output tiles with
// four waves of 64x64 (2x2 tiles of 32x32, transposed: MFMA operand A holds
// weight columns, operand B activation rows).
#pragma once

#include "loopq_internal.h"

namespace loopq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int kGemmMaxSets = 64;

struct GemmArgs {
  const void* a;     // tiled activation codes (int8 or fp6 layout)
  const float* sa;   // group-major activation steps [Ga][ld_sa]
  int ld_sa;
  int M, K, N;
  const void* w;     // packed nibbles (int8 kernel) or expanded fp6 codes
  const __half* sw;  // packed weight steps [Npad/32][Gw][32]
  int gshift;        // log2(group_w / 32)
  float* y;          // [M][N]
  int32_t* dots;     // [M][N][Ga] (mode 1)
  // grouped form: with rows_per_set > 0 (a multiple of 64), rows
  // [s * rows_per_set, (s + 1) * rows_per_set) take weights w_set[s], sw_set[s]
  int rows_per_set;
  const void* w_set[kGemmMaxSets];
  const __half* sw_set[kGemmMaxSets];
};

// The weights of the wave whose 64 rows start at m_base (wave-uniform).
__device__ __forceinline__ void tile_weights(const GemmArgs& g, int m_base, const void** w, const __half** sw) {
  if (g.rows_per_set > 0) {
    const int set = m_base / g.rows_per_set;
    *w = g.w_set[set];
    *sw = g.sw_set[set];
  } else {
    *w = g.w;
    *sw = g.sw;
  }
}

// raw buffer resource over [p, p + bytes): stride 0, gfx9 data format word;
// loads at or past `bytes` return 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Work-group -> 128x128 output tile.  Consecutive work-groups land on the 8
// XCDs in turn and each XCD has its own L2, so every XCD first gets one
// contiguous range of tile numbers; tiles are then walked in groups of 8 row
// panels, down the rows of a group before moving one column panel on, so an
// XCD's range is a compact block of row and column panels whose operands its
// L2 reads about once.  Everything here is wave-uniform.
__device__ __forceinline__ void map_tile(const GemmArgs& g, int wave, int* m_base, int* n_base) {
  const int Mp = (g.M + 127) >> 7;
  const int Np = (g.N + 127) >> 7;
  const int total = Mp * Np;
  const int xcd = blockIdx.x & 7;
  const int q = xcd * (total >> 3) + min(xcd, total & 7) + (int)(blockIdx.x >> 3);
  const int grp = q / (8 * Np);
  const int gm = min(Mp - grp * 8, 8);
  const int r = q - grp * 8 * Np;
  *m_base = (grp * 8 + r % gm) * 128 + (wave >> 1) * 64;
  *n_base = (r / gm) * 128 + (wave & 1) * 64;
}

// Split-K form for launches with fewer 128x128 tiles than CUs: 64x128
// tiles, the same XCD-aware walk over 64-row panels; waves 0 and 1 take the
// first half of the group pairs of their 64x64 quadrant, waves 2 and 3 (kh =
// 1) the second half of the same quadrants.
__device__ __forceinline__ void map_tile_split(const GemmArgs& g, int wave, int* m_base, int* n_base, int* kh) {
  const int Mp = (g.M + 63) >> 6;
  const int Np = (g.N + 127) >> 7;
  const int total = Mp * Np;
  const int xcd = blockIdx.x & 7;
  const int q = xcd * (total >> 3) + min(xcd, total & 7) + (int)(blockIdx.x >> 3);
  const int grp = q / (8 * Np);
  const int gm = min(Mp - grp * 8, 8);
  const int r = q - grp * 8 * Np;
  *m_base = (grp * 8 + r % gm) * 64;
  *n_base = (r / gm) * 128 + (wave & 1) * 64;
  *kh = wave >> 1;
}

// Four-way split-K form: one 64x64 quadrant per work-group, wave w takes the
// w-th quarter of the K pairs (kq = w).  Tile numbering and XCD placement as
// map_tile_split, over 64x64 tiles.
__device__ __forceinline__ void map_tile_split4(const GemmArgs& g, int wave, int* m_base, int* n_base, int* kq) {
  const int Mp = (g.M + 63) >> 6;
  const int Np = (g.N + 63) >> 6;
  const int total = Mp * Np;
  const int xcd = blockIdx.x & 7;
  const int q = xcd * (total >> 3) + min(xcd, total & 7) + (int)(blockIdx.x >> 3);
  const int grp = q / (8 * Np);
  const int gm = min(Mp - grp * 8, 8);
  const int r = q - grp * 8 * Np;
  *m_base = (grp * 8 + r % gm) * 64;
  *n_base = (r / gm) * 64;
  *kq = wave;
}

// Result element e of lane l of tile (t, u) is row m = m_base + 32 t + l % 32
// and column n = n_base + 32 u + 8 (e / 4) + 4 (l / 32) + e % 4.
__device__ __forceinline__ void store_y(const GemmArgs& g, const float (&acc)[2][2][16], int m_base,
                                        int n_base, int h, int c) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = m_base + 32 * t + c;
    if (row >= g.M) continue;
    float* yr = g.y + (int64_t)row * g.N;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n_base + 32 * u + 8 * q + 4 * h;
        if (col + 3 < g.N && (g.N & 3) == 0) {
          *reinterpret_cast<float4*>(yr + col) =
              float4{acc[t][u][4 * q], acc[t][u][4 * q + 1], acc[t][u][4 * q + 2], acc[t][u][4 * q + 3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col + r < g.N) yr[col + r] = acc[t][u][4 * q + r];
        }
      }
  }
}

}  // namespace loopq
