// Integer GEMM with per-group rescale for W4A4 / W4A8 (gfx950).
//
//   y[m][n] = sum_j s_a[m][j] * s_w[n][32j / group_w] * d[m][n][j],
//   d[m][n][j] = sum_{k in group j} q_a[m][k] * q_w[n][k]   (exact int32)
//
// Method: the integer form of the simulated quantize-dequantize product of
// Eq.(4)-quantized operands ("paper_specification.yaml", lq1_quantization:
// group-wise W4 with A4 or A8, group size 32; the README of the LoopQ
// reproduction, "Protocol": quantization simulated as quantize-dequantize).
//
// One V_MFMA_I32_32X32X32_I8 covers exactly one 32-wide K-group of a 32x32
// output tile, so its int32 result is the group dot d for 32x32 (m, n)
// pairs; the accumulator is not carried across groups.  The result is
// converted to fp32 and folded into an fp32 accumulator with the product of
// the two steps.  INT4 weight nibbles are unpacked to int8 in registers.
//
// Tiling: 256 threads = 4 waves in a 2x2 arrangement, 128x128 outputs per
// work-group, 64x64 (2x2 MFMA tiles) per wave.  Operands stream from global
// memory in the tiled layouts of loopq_internal.h (each wave load is one
// contiguous 1 KB / 512 B block); the next group is prefetched while the
// current one is multiplied and folded.
#include "loopq_internal.h"

namespace loopq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct GemmArgs {
  const int8_t* a;   // tiled codes
  const float* sa;   // group-major steps [Ga][ld_sa]
  int ld_sa;
  int M, K, N;
  const uint8_t* w;  // packed nibbles
  const __half* sw;  // packed steps [Npad/32][Gw][32]
  int gshift;        // log2(group_w / 32)
  float* y;          // [M][N]
  int32_t* dots;     // [M][N][Ga] (mode 1)
};

// 8 biased nibbles (q + 8) per dword -> 16 int8 codes, in K order
__device__ __forceinline__ v4i unpack_w(uint2 p) {
  v4i r;
  r[0] = (int)(((p.x & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[1] = (int)((((p.x >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[2] = (int)(((p.y & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[3] = (int)((((p.y >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  return r;
}

struct Stage {
  v4i a[2];
  uint2 b[2];
  float4 sa[2][4];
  float sw[2];
};

template <int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;    // K-half of the operands; row group of the result
  const int c = lane & 31;    // column of the result
  const int m_base = blockIdx.y * 128 + (wave >> 1) * 64;
  const int n_base = blockIdx.x * 128 + (wave & 1) * 64;
  const int Ga = g.K >> 5;
  const int Gw = ((g.K >> 5) + (1 << g.gshift) - 1) >> g.gshift;
  bool mv[2], nv[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    mv[t] = (m_base + 32 * t) < g.M;
    nv[t] = (n_base + 32 * t) < g.N;
  }
  if (!mv[0] || !nv[0]) return;  // the second tile is only valid if the first is

  const int8_t* a_ptr[2];
  const uint8_t* w_ptr[2];
  const __half* sw_ptr[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mb = (m_base >> 5) + t;
    const int nb = (n_base >> 5) + t;
    a_ptr[t] = g.a + (int64_t)mb * Ga * 1024 + lane * 16;
    w_ptr[t] = g.w + (int64_t)nb * Ga * kBlockBytes + lane * 8;
    sw_ptr[t] = g.sw + (int64_t)nb * Gw * 32 + c;
  }

  auto load = [&](int j, Stage& s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (mv[t]) s.a[t] = *reinterpret_cast<const v4i*>(a_ptr[t] + (int64_t)j * 1024);
      else s.a[t] = v4i{0, 0, 0, 0};
      if (nv[t]) s.b[t] = *reinterpret_cast<const uint2*>(w_ptr[t] + (int64_t)j * kBlockBytes);
      else s.b[t] = uint2{0x88888888u, 0x88888888u};
      if (MODE == 0) {
        const float* sap = g.sa + (int64_t)j * g.ld_sa + m_base + 32 * t + 4 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          s.sa[t][q] = mv[t] ? *reinterpret_cast<const float4*>(sap + 8 * q) : float4{0, 0, 0, 0};
        s.sw[t] = nv[t] ? __half2float(sw_ptr[t][(int64_t)(j >> g.gshift) * 32]) : 0.0f;
      }
    }
  };

  float acc[2][2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][u][e] = 0.0f;

  Stage cur, nxt;
  load(0, cur);
  for (int j = 0; j < Ga; ++j) {
    if (j + 1 < Ga) load(j + 1, nxt);
    const v4i b0 = unpack_w(cur.b[0]);
    const v4i b1 = unpack_w(cur.b[1]);
    v16i d[2][2];
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    d[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[0], b0, zero, 0, 0, 0);
    d[0][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[0], b1, zero, 0, 0, 0);
    d[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[1], b0, zero, 0, 0, 0);
    d[1][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[1], b1, zero, 0, 0, 0);
    if (MODE == 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 sa4 = cur.sa[t][q];
            const float sv[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int e = 4 * q + r;
              const float coef = sv[r] * cur.sw[u];
              acc[t][u][e] = __builtin_fmaf((float)d[t][u][e], coef, acc[t][u][e]);
            }
          }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (!mv[t] || !nv[u]) continue;
          const int col = n_base + 32 * u + c;
          if (col >= g.N) continue;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = m_base + 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
            if (row < g.M) g.dots[((int64_t)row * g.N + col) * Ga + j] = d[t][u][e];
          }
        }
    }
    if (j + 1 < Ga) cur = nxt;
  }

  if (MODE == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int col = n_base + 32 * u + c;
        if (!mv[t] || col >= g.N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m_base + 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
          if (row < g.M) g.y[(int64_t)row * g.N + col] = acc[t][u][e];
        }
      }
  }
}

__global__ __launch_bounds__(256) void tile_codes_kernel(const int8_t* __restrict__ canon,
                                                         const float* __restrict__ canon_scales,
                                                         int M, int K, int8_t* __restrict__ tiled,
                                                         float* __restrict__ gm_scales, int ld) {
  const int Ga = K >> 5;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 4-byte run
  const int64_t runs = (int64_t)M * (K >> 2);
  if (idx >= runs) return;
  const int row = (int)(idx / (K >> 2));
  const int k0 = (int)(idx - (int64_t)row * (K >> 2)) * 4;
  const uint32_t v = *reinterpret_cast<const uint32_t*>(canon + (int64_t)row * K + k0);
  const int j = k0 >> 5, kk = k0 & 31;
  *reinterpret_cast<uint32_t*>(tiled + ((int64_t)(row >> 5) * Ga + j) * 1024 + (kk >> 4) * 512 +
                               (row & 31) * 16 + (kk & 15)) = v;
  if (kk == 0 && gm_scales) gm_scales[(int64_t)j * ld + row] = canon_scales[(int64_t)row * Ga + j];
}

}  // namespace

hipError_t launch_gemm(const int8_t* a_tiled, const float* a_scales_gm, int ld_sa, int M, int K,
                       int N, const uint8_t* w_codes, const __half* w_scales, int gw, float* y,
                       int32_t* dots, int mode, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  GemmArgs g;
  g.a = a_tiled;
  g.sa = a_scales_gm;
  g.ld_sa = ld_sa;
  g.M = M;
  g.K = K;
  g.N = N;
  g.w = w_codes;
  g.sw = w_scales;
  g.gshift = gw == 128 ? 2 : 0;
  g.y = y;
  g.dots = dots;
  dim3 grid((N + 127) / 128, (M + 127) / 128);
  if (mode == 0)
    hipLaunchKernelGGL(gemm_kernel<0>, grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_kernel<1>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_tile_codes(const int8_t* canon_codes, const float* canon_scales, int M, int K,
                             int8_t* tiled_codes, float* gm_scales, int ld, hipStream_t s) {
  const int64_t runs = (int64_t)M * (K / 4);
  if (runs == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_codes_kernel, dim3((unsigned)((runs + 255) / 256)), dim3(256), 0, s,
                     canon_codes, canon_scales, M, K, tiled_codes, gm_scales, ld);
  return hipGetLastError();
}

}  // namespace loopq
