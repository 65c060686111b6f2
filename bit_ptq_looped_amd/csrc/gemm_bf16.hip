// Integer-exact GEMM on bf16 MFMA operands, with per-group rescale (gfx950).
//
//   y[m][n] = sum_j s_a[m][j] * s_w[n][32j / group_w] * d[m][n][j],
//   d[m][n][j] = sum_{k in group j} q_a[m][k] * q_w[n][k]
//
// Same arithmetic as the INT8 kernel (gemm_w4.hip): the integer form of the
// simulated quantize-dequantize product of Eq.(4) codes ("paper_specification
// .yaml", lq1_quantization).  Here the codes enter V_MFMA_F32_32X32X16_BF16
// as bf16, which holds every code exactly (|q| <= 127); products are at most
// 889 and a 32-element group sum at most 28,448 < 2^24, so the fp32 result of
// the two MFMAs that cover one group IS the exact group dot d -- no integer to
// float conversion is left for the vector ALU.  The rescale then costs two
// VALU operations per (m, n, group): the step product (v_fma_mix with the
// fp16 weight step) and the FMA into the fp32 accumulator; the step products
// themselves are outer products s_w (x) s_a and are formed on the matrix
// cores too (fp32 MFMA, K = 1), leaving one VALU FMA per (m, n, group).
//
// The packed INT4 weights are expanded once per call into bf16 operands in a
// workspace buffer (launch_expand_weights_bf16), so the inner loop does no
// nibble unpacking; activation codes arrive from the quantizer already in
// bf16.  Tiling, prefetch and the transposed result tiles are those of the
// INT8 kernel.
#include "loopq_internal.h"

namespace loopq {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

struct GemmBfArgs {
  const uint16_t* a;   // bf16 tiled activation codes
  const float* sa;     // group-major steps [Ga][ld_sa]
  int ld_sa;
  int M, K, N;
  const uint16_t* w;   // bf16 tiled expanded weights
  const __half* sw;    // packed steps [Npad/32][Gw][32] (slot order)
  int gshift;
  float* y;
  int32_t* dots;
};

struct StageBf {
  uint4 w[2][2];   // 16 bf16 weights per column tile (two MFMA operands)
  uint4 x[2][2];   // 16 bf16 codes per row tile
  float sa[2];     // activation steps of row l % 32 of row tiles h and 1 - h
  uint32_t sw;     // raw fp16 weight step of column l % 32 of column tile h
};

__device__ __forceinline__ v8bf as_v8bf(uint4 v) { return __builtin_bit_cast(v8bf, v); }

template <int MODE>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmBfArgs g) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int c = lane & 31;
  const int m_base = blockIdx.y * 128 + (wave >> 1) * 64;
  const int n_base = blockIdx.x * 128 + (wave & 1) * 64;
  if (m_base >= g.M || n_base >= g.N) return;
  const int Ga = g.K >> 5;
  const int Gw = ((g.K >> 5) + (1 << g.gshift) - 1) >> g.gshift;
  const int mlast = ((g.M + 31) >> 5) - 1;
  const int nlast = ((g.N + 31) >> 5) - 1;

  const uint4* x_ptr[2];
  const uint4* w_ptr[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mb = min((m_base >> 5) + t, mlast);  // edge tiles re-read a valid block
    const int nb = min((n_base >> 5) + t, nlast);
    x_ptr[t] = reinterpret_cast<const uint4*>(g.a + ((int64_t)mb * Ga) * 1024) + lane * 2;
    w_ptr[t] = reinterpret_cast<const uint4*>(g.w + ((int64_t)nb * Ga) * 1024) + lane * 2;
  }
  // steps feeding the outer-product MFMAs: lane l supplies the weight step of
  // column l % 32 of column tile h, and the activation steps of row l % 32 of
  // row tiles h and 1 - h
  const float* sa_ptr0 = g.sa + min((m_base >> 5) + h, mlast) * 32 + c;
  const float* sa_ptr1 = g.sa + min((m_base >> 5) + 1 - h, mlast) * 32 + c;
  const unsigned short* sw_ptr = reinterpret_cast<const unsigned short*>(g.sw) +
                                 (int64_t)min((n_base >> 5) + h, nlast) * Gw * 32 + step_slot(c);

  auto load = [&](int j, StageBf& s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint4* xp = x_ptr[t] + (int64_t)j * 128;  // 2048-byte blocks
      const uint4* wp = w_ptr[t] + (int64_t)j * 128;
      s.x[t][0] = xp[0];
      s.x[t][1] = xp[1];
      s.w[t][0] = wp[0];
      s.w[t][1] = wp[1];
    }
    if (MODE == 0) {
      s.sa[0] = sa_ptr0[(int64_t)j * g.ld_sa];
      s.sa[1] = sa_ptr1[(int64_t)j * g.ld_sa];
      s.sw = sw_ptr[(int64_t)(j >> g.gshift) * 32];
    }
  };

  float acc[2][2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][u][e] = 0.0f;

  auto mfma2 = [&](const StageBf& s, int t, int u) {
    const v16f zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    v16f d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(s.w[u][0]), as_v8bf(s.x[t][0]), zero,
                                                     0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(s.w[u][1]), as_v8bf(s.x[t][1]), d, 0, 0, 0);
  };
  // fold one 32x32 result tile with its step-product tile (16 VALU FMAs)
  auto fold = [&](const v16f& d, const v32f& cf, int half, int t, int u, int j) {
    if (MODE == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][u][e] = __builtin_fmaf(d[e], cf[16 * half + e], acc[t][u][e]);
    } else {
      const int row = m_base + 32 * t + c;
      if (row < g.M) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int col = n_base + 32 * u + 8 * (e >> 2) + 4 * h + (e & 3);
          if (col < g.N) g.dots[((int64_t)row * g.N + col) * Ga + j] = (int32_t)d[e];
        }
      }
    }
  };
  // The step products s_w[n] * s_a[m] of the four result tiles are outer
  // products: V_MFMA_F32_32X32X1_2B_F32 forms two 32x32 blocks at once, block b
  // from lanes 32b..32b+31, landing in the same element layout as the GEMM
  // tiles.  cA holds tiles (t0,u0) | (t1,u1), cB holds (t1,u0) | (t0,u1).
  // The MFMA of the next tile is issued before the current one is folded.
  auto compute = [&](const StageBf& s, int j) {
    v32f cA = {}, cB = {};
    if (MODE == 0) {
      const v32f z = {};
      const float swf = __half2float(__ushort_as_half((unsigned short)s.sw));
      cA = __builtin_amdgcn_mfma_f32_32x32x1f32(swf, s.sa[0], z, 0, 0, 0);
      cB = __builtin_amdgcn_mfma_f32_32x32x1f32(swf, s.sa[1], z, 0, 0, 0);
    }
    const v16f d00 = mfma2(s, 0, 0);
    const v16f d01 = mfma2(s, 0, 1);
    fold(d00, cA, 0, 0, 0, j);
    const v16f d10 = mfma2(s, 1, 0);
    fold(d01, cB, 1, 0, 1, j);
    const v16f d11 = mfma2(s, 1, 1);
    fold(d10, cB, 0, 1, 0, j);
    fold(d11, cA, 1, 1, 1, j);
  };

  StageBf s0, s1;
  load(0, s0);
  load(min(1, Ga - 1), s1);
  int j = 0;
  for (; j + 1 < Ga; j += 2) {
    compute(s0, j);
    __builtin_amdgcn_sched_barrier(0);
    load(min(j + 2, Ga - 1), s0);
    __builtin_amdgcn_sched_barrier(0);
    compute(s1, j + 1);
    __builtin_amdgcn_sched_barrier(0);
    load(min(j + 3, Ga - 1), s1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (j < Ga) compute(s0, j);

  if (MODE == 0) {
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
            *reinterpret_cast<float4*>(yr + col) = float4{acc[t][u][4 * q], acc[t][u][4 * q + 1],
                                                          acc[t][u][4 * q + 2], acc[t][u][4 * q + 3]};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (col + r < g.N) yr[col + r] = acc[t][u][4 * q + r];
          }
        }
    }
  }
}

// One thread per (column block, K-chunk, lane): 8 packed bytes (16 biased
// nibbles, K order i = 0..15) -> 16 bf16 at the same lane position of the
// bf16 tiled layout.
__global__ __launch_bounds__(256) void expand_bf16_kernel(const uint8_t* __restrict__ codes,
                                                          int64_t nthreads,
                                                          uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nthreads) return;
  const uint2 p = reinterpret_cast<const uint2*>(codes)[idx];
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t word0 = (i < 8) ? p.x : p.y;
    const int i0 = i & 7, i1 = (i + 1) & 7;
    const uint32_t n0 = (word0 >> (8 * (i0 & 3) + 4 * (i0 >> 2))) & 15u;
    const uint32_t n1 = (word0 >> (8 * (i1 & 3) + 4 * (i1 >> 2))) & 15u;
    const uint32_t b0 = __float_as_uint((float)((int)n0 - 8)) >> 16;
    const uint32_t b1 = __float_as_uint((float)((int)n1 - 8)) >> 16;
    o[i >> 1] = b0 | (b1 << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>(out) + idx * 2;
  dst[0] = uint4{o[0], o[1], o[2], o[3]};
  dst[1] = uint4{o[4], o[5], o[6], o[7]};
}

}  // namespace

hipError_t launch_expand_weights_bf16(const uint8_t* w_codes, int K, int N, uint16_t* out,
                                      hipStream_t s) {
  const int64_t nthreads = padded_cols(N) / 32 * (K / 32) * 64;
  hipLaunchKernelGGL(expand_bf16_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, s,
                     w_codes, nthreads, out);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t* a_tiled, const float* a_scales_gm, int ld_sa, int M,
                            int K, int N, const uint16_t* w_bf16, const __half* w_scales, int gw,
                            float* y, int32_t* dots, int mode, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  GemmBfArgs g;
  g.a = a_tiled;
  g.sa = a_scales_gm;
  g.ld_sa = ld_sa;
  g.M = M;
  g.K = K;
  g.N = N;
  g.w = w_bf16;
  g.sw = w_scales;
  g.gshift = gw == 128 ? 2 : 0;
  g.y = y;
  g.dots = dots;
  dim3 grid((N + 127) / 128, (M + 127) / 128);
  if (mode == 0)
    hipLaunchKernelGGL(gemm_bf16_kernel<0>, grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<1>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace loopq
