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
// pairs; the accumulator is not carried across groups.  The MFMA starts from
// the bit pattern of 1.5 * 2^23, so its int32 result reads as the fp32 number
// 1.5 * 2^23 + d and one exact subtraction gives d as a float; it is folded
// into an fp32 accumulator with the product of the two steps.  INT4 weight
// nibbles are unpacked to int8 in registers.  This kernel serves W4A8 (and
// W4A4 on request); gemm_f6.hip is the W4A4 kernel.
//
// Tiling: 256 threads = 4 waves in a 2x2 arrangement, 128x128 outputs per
// work-group, 64x64 (2x2 MFMA tiles) per wave; the two split-K forms of the
// fp6 kernel (64x128 tiles over half of K per wave, 64x64 over a quarter)
// where they spread a launch's waves over the SIMDs better (gemm_form).  Operands stream from global
// memory in the tiled layouts of loopq_internal.h (each wave load is one
// contiguous 1 KB / 512 B block); the loop is unrolled twice so the next
// group's loads are in flight while the current one is multiplied and folded,
// with no register copies between stages.
#include "gemm_tile.h"

namespace loopq {
namespace {

// 8 biased nibbles (q + 8) per dword -> 16 int8 codes, in K order
__device__ __forceinline__ v4i unpack_w(uint2 p) {
  v4i r;
  r[0] = (int)(((p.x & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[1] = (int)((((p.x >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[2] = (int)(((p.y & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[3] = (int)((((p.y >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  return r;
}

// Operands of one K-group, as loaded (raw: nothing is converted until used,
// so a prefetch never forces a wait).
struct Stage {
  uint2 w[2];        // packed nibbles: MFMA operand A, the wave's two 32-column tiles
  v4i x[2];          // activation codes: MFMA operand B, the wave's two 32-row tiles
  float sa[2];       // activation steps of row l % 32 of row tiles h and 1 - h
  uint32_t sw;       // raw fp16 weight step of column l % 32 of column tile h
};

// SPLIT (rescale mode only): 1, the two-way split-K form (64x128 tiles, waves
// 0-1 over the first half of the groups of their 64x64 quadrants, waves 2-3
// over the second half); 2, the four-way form (one 64x64 quadrant per
// work-group, wave w over the w-th quarter of the groups).  The partial sums
// are added through LDS in a fixed order (the first wave of a quadrant adds
// the others' and stores), as in the fp6 kernel; every wave of a split form
// reaches the barrier, so none returns early.
template <int MODE, int SPLIT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g) {
  __shared__ float red[SPLIT == 2 ? 3 * 64 * 64 : SPLIT ? 2 * 64 * 64 : 1];
  const int lane = threadIdx.x & 63;
  // the wave index is uniform; say so, so that tile bases live in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int c = lane & 31;
  int m_base, n_base, kh = 0;
  if (SPLIT == 2)
    map_tile_split4(g, wave, &m_base, &n_base, &kh);
  else if (SPLIT)
    map_tile_split(g, wave, &m_base, &n_base, &kh);
  else
    map_tile(g, wave, &m_base, &n_base);
  const bool active = m_base < g.M && n_base < g.N;
  if (!SPLIT && !active) return;
  const int Ga = g.K >> 5;
  const int Gw = ((g.K >> 5) + (1 << g.gshift) - 1) >> g.gshift;
  const int mlast = ((g.M + 31) >> 5) - 1;
  const int nlast = ((g.N + 31) >> 5) - 1;

  // Every operand load is a buffer load: a wave-uniform resource (tile start,
  // scalar registers), a per-lane byte offset fixed along K, and the group
  // offset as the scalar offset, so the K loop does no vector address
  // arithmetic.  Tiles past the matrix edge re-read the last valid block
  // (always in bounds); their results are dropped at the store.
  const void* wp;
  const __half* swp;
  tile_weights(g, active ? m_base : 0, &wp, &swp);  // the grouped form's weight set of these rows
  __amdgpu_buffer_rsrc_t x_rs[2], w_rs[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mb = min((m_base >> 5) + t, mlast);
    const int nb = min((n_base >> 5) + t, nlast);
    x_rs[t] = make_rsrc(reinterpret_cast<const char*>(g.a) + (int64_t)mb * Ga * 1024, (uint32_t)Ga * 1024u);
    w_rs[t] = make_rsrc(reinterpret_cast<const uint8_t*>(wp) + (int64_t)nb * Ga * kBlockBytes,
                        (uint32_t)Ga * kBlockBytes);
  }
  const int x_off = lane * 16;
  const int w_off = lane * 8;
  // steps feeding the outer-product MFMAs: lane l supplies the weight step of
  // column l % 32 of column tile h, and the activation steps of row l % 32 of
  // row tiles h and 1 - h
  const __amdgpu_buffer_rsrc_t sa_rs = make_rsrc(g.sa, (uint32_t)g.ld_sa * (uint32_t)Ga * 4u);
  const __amdgpu_buffer_rsrc_t sw_rs = make_rsrc(swp, (uint32_t)(nlast + 1) * (uint32_t)Gw * 64u);
  const int sa_off0 = (min((m_base >> 5) + h, mlast) * 32 + c) * 4;
  const int sa_off1 = (min((m_base >> 5) + 1 - h, mlast) * 32 + c) * 4;
  const int sw_off = (min((n_base >> 5) + h, nlast) * Gw * 32 + step_slot(c)) * 2;

  auto load = [&](int j, Stage& s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s.x[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(x_rs[t], x_off, j * 1024, 0));
      s.w[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(w_rs[t], w_off, j * kBlockBytes, 0));
    }
    if (MODE == 0) {
      const int so = j * g.ld_sa * 4;
      s.sa[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sa_rs, sa_off0, so, 0));
      s.sa[1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sa_rs, sa_off1, so, 0));
      s.sw = __builtin_amdgcn_raw_buffer_load_b16(sw_rs, sw_off, (j >> g.gshift) * 64, 0);
    }
  };

  float acc[2][2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][u][e] = 0.0f;

  // In the rescale the integer MFMA starts from the bit pattern of
  // kMagic = 1.5 * 2^23 instead of 0: for |d| < 2^22 the int32 result
  // kMagicBits + d is the fp32 number kMagic + d exactly, so one exact fp32
  // subtraction recovers d as a float (cheaper than an int-to-float convert).
  // The dots-only form starts from 0.
  constexpr int kMagicBits = 0x4B400000;
  constexpr float kMagic = 12582912.0f;
  const int cinit = MODE == 0 ? kMagicBits : 0;
  const v16i c0 = {cinit, cinit, cinit, cinit, cinit, cinit, cinit, cinit,
                   cinit, cinit, cinit, cinit, cinit, cinit, cinit, cinit};
  auto mfma = [&](const Stage& s, const v4i& wu, int t) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(wu, s.x[t], c0, 0, 0, 0);
  };
  // fold one 32x32 result tile: recover the group dots as floats, FMA with
  // the step-product tile
  auto fold = [&](const v16i& d, const v32f& cf, int half, int t, int u, int j) {
    if (MODE == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        acc[t][u][e] = __builtin_fmaf(__int_as_float(d[e]) - kMagic, cf[16 * half + e], acc[t][u][e]);
    } else {
      const int row = m_base + 32 * t + c;
      if (row < g.M) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int col = n_base + 32 * u + 8 * (e >> 2) + 4 * h + (e & 3);
          if (col < g.N) g.dots[((int64_t)row * g.N + col) * Ga + j] = d[e];
        }
      }
    }
  };
  // Step products s_w[n] * s_a[m] of the four result tiles come from two
  // V_MFMA_F32_32X32X1_2B_F32 outer products (block b from lanes 32b..32b+31,
  // same element layout as the GEMM tiles): cA = (t0,u0) | (t1,u1),
  // cB = (t1,u0) | (t0,u1).  The MFMA of the next tile is issued before the
  // current tile is folded.
  auto compute = [&](const Stage& s, int j) {
    v32f cA = {}, cB = {};
    if (MODE == 0) {
      const v32f z = {};
      const float swf = __half2float(__ushort_as_half((unsigned short)s.sw));
      cA = __builtin_amdgcn_mfma_f32_32x32x1f32(swf, s.sa[0], z, 0, 0, 0);
      cB = __builtin_amdgcn_mfma_f32_32x32x1f32(swf, s.sa[1], z, 0, 0, 0);
    }
    const v4i w0 = unpack_w(s.w[0]);
    const v4i w1 = unpack_w(s.w[1]);
    const v16i d00 = mfma(s, w0, 0);
    const v16i d01 = mfma(s, w1, 0);
    fold(d00, cA, 0, 0, 0, j);
    const v16i d10 = mfma(s, w0, 1);
    fold(d01, cB, 1, 0, 1, j);
    const v16i d11 = mfma(s, w1, 1);
    fold(d10, cB, 0, 1, 0, j);
    fold(d11, cA, 1, 1, 1, j);
  };

  // this wave's groups [j0, j1).  Loads past the last group re-read it (in
  // bounds, unused), so the loop body is one basic block the barriers can
  // order.
  const int half = (Ga + 1) >> 1;
  const int quarter = (Ga + 3) >> 2;
  const int j0 = SPLIT == 2 ? min(Ga, kh * quarter) : SPLIT && kh ? half : 0;
  const int j1 = SPLIT == 2 ? min(Ga, j0 + quarter) : SPLIT && !kh ? half : Ga;
  if (active && j0 < j1) {
    Stage s0, s1;
    load(j0, s0);
    load(min(j0 + 1, j1 - 1), s1);
    int j = j0;
    for (; j + 1 < j1; j += 2) {
      compute(s0, j);
      __builtin_amdgcn_sched_barrier(0);
      load(min(j + 2, j1 - 1), s0);
      __builtin_amdgcn_sched_barrier(0);
      compute(s1, j + 1);
      __builtin_amdgcn_sched_barrier(0);
      load(min(j + 3, j1 - 1), s1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j < j1) compute(s0, j);
  }

  if (SPLIT == 2) {
    if (kh > 0 && active) {
      float* r = red + (kh - 1) * 64 * 64;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 16; ++e) r[((t * 2 + u) * 16 + e) * 64 + lane] = acc[t][u][e];
    }
    __syncthreads();
    if (kh > 0 || !active) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[t][u][e] += red[w * 64 * 64 + ((t * 2 + u) * 16 + e) * 64 + lane];
  } else if (SPLIT) {
    float* r = red + (wave & 1) * 64 * 64;
    if (kh == 1 && active) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 16; ++e) r[((t * 2 + u) * 16 + e) * 64 + lane] = acc[t][u][e];
    }
    __syncthreads();
    if (kh == 1 || !active) return;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][u][e] += r[((t * 2 + u) * 16 + e) * 64 + lane];
  }
  if (MODE == 0) store_y(g, acc, m_base, n_base, h, c);
}

__global__ __launch_bounds__(256) void tile_codes_kernel(const int8_t* __restrict__ canon,
                                                         const float* __restrict__ canon_scales,
                                                         int M, int K, void* __restrict__ tiled,
                                                         int fmt, float* __restrict__ gm_scales,
                                                         int ld) {
  const int Ga = K >> 5;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 4-code run
  const int64_t runs = (int64_t)M * (K >> 2);
  if (idx >= runs) return;
  const int row = (int)(idx / (K >> 2));
  const int k0 = (int)(idx - (int64_t)row * (K >> 2)) * 4;
  const uint32_t v = *reinterpret_cast<const uint32_t*>(canon + (int64_t)row * K + k0);
  const int j = k0 >> 5, kk = k0 & 31;
  if (fmt == kCodesTiledF6) {
    // runs idx .. idx + 3 (an aligned quad of lanes) are the 16 codes of one
    // half-group: runs is a multiple of 8 and K of 32, so quads stay whole
    store_f6_run(tiled, (int)group_pairs(K), row, k0, e2m3_of_codes4(v));
  } else {
    *reinterpret_cast<uint32_t*>(reinterpret_cast<int8_t*>(tiled) + ((int64_t)(row >> 5) * Ga + j) * 1024 +
                                 (kk >> 4) * 512 + (row & 31) * 16 + (kk & 15)) = v;
  }
  if (kk == 0 && gm_scales) gm_scales[(int64_t)j * ld + row] = canon_scales[(int64_t)row * Ga + j];
}

}  // namespace

hipError_t launch_gemm(const int8_t* a_tiled, const float* a_scales_gm, int ld_sa, int M, int K,
                       int N, const uint8_t* w_codes, const __half* w_scales, int gw, float* y,
                       int32_t* dots, int mode, hipStream_t s, const GemmSets* sets) {
  if (M <= 0) return hipSuccess;
  GemmArgs g{};
  if (sets && sets->rows_per_set > 0) {
    if (sets->rows_per_set % 64 || sets->n < 1 || sets->n > kGemmMaxSets ||
        (int64_t)sets->n * sets->rows_per_set != M)
      return hipErrorInvalidValue;
    g.rows_per_set = sets->rows_per_set;
    for (int i = 0; i < sets->n; ++i) {
      g.w_set[i] = sets->w[i];
      g.sw_set[i] = sets->sw[i];
    }
  }
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
  // the tile form as for the fp6 kernel (gemm_form: the busiest SIMD's waves
  // in rounds of two); the dots mode always takes whole tiles
  const int form = mode == 0 ? gemm_form(M, N, K) : 0;
  if (form == 2) {
    dim3 grid((unsigned)((int64_t)((N + 63) / 64) * ((M + 63) / 64)));
    hipLaunchKernelGGL((gemm_kernel<0, 2>), grid, dim3(256), 0, s, g);
  } else if (form == 1) {
    dim3 grid((unsigned)((int64_t)((N + 127) / 128) * ((M + 63) / 64)));
    hipLaunchKernelGGL((gemm_kernel<0, 1>), grid, dim3(256), 0, s, g);
  } else {
    dim3 grid(((N + 127) / 128) * ((M + 127) / 128));
    if (mode == 0)
      hipLaunchKernelGGL((gemm_kernel<0, 0>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_kernel<1, 0>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_tile_codes(const int8_t* canon_codes, const float* canon_scales, int M, int K,
                             void* tiled_codes, int fmt, float* gm_scales, int ld, hipStream_t s) {
  const int64_t runs = (int64_t)M * (K / 4);
  if (runs == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_codes_kernel, dim3((unsigned)((runs + 255) / 256)), dim3(256), 0, s,
                     canon_codes, canon_scales, M, K, tiled_codes, fmt, gm_scales, ld);
  return hipGetLastError();
}

}  // namespace loopq
