// W4A4 GEMM with per-group rescale on fp6 operands (gfx950).
//
//   y[m][n] = sum_j s_a[m][j] * s_w[n][32j / group_w] * d[m][n][j],
//   d[m][n][j] = sum_{k in group j} q_a[m][k] * q_w[n][k]
//
// Method: the integer form of the simulated quantize-dequantize product of
// Eq.(4)-quantized operands ("paper_specification.yaml", lq1_quantization:
// group-wise W4A4, group size 32; the README of the LoopQ reproduction,
// "Protocol": quantization simulated as quantize-dequantize).
//
// W4A4 codes lie in [-7, 7], which the e2m3 fp6 format holds exactly, and
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 multiplies e2m3 operands at the INT8 MFMA
// rate with exact fp32 accumulation of such small integers (|d| <= 1568).  Its
// K of 64 is a pair of groups: lanes 0..31 of an operand carry group 2p,
// lanes 32..63 group 2p + 1.  Multiplying the activation operand by the
// weight operand with one half of its lanes zeroed gives one group's dots,
// already as exact fp32, so the fold needs no conversion: one FMA per output
// and group, with the step products s_a * s_w from fp32 outer-product MFMAs
// as in the INT8 kernel.  The zeroing is done by the instruction's own E8M0
// block scales (2^-127 on the weight lanes of the other group), so the
// operands go in as loaded.
//
// Tiling, operand orientation, tile order and output store are those of the
// INT8 kernel (gemm_tile.h).  The K loop runs over group pairs with two
// register stages (one pair computing while the next pair's loads fly).
// Staging operands through LDS with direct-to-LDS loads (several pairs in
// flight, one barrier per pair) measured slower on this kernel than the
// register pipeline, and is not used.
#include "gemm_tile.h"

#include <cmath>

namespace loopq {
namespace {

// Operands of one group pair, as loaded: the 24 bytes per lane of the wave's
// two weight blocks (MFMA operand A) and two activation blocks (operand B),
// as 16 + 8 bytes, and the steps of the pair's two groups.
struct F6Stage {
  v4i wa[2];
  uint2 wc[2];
  v4i xa[2];
  uint2 xc[2];
  float sa[2][2];  // [group of the pair][row tile h / 1 - h]
  uint32_t sw[2];  // raw fp16 weight step per group of the pair
};

// e2m3 operands use the first six registers of the operand tuple
__device__ __forceinline__ v8i f6_operand(const v4i& a, const uint2& b) {
  return v8i{a[0], a[1], a[2], a[3], (int)b.x, (int)b.y, 0, 0};
}

// A 32x32 result tile gives lane l the 16 elements e at rows
// 8 (e / 4) + 4 (l / 32) + e % 4 of column l % 32.  coef_row(i) is the row of
// the next element (e + 1 mod 16) of the lane holding row i.  The coefficient
// MFMA is fed the weight step of row coef_row(i) in place of row i, so its
// element e is the coefficient of result element e + 1.  The fold then pairs
// result register e + 1 with coefficient register e: as both tuples are
// aligned, the two sit at opposite register parity, and the FMA never reads
// all three operands from one parity (which costs about 1.7x its issue time).
__device__ __forceinline__ int coef_row(int i) {
  return (i & 3) < 3 ? i + 1 : ((((i >> 3) + 1) & 3) << 3) | (i & 4);
}

// SPLIT (rescale mode only): 1, the split-K form of map_tile_split; the two
// halves of each quadrant's sum are added through LDS, the first half's wave
// adding the second's (a fixed order), and only the first half's wave
// stores.  2, the four-way form of map_tile_split4: the four waves of a
// work-group take the four quarters of one quadrant's K pairs, and wave 0
// adds waves 1, 2, 3 in that order and stores.  Every wave of a split form
// reaches the barrier, so none returns early.
template <int MODE, int SPLIT>
__global__ __launch_bounds__(256, 2) void gemm_f6_kernel(GemmArgs g) {
  __shared__ float red[SPLIT == 2 ? 3 * 64 * 64 : SPLIT ? 2 * 64 * 64 : 1];
  const int lane = threadIdx.x & 63;
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
  const int Gp = (Ga + 1) >> 1;
  const int Gw = (Ga + (1 << g.gshift) - 1) >> g.gshift;
  const int mlast = ((g.M + 31) >> 5) - 1;
  const int nlast = ((g.N + 31) >> 5) - 1;

  // buffer loads: wave-uniform resource per tile, fixed per-lane offset, the
  // pair offset as scalar offset (tiles past the edge re-read the last block)
  const void* wp;
  const __half* swp;
  tile_weights(g, active ? m_base : 0, &wp, &swp);  // the grouped form's weight set of these rows
  __amdgpu_buffer_rsrc_t x_rs[2], w_rs[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int mb = min((m_base >> 5) + t, mlast);
    const int nb = min((n_base >> 5) + t, nlast);
    x_rs[t] = make_rsrc(reinterpret_cast<const char*>(g.a) + (int64_t)mb * Gp * kF6BlockBytes,
                        (uint32_t)Gp * kF6BlockBytes);
    w_rs[t] = make_rsrc(reinterpret_cast<const char*>(wp) + (int64_t)nb * Gp * kF6BlockBytes,
                        (uint32_t)Gp * kF6BlockBytes);
  }
  const int op_off = lane * 24;
  // step resources exist only in the rescale mode (the dots mode passes null)
  const __amdgpu_buffer_rsrc_t sa_rs = make_rsrc(g.sa, MODE == 0 ? (uint32_t)g.ld_sa * (uint32_t)Ga * 4u : 0u);
  const __amdgpu_buffer_rsrc_t sw_rs = make_rsrc(swp, MODE == 0 ? (uint32_t)(nlast + 1) * (uint32_t)Gw * 64u : 0u);
  const int sa_off0 = (min((m_base >> 5) + h, mlast) * 32 + c) * 4;
  const int sa_off1 = (min((m_base >> 5) + 1 - h, mlast) * 32 + c) * 4;
  const int sw_off = (min((n_base >> 5) + h, nlast) * Gw * 32 + step_slot(coef_row(c))) * 2;

  auto load = [&](int p, F6Stage& s) {
    const int po = p * kF6BlockBytes;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s.wa[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(w_rs[t], op_off, po, 0));
      s.wc[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(w_rs[t], op_off + 16, po, 0));
      s.xa[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(x_rs[t], op_off, po, 0));
      s.xc[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(x_rs[t], op_off + 16, po, 0));
    }
    if (MODE == 0) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = min(2 * p + q, Ga - 1);  // the missing half of an odd pair re-reads (unused)
        const int so = j * g.ld_sa * 4;
        s.sa[q][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sa_rs, sa_off0, so, 0));
        s.sa[q][1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sa_rs, sa_off1, so, 0));
        s.sw[q] = __builtin_amdgcn_raw_buffer_load_b16(sw_rs, sw_off, (j >> g.gshift) * 64, 0);
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

  // Block scales of the weight operand (E8M0, one per lane = one output
  // column and K-half): 2^0 on the half that carries the group being
  // multiplied, 2^-127 on the other.  The other group's dot then adds at most
  // 1568 * 2^-127 < 2^-116, which leaves a nonzero integer dot unchanged in
  // fp32 and truncates to 0 where the dot is 0.
  const int wscale[2] = {h == 0 ? 127 : 0, h == 1 ? 127 : 0};
  auto mfma = [&](const v8i& w, const v8i& x, int q) {
    const v16f z = {};
    // formats: 2 = e2m3 for both operands; activation scale 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, z, 2, 2, 0, wscale[q], 0, 127);
  };
  auto fold = [&](const v16f& d, const v32f& cf, int half, int t, int u, int j) {
    if (MODE == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        acc[t][u][e] = __builtin_fmaf(d[e], cf[16 * half + ((e + 15) & 15)], acc[t][u][e]);
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
  // one group q of the pair: weight operands keep the lanes of K-half q
  // MFMA and VALU work of one SIMD do not overlap on this chip, and a fold
  // issued right behind the MFMA that produces its operand stalls on it.
  // Each group therefore runs as two blocks, fenced so the scheduler keeps
  // them apart: one coefficient MFMA and the two result MFMAs that use it,
  // then their two folds (the results are complete by the time the folds
  // issue).
  auto group = [&](const F6Stage& s, const v8i (&x)[2], int q, int j) {
    const float swf = MODE == 0 ? __half2float(__ushort_as_half((unsigned short)s.sw[q])) : 0.0f;
    const v8i w0 = f6_operand(s.wa[0], s.wc[0]);
    const v8i w1 = f6_operand(s.wa[1], s.wc[1]);
    auto coef = [&](float sa) -> v32f {
      v32f cf = {};
      if (MODE == 0) cf = __builtin_amdgcn_mfma_f32_32x32x1f32(swf, sa, v32f{}, 0, 0, 0);
      return cf;
    };
    __builtin_amdgcn_sched_barrier(0);
    const v32f cA = coef(s.sa[q][0]);  // (t0,u0) | (t1,u1)
    const v16f d00 = mfma(w0, x[0], q);
    const v16f d11 = mfma(w1, x[1], q);
    __builtin_amdgcn_sched_barrier(0);
    fold(d00, cA, 0, 0, 0, j);
    fold(d11, cA, 1, 1, 1, j);
    __builtin_amdgcn_sched_barrier(0);
    const v32f cB = coef(s.sa[q][1]);  // (t1,u0) | (t0,u1)
    const v16f d01 = mfma(w1, x[0], q);
    const v16f d10 = mfma(w0, x[1], q);
    __builtin_amdgcn_sched_barrier(0);
    fold(d01, cB, 1, 0, 1, j);
    fold(d10, cB, 0, 1, 0, j);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute = [&](const F6Stage& s, int p) {
    const v8i x[2] = {f6_operand(s.xa[0], s.xc[0]), f6_operand(s.xa[1], s.xc[1])};
    group(s, x, 0, 2 * p);
    if (2 * p + 1 < Ga) group(s, x, 1, 2 * p + 1);  // wave-uniform
  };

  // this wave's group pairs [p0, p1)
  const int half = (Gp + 1) >> 1;
  const int quarter = (Gp + 3) >> 2;
  const int p0 = SPLIT == 2 ? min(Gp, kh * quarter) : SPLIT && kh ? half : 0;
  const int p1 = SPLIT == 2 ? min(Gp, p0 + quarter) : SPLIT && !kh ? half : Gp;
  // Loads past the last pair re-read it (in bounds, unused), so the loop
  // body is one basic block the barriers can order.
  if (active && p0 < p1) {
    F6Stage s0, s1;
    load(p0, s0);
    load(min(p0 + 1, p1 - 1), s1);
    int p = p0;
    for (; p + 1 < p1; p += 2) {
      compute(s0, p);
      __builtin_amdgcn_sched_barrier(0);
      load(min(p + 2, p1 - 1), s0);
      __builtin_amdgcn_sched_barrier(0);
      compute(s1, p + 1);
      __builtin_amdgcn_sched_barrier(0);
      load(min(p + 3, p1 - 1), s1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (p < p1) compute(s0, p);
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

// One thread per (column n of the padded weight, group j): the 32 biased
// nibbles of the packed layout -> 24 bytes of e2m3 codes in the fp6 layout.
// Threads run over (column block, group, column): the 32 threads of a block
// and group read 256 contiguous bytes per K-half and write 768 contiguous
// bytes.
__global__ __launch_bounds__(256) void expand_f6_kernel(const uint8_t* __restrict__ w, int K, int Npad,
                                                        char* __restrict__ out) {
  const int Ga = K >> 5;
  const int Gp = (Ga + 1) >> 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Npad * Ga) return;
  const int cc = (int)(idx & 31);
  const int64_t bj = idx >> 5;  // nb * Ga + j
  const int nb = (int)(bj / Ga);
  const int j = (int)(bj - (int64_t)nb * Ga);
  const uint8_t* blk = w + ((int64_t)nb * Ga + j) * kBlockBytes;
  uint32_t piece[8];  // 24-bit e2m3 runs of codes 4r .. 4r + 3
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint2 pk = *reinterpret_cast<const uint2*>(blk + hh * 256 + cc * 8);
    // biased nibble q + 8 -> two's complement nibble q & 15 is an xor with 8
    const uint32_t lo = pk.x ^ 0x88888888u, hi = pk.y ^ 0x88888888u;
    piece[4 * hh + 0] = e2m3_of_codes4(lo);        // codes 16hh + 0..3
    piece[4 * hh + 1] = e2m3_of_codes4(lo >> 4);   // 16hh + 4..7
    piece[4 * hh + 2] = e2m3_of_codes4(hi);        // 16hh + 8..11
    piece[4 * hh + 3] = e2m3_of_codes4(hi >> 4);   // 16hh + 12..15
  }
  uint32_t dw[6];
#pragma unroll
  for (int qd = 0; qd < 2; ++qd) {
    const uint32_t* v = piece + 4 * qd;
    dw[3 * qd + 0] = v[0] | (v[1] << 24);
    dw[3 * qd + 1] = (v[1] >> 8) | (v[2] << 16);
    dw[3 * qd + 2] = (v[2] >> 16) | (v[3] << 8);
  }
  uint2* dst = reinterpret_cast<uint2*>(out + ((int64_t)nb * Gp + (j >> 1)) * kF6BlockBytes +
                                        (cc + 32 * (j & 1)) * 24);
  dst[0] = uint2{dw[0], dw[1]};
  dst[1] = uint2{dw[2], dw[3]};
  dst[2] = uint2{dw[4], dw[5]};
}

}  // namespace

hipError_t launch_expand_weights_f6(const uint8_t* w_codes, int K, int N, void* out, hipStream_t s) {
  const int64_t Npad = padded_cols(N);
  const int64_t threads = Npad * (K / 32);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(expand_f6_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, w_codes,
                     K, (int)Npad, reinterpret_cast<char*>(out));
  return hipGetLastError();
}

// Which tile form spreads a launch best over the chip's SIMDs (four per CU):
// 0 the 128x128 form (every wave over all of K), 1 the two-way split-K form
// (64x128 tiles, half of K per wave), 2 the four-way form (64x64 tiles, a
// quarter of K per wave).  The waves of a launch land about evenly on the
// SIMDs, two at a time (two work-groups per CU), so the busiest SIMD takes
// ceil(waves / SIMDs) waves in rounds of two; a wave that runs alone in the
// last round hides none of its latencies (measured about 25% slower), and a
// split wave pays a fixed exchange through LDS (about one group pair of work
// in the two-way form, one and a half in the four-way form).  Work is counted
// in group pairs.  This picks the four-way form for the 1024-row launches at
// N = 2048 and 2560, the two-way form for the other 1024-row launches, for
// 4096 rows at N = 5632, and for the 8192-row K = 6912 projection (measured
// 6% faster there than whole tiles), and whole tiles elsewhere.  The
// four-way form needs 32 group pairs of K (8 per wave).
int gemm_form(int M, int N, int K) {
  const int64_t simds = 4 * (int64_t)device_cu_count();
  const double pairs = (double)(((K >> 5) + 1) >> 1);
  auto cost = [&](int64_t tiles, double work) {
    const int64_t n = (4 * tiles + simds - 1) / simds;  // waves on the busiest SIMD
    return (double)(n / 2) * 2.0 * work + ((n & 1) ? 1.25 * work : 0.0);
  };
  const int64_t t0 = (int64_t)((N + 127) / 128) * ((M + 127) / 128);
  const int64_t t1 = (int64_t)((N + 127) / 128) * ((M + 63) / 64);
  const int64_t t2 = (int64_t)((N + 63) / 64) * ((M + 63) / 64);
  const double c0 = cost(t0, pairs);
  const double c1 = cost(t1, pairs / 2.0 + 1.0);
  const double c2 = pairs >= 32 ? cost(t2, pairs / 4.0 + 1.5) : 1e30;
  if (c2 < c1 && c2 < c0) return 2;
  return c1 < c0 ? 1 : 0;
}

hipError_t launch_gemm_f6(const void* a_tiled, const float* a_scales_gm, int ld_sa, int M, int K,
                          int N, const void* w_f6, const __half* w_scales, int gw, float* y,
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
  g.w = w_f6;
  g.sw = w_scales;
  g.gshift = gw == 128 ? 2 : 0;
  g.y = y;
  g.dots = dots;
  const int64_t tiles = (int64_t)((N + 127) / 128) * ((M + 127) / 128);
  const int64_t tiles_split = (int64_t)((N + 127) / 128) * ((M + 63) / 64);
  const int form = mode == 0 ? gemm_form(M, N, K) : 0;
  if (form == 2) {
    dim3 grid((unsigned)((int64_t)((N + 63) / 64) * ((M + 63) / 64)));
    hipLaunchKernelGGL((gemm_f6_kernel<0, 2>), grid, dim3(256), 0, s, g);
  } else if (form == 1) {
    dim3 grid((unsigned)tiles_split);
    hipLaunchKernelGGL((gemm_f6_kernel<0, 1>), grid, dim3(256), 0, s, g);
  } else {
    dim3 grid((unsigned)tiles);
    if (mode == 0)
      hipLaunchKernelGGL((gemm_f6_kernel<0, 0>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_f6_kernel<1, 0>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace loopq
