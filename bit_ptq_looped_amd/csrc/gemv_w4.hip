// Small-row (decode) form of the W4A4 / W4A8 GEMM with per-group rescale
// (gfx950):
//
//   y[m][n] = sum_j s_a[m][j] * s_w[n][32j / group_w] * d[m][n][j],
//   d[m][n][j] = sum_{k in group j} q_a[m][k] * q_w[n][k]   (exact int32)
//
// Method: the integer form of the simulated quantize-dequantize product of
// Eq.(4)-quantized operands ("paper_specification.yaml", lq1_quantization;
// the README of the LoopQ reproduction, "Protocol").  With a handful of token
// rows (decode: M * T <= 16) the product is bound by streaming the packed
// INT4 weights from HBM once; the weights are read as packed (no operand
// expansion) and the group dots run on the VALU with V_DOT4_I32_I8 (exact).
//
// Work split: one work-group per 8 output columns, all of K.  Thread t takes
// column t % 8 of the group's 8 and K-slice t / 8 of 32: groups j = slice,
// slice + 32, ...  For each group it unpacks the column's 32 nibbles, forms
// the dots with every row's 32 codes (read from the canonical code matrix;
// the 8 threads of a slice read the same bytes), and folds them with the step
// product fl32(s_w * s_a) as the MFMA kernels do.  The 32 slice partials of a
// column are summed in a fixed order through LDS, so results are
// deterministic.
#include "loopq_internal.h"

namespace loopq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

struct GemvArgs {
  const int8_t* a;   // canonical codes [R][K]
  const float* sa;   // row-major steps [R][K/32] (mode 0)
  int R, K, N;
  const uint8_t* w;  // packed nibbles
  const __half* sw;  // packed steps [Npad/32][Gw][32] (mode 0)
  int gshift;
  float* y;          // [R][N] (mode 0)
  int32_t* dots;     // [R][N][K/32] (mode 1)
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

constexpr int kGemvCols = 8;
constexpr int kGemvSlices = 32;

template <int RM, int MODE>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs g) {
  __shared__ float red[kGemvSlices][RM][kGemvCols];
  const int t = threadIdx.x;
  const int c8 = t & (kGemvCols - 1);
  const int slice = t >> 3;
  const int n = blockIdx.x * kGemvCols + c8;  // < padded N: padded columns hold code 0
  const int nb = n >> 5, cc = n & 31;
  const int Ga = g.K >> 5;
  const int Gw = (Ga + (1 << g.gshift) - 1) >> g.gshift;
  const int R = g.R;

  float acc[RM];
#pragma unroll
  for (int m = 0; m < RM; ++m) acc[m] = 0.0f;

  for (int j = slice; j < Ga; j += kGemvSlices) {
    const uint8_t* blk = g.w + ((int64_t)nb * Ga + j) * kBlockBytes + cc * 8;
    const v4i w0 = unpack16(*reinterpret_cast<const uint2*>(blk));        // K 32j + 0..15
    const v4i w1 = unpack16(*reinterpret_cast<const uint2*>(blk + 256));  // K 32j + 16..31
    float swf = 0.0f;
    if (MODE == 0)
      swf = __half2float(g.sw[((int64_t)nb * Gw + (j >> g.gshift)) * 32 + step_slot(cc)]);
#pragma unroll
    for (int m = 0; m < RM; ++m) {
      if (m < R) {
        const v4i* ap = reinterpret_cast<const v4i*>(g.a + (int64_t)m * g.K + j * 32);
        const v4i a0 = ap[0], a1 = ap[1];
        int d = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_sdot4(a0[i], w0[i], d, false);
#pragma unroll
        for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_sdot4(a1[i], w1[i], d, false);
        if (MODE == 0) {
          const float coef = swf * g.sa[(int64_t)m * Ga + j];  // fl32(s_w * s_a)
          acc[m] = __builtin_fmaf((float)d, coef, acc[m]);
        } else if (n < g.N) {
          g.dots[((int64_t)m * g.N + n) * Ga + j] = d;
        }
      }
    }
  }
  if (MODE != 0) return;
#pragma unroll
  for (int m = 0; m < RM; ++m) red[slice][m][c8] = acc[m];
  __syncthreads();
  // one thread per (row, column): the slice partials in slice order
  for (int o = t; o < RM * kGemvCols; o += 256) {
    const int m = o / kGemvCols, c = o % kGemvCols;
    const int col = blockIdx.x * kGemvCols + c;
    if (m < R && col < g.N) {
      float s = 0.0f;
      for (int q = 0; q < kGemvSlices; ++q) s += red[q][m][c];
      g.y[(int64_t)m * g.N + col] = s;
    }
  }
}

}  // namespace

hipError_t launch_gemv(const int8_t* a_canon, const float* a_scales, int R, int K, int N,
                       const uint8_t* w_codes, const __half* w_scales, int gw, float* y,
                       int32_t* dots, int mode, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (R > kGemvMaxRows) return hipErrorInvalidValue;
  GemvArgs g;
  g.a = a_canon;
  g.sa = a_scales;
  g.R = R;
  g.K = K;
  g.N = N;
  g.w = w_codes;
  g.sw = w_scales;
  g.gshift = gw == 128 ? 2 : 0;
  g.y = y;
  g.dots = dots;
  const dim3 grid((unsigned)(padded_cols(N) / kGemvCols));
  if (R <= 4) {
    if (mode == 0)
      hipLaunchKernelGGL((gemv_kernel<4, 0>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemv_kernel<4, 1>), grid, dim3(256), 0, s, g);
  } else {
    if (mode == 0)
      hipLaunchKernelGGL((gemv_kernel<kGemvMaxRows, 0>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemv_kernel<kGemvMaxRows, 1>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace loopq
