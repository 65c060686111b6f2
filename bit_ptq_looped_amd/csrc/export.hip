// Test export of the activation codes a forward call leaves in its workspace
// (gfx950).  The GEMM paths keep their codes in internal tiled layouts (e2m3
// fp6 operands for W4A4, int8 blocks for W4A8, loopq_internal.h); the
// few-row path keeps canonical codes.  This turns any of them back into
// canonical int8 codes [rows][K] and row-major fp32 steps [rows][K/32], so
// the codes the product actually consumed can be compared with Eq.(4)
// ("paper_specification.yaml", lq1_quantization) bit for bit.
#include "loopq_internal.h"

namespace loopq {
namespace {

// An e2m3 field (sign, two exponent bits with bias 1, three mantissa bits)
// as the integer it encodes.  Every pattern of a code -7..7 is an exact
// integer; any other pattern (a fraction, or 7.5) comes back as -128, a
// value no code takes, so a damaged field cannot pass for a code.
__device__ __forceinline__ int code_of_e2m3(uint32_t f) {
  const int m = (int)(f & 7u), e = (int)((f >> 3) & 3u);
  const int v8 = e == 0 ? m : (8 + m) << (e - 1);  // 8 x the magnitude
  if ((v8 & 7) != 0 || v8 > 56) return -128;
  const int v = v8 >> 3;
  return (f & 32u) ? -v : v;
}

// One thread per (row, group): 32 codes and the step.
__global__ __launch_bounds__(256) void export_act_kernel(const uint8_t* __restrict__ codes,
                                                         const float* __restrict__ steps, int rows, int K,
                                                         int fmt, int ld, int steps_gm,
                                                         int8_t* __restrict__ out_codes,
                                                         float* __restrict__ out_steps) {
  const int Ga = K >> 5;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * Ga) return;
  const int row = (int)(idx / Ga);
  const int j = (int)(idx - (int64_t)row * Ga);
  int8_t* o = out_codes + (int64_t)row * K + j * 32;
  if (fmt == kCodesTiledF6) {
    // 24 bytes per (row, group), code i at bits 6i .. 6i + 5 (little endian)
    const uint8_t* p = codes + ((int64_t)(row >> 5) * group_pairs(K) + (j >> 1)) * kF6BlockBytes +
                       ((row & 31) + 32 * (j & 1)) * 24;
    uint32_t w[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int b = 6 * i, wi = b >> 5, sh = b & 31;
      uint32_t v = w[wi] >> sh;
      if (sh > 26) v |= w[wi + 1] << (32 - sh);
      o[i] = (int8_t)code_of_e2m3(v & 63u);
    }
  } else if (fmt == kCodesTiledI8) {
    // block (row / 32, j) of 1 KiB: K-half h, row r, byte i at h * 512 + r * 16 + i
    const uint8_t* p = codes + ((int64_t)(row >> 5) * Ga + j) * 1024 + (row & 31) * 16;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) o[kk] = (int8_t)p[(kk >> 4) * 512 + (kk & 15)];
  } else {
    const uint8_t* p = codes + (int64_t)row * K + j * 32;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) o[kk] = (int8_t)p[kk];
  }
  out_steps[(int64_t)row * Ga + j] = steps_gm ? steps[(int64_t)j * ld + row] : steps[(int64_t)row * Ga + j];
}

}  // namespace

hipError_t launch_export_act(const void* codes, const float* steps, int rows, int K, int fmt, int ld,
                             int steps_gm, int8_t* out_codes, float* out_steps, hipStream_t s) {
  const int64_t n = (int64_t)rows * (K / 32);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(export_act_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(codes), steps, rows, K, fmt, ld, steps_gm, out_codes,
                     out_steps);
  return hipGetLastError();
}

}  // namespace loopq
