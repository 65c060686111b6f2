// Offline weight-side kernels: transform fold (fp64), INT4 packing, export.
//
// Fold: "paper_specification.yaml", loopq_components.shared_transformed_backbone
// and implementation_status lq3 (the weights absorb the exact inverse
// transpose of the transform, before any quantization).  Row n of the [N][K] weight storage is output column n, and
//   w~[n] = vec_r(P1^-1 * reshape(w[n], n1, n2) * P2^-T),
// accumulated in fp64 and rounded once to fp32.  The factors are inverted on
// the GPU by Gauss-Jordan elimination with partial pivoting in fp64.
//
// Packing: Eq.(4) (lq1_quantization) with clip 1 on each K-group of group_w
// (32, or 128 as in "Quantizing Looped Transformers", Figure 3):
//   s = fl16(fl32(absmax / 7)), q = clamp(rint(fl32(w / s)), -7, 7), q = 0 if s == 0.
// Codes go to the tiled nibble layout described in loopq_internal.h.
#include "loopq_internal.h"

namespace loopq {

// Status word of the synchronizing offline calls: bit 0 = a weight step
// overflowed fp16, bit 1 = a singular transform factor.
__device__ int g_loopq_status;

namespace {

__global__ void reset_status_kernel() { g_loopq_status = 0; }

__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ w, int K, int N, int gw,
                                                   uint8_t* __restrict__ codes,
                                                   __half* __restrict__ scales) {
  const int Gw = (K + gw - 1) / gw;
  const int Npad = (N + 31) / 32 * 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)Npad * Gw) return;
  const int n = (int)(idx / Gw);
  const int jw = (int)(idx - (int64_t)n * Gw);
  const int k0 = jw * gw;
  const int k1 = min(K, k0 + gw);
  const bool real = n < N;
  const float* wr = w + (int64_t)(real ? n : 0) * K;

  float amax = 0.0f;
  if (real)
    for (int k = k0; k < k1; ++k) amax = fmaxf(amax, fabsf(wr[k]));
  const float s32 = amax / 7.0f;           // correctly rounded fp32 division
  const __half s16 = __float2half_rn(s32);  // RNE to binary16
  const float sdiv = __half2float(s16);
  if (__builtin_isinf(sdiv)) atomicOr(&g_loopq_status, 1);
  const int nb = n >> 5, c = n & 31;
  scales[((int64_t)nb * Gw + jw) * 32 + step_slot(c)] = s16;

  const int Kc = K >> 5;
  for (int kc = k0 >> 5; kc < (k1 >> 5); ++kc) {
    uint8_t* blk = codes + ((int64_t)nb * Kc + kc) * kBlockBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        uint32_t word = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int klo = kc * 32 + h * 16 + d * 8 + b;
          int qlo = 0, qhi = 0;
          if (real && sdiv > 0.0f) {
            qlo = (int)fminf(fmaxf(__builtin_rintf(wr[klo] / sdiv), -7.0f), 7.0f);
            qhi = (int)fminf(fmaxf(__builtin_rintf(wr[klo + 4] / sdiv), -7.0f), 7.0f);
          }
          const uint32_t byte = (uint32_t)(qlo + 8) | ((uint32_t)(qhi + 8) << 4);
          word |= byte << (8 * b);
        }
        *reinterpret_cast<uint32_t*>(blk + h * 256 + c * 8 + d * 4) = word;
      }
    }
  }
}

__global__ __launch_bounds__(256) void export_kernel(const uint8_t* __restrict__ codes,
                                                     const __half* __restrict__ scales, int K,
                                                     int N, int gw, int8_t* __restrict__ out_codes,
                                                     uint16_t* __restrict__ out_scales) {
  const int Kc = K >> 5;
  const int Gw = (K + gw - 1) / gw;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)N * Kc) return;
  const int n = (int)(idx / Kc);
  const int kc = (int)(idx - (int64_t)n * Kc);
  const int nb = n >> 5, c = n & 31;
  const uint8_t* blk = codes + ((int64_t)nb * Kc + kc) * kBlockBytes;
  for (int h = 0; h < 2; ++h)
    for (int i = 0; i < 16; ++i) {
      const uint8_t byte = blk[h * 256 + c * 8 + (i >> 3) * 4 + (i & 3)];
      const int nib = ((i & 7) < 4) ? (byte & 15) : (byte >> 4);
      out_codes[(int64_t)n * K + kc * 32 + h * 16 + i] = (int8_t)(nib - 8);
    }
  if (out_scales != nullptr && (kc * 32) % gw == 0) {
    const int jw = kc * 32 / gw;
    out_scales[(int64_t)n * Gw + jw] =
        __half_as_ushort(scales[((int64_t)nb * Gw + jw) * 32 + step_slot(c)]);
  }
}

// Gauss-Jordan inverse of one n x n fp32 factor in fp64; aug is [n][2n] fp64
// scratch, inv receives [n][n] fp64.  One work-group of 256 threads.
__global__ __launch_bounds__(256) void invert_kernel(const float* __restrict__ P, int n,
                                                     double* __restrict__ aug,
                                                     double* __restrict__ inv) {
  __shared__ double s_f[128];
  __shared__ double s_val[256];
  __shared__ int s_idx[256];
  const int tid = threadIdx.x;
  const int w2 = 2 * n;
  for (int e = tid; e < n * w2; e += 256) {
    const int r = e / w2, k = e - (e / w2) * w2;
    aug[e] = k < n ? (double)P[r * n + k] : (k - n == r ? 1.0 : 0.0);
  }
  __syncthreads();
  for (int c = 0; c < n; ++c) {
    // pivot: largest |aug[r][c]| over r >= c (first index on ties)
    double best = -1.0;
    int bi = c;
    for (int r = c + tid; r < n; r += 256) {
      const double v = fabs(aug[r * w2 + c]);
      if (v > best) { best = v; bi = r; }
    }
    s_val[tid] = best;
    s_idx[tid] = bi;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) {
        const double v2 = s_val[tid + off];
        const int i2 = s_idx[tid + off];
        if (v2 > s_val[tid] || (v2 == s_val[tid] && i2 < s_idx[tid])) {
          s_val[tid] = v2;
          s_idx[tid] = i2;
        }
      }
      __syncthreads();
    }
    const int p = s_idx[0];
    const double pv = s_val[0];
    if (tid == 0 && !(pv > 0.0)) atomicOr(&g_loopq_status, 2);
    if (p != c)
      for (int k = tid; k < w2; k += 256) {
        const double t = aug[c * w2 + k];
        aug[c * w2 + k] = aug[p * w2 + k];
        aug[p * w2 + k] = t;
      }
    __syncthreads();
    const double piv = aug[c * w2 + c];
    for (int r = tid; r < n; r += 256) s_f[r] = aug[r * w2 + c];
    __syncthreads();
    for (int k = tid; k < w2; k += 256) aug[c * w2 + k] = aug[c * w2 + k] / piv;
    __syncthreads();
    for (int e = tid; e < n * w2; e += 256) {
      const int r = e / w2, k = e - (e / w2) * w2;
      if (r != c) aug[e] = aug[e] - s_f[r] * aug[c * w2 + k];
    }
    __syncthreads();
  }
  for (int e = tid; e < n * n; e += 256) {
    const int r = e / n, k = e - (e / n) * n;
    inv[e] = aug[r * w2 + n + k];
  }
}

// One work-group per weight row: U = W_n * P2inv^T (fp64), out = P1inv * U.
__global__ __launch_bounds__(256) void fold_kernel(const float* __restrict__ w, int K,
                                                   const double* __restrict__ P1i, int n1,
                                                   const double* __restrict__ P2i, int n2,
                                                   float* __restrict__ out) {
  extern __shared__ double s_buf[];
  double* sW = s_buf;      // [n1][n2]
  double* sU = s_buf + K;  // [n1][n2]
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const float* wr = w + (int64_t)n * K;
  for (int k = tid; k < K; k += 256) sW[k] = (double)wr[k];
  __syncthreads();
  for (int e = tid; e < K; e += 256) {
    const int a = e / n2, j = e - (e / n2) * n2;
    double acc = 0.0;
    for (int b = 0; b < n2; ++b) acc = fma(sW[a * n2 + b], P2i[j * n2 + b], acc);
    sU[e] = acc;
  }
  __syncthreads();
  for (int e = tid; e < K; e += 256) {
    const int i = e / n2, j = e - (e / n2) * n2;
    double acc = 0.0;
    for (int a = 0; a < n1; ++a) acc = fma(P1i[i * n1 + a], sU[a * n2 + j], acc);
    out[(int64_t)n * K + e] = (float)acc;  // one rounding to fp32 (RNE)
  }
}

}  // namespace

hipError_t reset_status(hipStream_t s) {
  hipLaunchKernelGGL(reset_status_kernel, dim3(1), dim3(1), 0, s);
  return hipGetLastError();
}

hipError_t read_status(int* host_status, hipStream_t s) {
  hipError_t e = hipMemcpyFromSymbolAsync(host_status, HIP_SYMBOL(g_loopq_status), sizeof(int), 0,
                                          hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

hipError_t launch_pack_weights(const float* w, int K, int N, int gw, uint8_t* codes,
                               __half* scales, hipStream_t s) {
  const int64_t threads = padded_cols(N) * weight_groups(K, gw);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, K, N, gw, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_export_weights(const uint8_t* codes, const __half* scales, int K, int N, int gw,
                                 int8_t* out_codes, uint16_t* out_scales, hipStream_t s) {
  const int64_t threads = (int64_t)N * (K / 32);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(export_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes, scales, K, N,
                     gw, out_codes, out_scales);
  return hipGetLastError();
}

// ws layout (fp64): aug [128][256], P1inv [n1][n1], P2inv [n2][n2]
hipError_t launch_fold(const float* w, int K, int N, const float* P1, int n1, const float* P2,
                       int n2, float* out, void* ws, hipStream_t s) {
  double* aug = reinterpret_cast<double*>(ws);
  double* p1i = aug + 128 * 256;
  double* p2i = p1i + n1 * n1;
  hipLaunchKernelGGL(invert_kernel, dim3(1), dim3(256), 0, s, P1, n1, aug, p1i);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(invert_kernel, dim3(1), dim3(256), 0, s, P2, n2, aug, p2i);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int lds = 2 * K * (int)sizeof(double);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(fold_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fold_kernel, dim3(N), dim3(256), lds, s, w, K, p1i, n1, p2i, n2, out);
  return hipGetLastError();
}

}  // namespace loopq
