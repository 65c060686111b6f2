// Input of one step of the adapter recurrence: x = cat(s, e) per row.
//
// "Quantizing Looped Transformers: Feedback Exposure and Calibration
// Blindness", Figure 4 (the Huginn recurrence loop): the adapter maps the
// concatenation of the recurrent state and the embedding back to the model
// width, so loop t + 1's quantized input is cat(s_{t+1}, e) with s_{t+1} the
// previous loop's output.  One float4 per thread, rows of 2N fp32.
#include "loopq_internal.h"

namespace loopq {
namespace {

__global__ __launch_bounds__(256) void concat_state_kernel(const float* __restrict__ s, const float* __restrict__ e,
                                                           float* __restrict__ x, int M, int N) {
  const int n4 = N >> 2;
  const int64_t total = (int64_t)M * 2 * n4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / (2 * n4);
    const int c = (int)(i - m * 2 * n4);
    const float4 v = c < n4 ? reinterpret_cast<const float4*>(s)[m * n4 + c]
                            : reinterpret_cast<const float4*>(e)[m * n4 + (c - n4)];
    reinterpret_cast<float4*>(x)[i] = v;
  }
}

}  // namespace

hipError_t launch_concat_state(const float* s, const float* e, float* x, int M, int N, hipStream_t st) {
  const int64_t total = (int64_t)M * (N / 2);  // float4 of the M x 2N output
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(concat_state_kernel, dim3((unsigned)blocks), dim3(256), 0, st, s, e, x, M, N);
  return hipGetLastError();
}

}  // namespace loopq
