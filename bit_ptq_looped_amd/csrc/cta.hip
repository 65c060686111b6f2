// CTA: the loop-transition adapter.
//
// "paper_specification.yaml", loopq_components.cta (Section 4.3, Eq.(7)):
// an affine plus gated low-rank adapter applied only at loop transitions, U
// and V shared, a_t, b_t and eta_t per transition; experiment_hyperparameters
// cta_rank 8.  The equation itself is not printed on the pages; this path
// takes the map  h -> a_t * h + b_t + eta_t * U (V^T h)  per row (a, b
// elementwise, eta a scalar gate, U and V [K][r]), identity at a = 1, b = 0,
// eta = 0, and stores the result in the state's type (bf16 rounded to nearest
// even, or fp32).
//
// One work-group takes kRows consecutive rows.  Pass 1 forms z = V^T h of
// each row (each thread runs over its k in order, then a butterfly within the
// wave and the four waves in order: a fixed reduction order, so the result
// does not depend on timing); pass 2 re-reads the rows (from L2) and writes
// fma(eta, sum_j U[k][j] z_j, fma(a_k, h_k, b_k)).  Rows whose transition
// index is negative are copied unchanged (loop 0 of a looped forward).  A row
// is read completely before any of its elements is written, so the output
// may be the input itself.
#include "loopq_internal.h"
#include "quant_core.h"

namespace loopq {
namespace {

constexpr int kRows = 4;      // rows per work-group
constexpr int kMaxRank = 16;  // largest r

struct CtaArgs {
  const void* h;     // [rows][K], bf16 or fp32
  void* out;         // same layout and type (may be h)
  const float* U;    // [K][r]
  const float* V;    // [K][r]
  const float* a;    // [transitions][K]
  const float* b;    // [transitions][K]
  ClipTable eta;     // eta of each transition
  int64_t rows;
  int K, r, bf16;
  int64_t rows_per_tr;  // rows of one transition block
  int first;            // transition of the first block (-1: copy it)
};

// 8 consecutive elements of row m from k (k % 8 == 0)
__device__ __forceinline__ void load8(const CtaArgs& g, int64_t m, int k, float (&v)[8]) {
  if (g.bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(g.h) + m * g.K + k);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_bits_to_float(w[q] & 0xffffu);
      v[2 * q + 1] = bf16_bits_to_float(w[q] >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(g.h) + m * g.K + k);
    const float4 x0 = p[0], x1 = p[1];
    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
    v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
  }
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite values; a NaN
// stays a NaN)
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void store8(const CtaArgs& g, int64_t m, int k, const float (&v)[8]) {
  if (g.bf16) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = bf16_bits_rne(v[2 * q]) | (bf16_bits_rne(v[2 * q + 1]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(g.out) + m * g.K + k) = uint4{w[0], w[1], w[2], w[3]};
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(g.out) + m * g.K + k);
    p[0] = float4{v[0], v[1], v[2], v[3]};
    p[1] = float4{v[4], v[5], v[6], v[7]};
  }
}

__global__ __launch_bounds__(256) void cta_kernel(CtaArgs g) {
  __shared__ float red[4][kRows][kMaxRank];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * kRows;
  const int K = g.K, r = g.r;
  int tr[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
    tr[i] = row0 + i < g.rows ? (int)((row0 + i) / g.rows_per_tr) + g.first : -2;  // -2: past the end

  // pass 1: z = V^T h of every adapted row
  float acc[kRows][kMaxRank];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
#pragma unroll
    for (int j = 0; j < kMaxRank; ++j) acc[i][j] = 0.0f;
  for (int k = tid * 8; k < K; k += 256 * 8) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      if (tr[i] < 0) continue;  // uniform over the work-group
      float hv[8];
      load8(g, row0 + i, k, hv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float* vk = g.V + (int64_t)(k + e) * r;
#pragma unroll
        for (int j = 0; j < kMaxRank; ++j)
          if (j < r) acc[i][j] = fmaf(vk[j], hv[e], acc[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    if (tr[i] < 0) continue;
#pragma unroll
    for (int j = 0; j < kMaxRank; ++j) {
      if (j >= r) continue;
      float v = acc[i][j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) red[wave][i][j] = v;
    }
  }
  __syncthreads();
  float z[kRows][kMaxRank];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
#pragma unroll
    for (int j = 0; j < kMaxRank; ++j)
      z[i][j] = (tr[i] >= 0 && j < r) ? ((red[0][i][j] + red[1][i][j]) + red[2][i][j]) + red[3][i][j] : 0.0f;

  // pass 2: the adapted rows (copied rows unchanged)
  for (int k = tid * 8; k < K; k += 256 * 8) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      if (tr[i] == -2) continue;
      float hv[8];
      load8(g, row0 + i, k, hv);
      if (tr[i] >= 0) {
        const float* ak = g.a + (int64_t)tr[i] * K + k;
        const float* bk = g.b + (int64_t)tr[i] * K + k;
        const float eta = g.eta.c[tr[i]];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float* uk = g.U + (int64_t)(k + e) * r;
          float s = 0.0f;
#pragma unroll
          for (int j = 0; j < kMaxRank; ++j)
            if (j < r) s = fmaf(uk[j], z[i][j], s);
          hv[e] = fmaf(eta, s, fmaf(ak[e], hv[e], bk[e]));
        }
      }
      store8(g, row0 + i, k, hv);
    }
  }
}

}  // namespace

hipError_t launch_cta(const void* h, int bf16, int64_t rows, int K, const float* U, const float* V, int r,
                      const float* a, const float* b, const float* eta, int ntr, int64_t rows_per_tr, int first,
                      void* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K <= 0 || K % 32 != 0 || r < 1 || r > kMaxRank || rows_per_tr <= 0 || ntr < 0 || ntr > 64)
    return hipErrorInvalidValue;
  CtaArgs g;
  memset(&g, 0, sizeof(g));
  g.h = h;
  g.out = out;
  g.U = U;
  g.V = V;
  g.a = a;
  g.b = b;
  for (int t = 0; t < ntr; ++t) g.eta.c[t] = eta[t];
  g.rows = rows;
  g.K = K;
  g.r = r;
  g.bf16 = bf16;
  g.rows_per_tr = rows_per_tr;
  g.first = first;
  // every row's transition must have parameters
  const int64_t last_tr = (rows - 1) / rows_per_tr + first;
  if (last_tr >= ntr) return hipErrorInvalidValue;
  const int64_t blocks = (rows + kRows - 1) / kRows;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cta_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

int cta_max_rank() { return kMaxRank; }

}  // namespace loopq
