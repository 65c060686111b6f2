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
// Resident form (rank 8, K <= 2560: the hidden sizes of the block and the
// stack):
// each wave issues every load of its rows (4 bf16 rows or 2 fp32 rows, all
// of K) at once and keeps them in registers through both passes, so each row
// is read from HBM once and the wait for it is paid once; the tiles of V, and
// then of U, a and b, are loaded into registers one tile ahead and staged in
// LDS behind a barrier.  Its arithmetic is the general form's, in the same
// order, so both give the same bits.
//
// General form (any K): a work-group takes up to 16 consecutive rows of one
// transition block (4 per wave) and runs over K in tiles of 512 (8
// consecutive elements per lane).  Pass 1 forms z = V^T h of each row: the
// tile of V is staged in LDS (element k of column j at [j][k % 8][lane],
// conflict-free reads), every
// lane accumulates its elements in order and the wave sums its lanes by a
// butterfly -- a fixed order, so the result does not depend on timing.  Pass 2
// re-reads the rows (from L2) with the tiles of U, a and b in LDS and writes
// fma(eta, sum_j U[k][j] z_j, fma(a_k, h_k, b_k)).  Rows whose transition
// index is negative are copied unchanged (loop 0 of a looped forward).  A
// work-group reads all of its rows before it writes any of them and rows of
// different work-groups are disjoint, so the output may be the input itself.
#include "loopq_internal.h"
#include "quant_core.h"

namespace loopq {
namespace {

constexpr int kRows = 16;     // rows per work-group (4 per wave)
constexpr int kTile = 512;    // elements of K per tile (8 per lane)
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
  int64_t rows_per_tr;  // rows of one transition block (blockIdx.y)
  int first;            // transition of block 0 (-1: copy it)
  int vec;              // U and V 16-byte aligned with r equal to the kernel's R
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

// two fp32 values -> their bf16 bits (low half the first), round to nearest,
// ties to even, one V_CVT_PK_BF16_F32 (a NaN stays a NaN)
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void store8(const CtaArgs& g, int64_t m, int k, const float (&v)[8]) {
  if (g.bf16) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = bf16x2_rne(v[2 * q], v[2 * q + 1]);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(g.out) + m * g.K + k) = uint4{w[0], w[1], w[2], w[3]};
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(g.out) + m * g.K + k);
    p[0] = float4{v[0], v[1], v[2], v[3]};
    p[1] = float4{v[4], v[5], v[6], v[7]};
  }
}

template <int R>  // R >= r: columns of U and V (those past r are zero)
__global__ __launch_bounds__(256) void cta_kernel(CtaArgs g) {
  __shared__ float sW[R * kTile];  // V, then U: column j, element k0 + 8 l + e at [j][e][l]
  __shared__ float sA[kTile], sB[kTile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = g.K, r = g.r;
  const int tr = (int)blockIdx.y + g.first;  // uniform over the work-group
  const int64_t rb0 = (int64_t)blockIdx.y * g.rows_per_tr;
  const int64_t rb1 = min(rb0 + g.rows_per_tr, g.rows);
  const int64_t r0 = rb0 + (int64_t)blockIdx.x * kRows + wave * 4;  // this wave's first row
  const int nr = (int)max((int64_t)0, min((int64_t)4, rb1 - r0));    // its rows (0..4)

  // stage elements [k0, k0 + kn) of the columns of W ([K][r]) into sW
  auto stage = [&](const float* __restrict__ W, int k0, int kn) {
    for (int q = tid; q < kn * R; q += 256) {
      const int kk = q / R, j = q - kk * R;
      sW[j * kTile + (kk & 7) * 64 + (kk >> 3)] = j < r ? W[(int64_t)(k0 + kk) * r + j] : 0.0f;
    }
  };

  float z[4][R];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) z[i][j] = 0.0f;

  if (tr >= 0) {  // pass 1: z = V^T h
    for (int k0 = 0; k0 < K; k0 += kTile) {
      const int kn = min(kTile, K - k0);
      __syncthreads();  // the previous tile is no longer read
      stage(g.V, k0, kn);
      __syncthreads();
      const int k = k0 + 8 * lane;
      if (k < k0 + kn) {
        float hv[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nr) load8(g, r0 + i, k, hv[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v[R];
#pragma unroll
          for (int j = 0; j < R; ++j) v[j] = sW[j * kTile + e * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < nr)
#pragma unroll
              for (int j = 0; j < R; ++j) z[i][j] = fmaf(v[j], hv[i][e], z[i][j]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < R; ++j) {
        float v = z[i][j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        z[i][j] = v;
      }
  }

  // pass 2: the adapted rows (copied rows unchanged)
  const float eta = tr >= 0 ? g.eta.c[tr] : 0.0f;
  for (int k0 = 0; k0 < K; k0 += kTile) {
    const int kn = min(kTile, K - k0);
    if (tr >= 0) {
      __syncthreads();
      stage(g.U, k0, kn);
      for (int q = tid; q < kn; q += 256) {
        sA[(q & 7) * 64 + (q >> 3)] = g.a[(int64_t)tr * K + k0 + q];
        sB[(q & 7) * 64 + (q >> 3)] = g.b[(int64_t)tr * K + k0 + q];
      }
      __syncthreads();
    }
    const int k = k0 + 8 * lane;
    if (k >= k0 + kn || nr == 0) continue;
    float hv[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < nr) load8(g, r0 + i, k, hv[i]);
    if (tr >= 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float u[R];
#pragma unroll
        for (int j = 0; j < R; ++j) u[j] = sW[j * kTile + e * 64 + lane];
        const float ak = sA[e * 64 + lane], bk = sB[e * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = 0.0f;
#pragma unroll
          for (int j = 0; j < R; ++j) s = fmaf(u[j], z[i][j], s);
          hv[i][e] = fmaf(eta, s, fmaf(ak, hv[i][e], bk));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < nr) store8(g, r0 + i, k, hv[i]);
  }
}

constexpr int kResTiles = 5;  // the resident form's largest K: kResTiles * kTile

// The resident form: RW rows per wave (4 bf16 or 2 fp32, 4 * RW per
// work-group), NT tiles of K, every row element loaded once into hw.
template <int R, int NT, bool BF16>
__global__ __launch_bounds__(256) void cta_resident_kernel(CtaArgs g) {
  constexpr int RW = BF16 ? 4 : 2;  // rows per wave
  constexpr int NW = BF16 ? 4 : 8;  // 32-bit words of a lane's 8 elements
  constexpr int NP = 2 * R;         // staged elements per thread and tile
  __shared__ float sW[R * kTile];   // as in the general form
  __shared__ float sA[kTile], sB[kTile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = g.K;
  const int tr = (int)blockIdx.y + g.first;
  const int64_t rb0 = (int64_t)blockIdx.y * g.rows_per_tr;
  const int64_t rb1 = min(rb0 + g.rows_per_tr, g.rows);
  const int64_t r0 = rb0 + (int64_t)blockIdx.x * (4 * RW) + wave * RW;
  const int nr = (int)max((int64_t)0, min((int64_t)RW, rb1 - r0));

  uint32_t hw[NT][RW][NW];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int k = t * kTile + 8 * lane;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if (i < nr && k < K) {
        const uint4* p = BF16 ? reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(g.h) + (r0 + i) * K + k)
                              : reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(g.h) + (r0 + i) * K + k);
#pragma unroll
        for (int v = 0; v < NW / 4; ++v) {
          const uint4 u = p[v];
          hw[t][i][4 * v] = u.x; hw[t][i][4 * v + 1] = u.y; hw[t][i][4 * v + 2] = u.z; hw[t][i][4 * v + 3] = u.w;
        }
      } else {
#pragma unroll
        for (int w = 0; w < NW; ++w) hw[t][i][w] = 0u;
      }
    }
  }
  auto elems = [&](int t, int i, float (&v)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      v[q] = BF16 ? bf16_bits_to_float(q & 1 ? hw[t][i][q >> 1] >> 16 : hw[t][i][q >> 1] & 0xffffu)
                  : __uint_as_float(hw[t][i][q]);
  };

  // the thread's share of tile t of W ([K][r]) into pre; element (kk, j) of
  // the tile goes to sW[j][kk % 8][kk / 8]
  auto fetch = [&](const float* __restrict__ W, int t, float (&pre)[NP]) {
    const int k0 = t * kTile, kn = min(kTile, K - k0);
    if (g.vec) {
#pragma unroll
      for (int s = 0; s < NP / 4; ++s) {
        const int f = 4 * (tid + 256 * s), kk = f / R;
        float4 u = float4{0.0f, 0.0f, 0.0f, 0.0f};
        if (kk < kn) u = *reinterpret_cast<const float4*>(W + (int64_t)k0 * R + f);
        pre[4 * s] = u.x; pre[4 * s + 1] = u.y; pre[4 * s + 2] = u.z; pre[4 * s + 3] = u.w;
      }
    } else {
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        const int q = tid + 256 * s, kk = q / R, j = q % R;
        pre[s] = j < g.r && kk < kn ? W[(int64_t)(k0 + kk) * g.r + j] : 0.0f;
      }
    }
  };
  auto put = [&](const float (&pre)[NP]) {
    if (g.vec) {
#pragma unroll
      for (int s = 0; s < NP / 4; ++s) {
        const int f = 4 * (tid + 256 * s), kk = f / R, j = f % R;
#pragma unroll
        for (int c = 0; c < 4; ++c) sW[(j + c) * kTile + (kk & 7) * 64 + (kk >> 3)] = pre[4 * s + c];
      }
    } else {
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        const int q = tid + 256 * s, kk = q / R, j = q % R;
        sW[j * kTile + (kk & 7) * 64 + (kk >> 3)] = pre[s];
      }
    }
  };

  float z[RW][R];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) z[i][j] = 0.0f;

  float pre[NP];
  if (tr >= 0) {  // pass 1: z = V^T h
    fetch(g.V, 0, pre);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t * kTile >= K) break;
      __syncthreads();  // the previous tile is no longer read
      put(pre);
      if (t + 1 < NT && (t + 1) * kTile < K) fetch(g.V, t + 1, pre);
      __syncthreads();
      if (t * kTile + 8 * lane < K) {
        float hv[RW][8];
#pragma unroll
        for (int i = 0; i < RW; ++i) elems(t, i, hv[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v[R];
#pragma unroll
          for (int j = 0; j < R; ++j) v[j] = sW[j * kTile + e * 64 + lane];
#pragma unroll
          for (int i = 0; i < RW; ++i)
            if (i < nr)
#pragma unroll
              for (int j = 0; j < R; ++j) z[i][j] = fmaf(v[j], hv[i][e], z[i][j]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int j = 0; j < R; ++j) {
        float v = z[i][j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        z[i][j] = v;
      }
  }

  // pass 2: the adapted rows (copied rows unchanged)
  const float eta = tr >= 0 ? g.eta.c[tr] : 0.0f;
  float pa[2], pb[2];
  auto fetch_ab = [&](int t) {
    const int k0 = t * kTile, kn = min(kTile, K - k0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q = tid + 256 * s;
      pa[s] = q < kn ? g.a[(int64_t)tr * K + k0 + q] : 0.0f;
      pb[s] = q < kn ? g.b[(int64_t)tr * K + k0 + q] : 0.0f;
    }
  };
  if (tr >= 0) {
    fetch(g.U, 0, pre);
    fetch_ab(0);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t * kTile >= K) break;
    if (tr >= 0) {
      __syncthreads();
      put(pre);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int q = tid + 256 * s;
        sA[(q & 7) * 64 + (q >> 3)] = pa[s];
        sB[(q & 7) * 64 + (q >> 3)] = pb[s];
      }
      if (t + 1 < NT && (t + 1) * kTile < K) {
        fetch(g.U, t + 1, pre);
        fetch_ab(t + 1);
      }
      __syncthreads();
    }
    const int k = t * kTile + 8 * lane;
    if (k >= K || nr == 0) continue;
    float hv[RW][8];
#pragma unroll
    for (int i = 0; i < RW; ++i) elems(t, i, hv[i]);
    if (tr >= 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float u[R];
#pragma unroll
        for (int j = 0; j < R; ++j) u[j] = sW[j * kTile + e * 64 + lane];
        const float ak = sA[e * 64 + lane], bk = sB[e * 64 + lane];
#pragma unroll
        for (int i = 0; i < RW; ++i) {
          float s = 0.0f;
#pragma unroll
          for (int j = 0; j < R; ++j) s = fmaf(u[j], z[i][j], s);
          hv[i][e] = fmaf(eta, s, fmaf(ak, hv[i][e], bk));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i)
      if (i < nr) store8(g, r0 + i, k, hv[i]);
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
  const int64_t nblk = (rows + rows_per_tr - 1) / rows_per_tr;
  if (nblk - 1 + first >= ntr || nblk > 65535) return hipErrorInvalidValue;
  const int64_t per_blk = min(rows_per_tr, rows);
  const int R = r <= 8 ? 8 : 16;
  const int nt = (K + kTile - 1) / kTile;
  // the resident form for rank 8 up to 5 tiles of K, where it keeps two
  // waves per SIMD; other shapes take the general form
  if (R == 8 && nt <= kResTiles) {
    using Fn = void (*)(CtaArgs);
    static const Fn res[2][kResTiles] = {
        {cta_resident_kernel<8, 1, false>, cta_resident_kernel<8, 2, false>, cta_resident_kernel<8, 3, false>,
         cta_resident_kernel<8, 4, false>, cta_resident_kernel<8, 5, false>},
        {cta_resident_kernel<8, 1, true>, cta_resident_kernel<8, 2, true>, cta_resident_kernel<8, 3, true>,
         cta_resident_kernel<8, 4, true>, cta_resident_kernel<8, 5, true>}};
    const int wg_rows = bf16 ? 16 : 8;  // 4 waves of 4 bf16 or 2 fp32 rows
    const int64_t gx = (per_blk + wg_rows - 1) / wg_rows;
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    g.vec = r == R && (reinterpret_cast<uintptr_t>(U) & 15) == 0 && (reinterpret_cast<uintptr_t>(V) & 15) == 0;
    hipLaunchKernelGGL(res[bf16 ? 1 : 0][nt - 1], dim3((unsigned)gx, (unsigned)nblk), dim3(256), 0, s, g);
    return hipGetLastError();
  }
  const int64_t gx = (per_blk + kRows - 1) / kRows;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)nblk);
  if (R == 8)
    hipLaunchKernelGGL(cta_kernel<8>, grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(cta_kernel<16>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

int cta_max_rank() { return kMaxRank; }

}  // namespace loopq
