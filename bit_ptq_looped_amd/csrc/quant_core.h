// Device helpers shared by the activation quantizer (quant_act.hip) and the
// few-row decode kernel (decode.hip): the Eq.(4) group quantizer arithmetic,
// the LDS strides of the Kronecker factors and the factor shapes compiled
// in.  Both translation units quantize with exactly this code, so they
// produce the same codes from the same x~.
#pragma once

#include "loopq_internal.h"

namespace loopq {

typedef float v4f __attribute__((ext_vector_type(4)));

// v if mask is all ones, +0 if it is zero (bitwise, so no branch is formed)
__device__ __forceinline__ float masked(float v, uint32_t mask) {
  return __uint_as_float(__float_as_uint(v) & mask);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// max over the 8 consecutive lanes of a group: quad swaps 1 and 2, then the
// half-row mirror pairs each lane with one of the other quad (DPP, no LDS)
__device__ __forceinline__ float group8_max(float v) {
  int b = __float_as_int(v);
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x141, 0xF, 0xF, false))));
  return __int_as_float(b);
}

// The Eq.(4) step of a group with absolute maximum amax, clip c and
// rq = fl32(1 / qmax): base = fl32(amax / qmax) is formed as
// q0 = fl32(amax * rq), then one FMA correction q0 + (amax - q0 qmax) rq; for
// qmax = 7 and 127 this equals the correctly rounded quotient for every
// finite non-negative fp32 amax (checked exhaustively over all of them).
// s = fl32(c * base).
__device__ __forceinline__ float step_of(float amax, float clip, float qmaxf, float rq) {
  const float q0 = amax * rq;
  const float base = __builtin_fmaf(__builtin_fmaf(-q0, qmaxf, amax), rq, q0);  // = fl32(amax / qmax)
  return clip * base;  // one fp32 product
}

// The codes of 4 elements on step s, packed as int8 bytes:
// clamp(rint(fl32(x / s)), -qmax, qmax), 0 when s == 0.  The quotient is
// formed as p = fl32(x * r) with r the hardware reciprocal of s (within
// 1 ulp): |p - x/s| < 3 * 2^-24 |x/s| and |fl32(x/s) - x/s| <= 2^-24 |x/s|,
// so below the clamp (|x/s| < 128) p and fl32(x/s) differ by less than
// 2^-15.  The distance d = |x * r - rint(p)| is taken with one FMA (within
// 2^-17 of |p - rint(p)|); if d <= 0.5 - 2^-14 then fl32(x/s) lies within
// 0.5 - 3 * 2^-17 of rint(p) and rounds to the same integer.  Runs with a
// larger d, and any run whose r is not a positive finite normal-range value
// (s outside about [2^-126, 2^126]), are redone with the correctly rounded
// division.  Above the clamp both sides saturate alike.
__device__ __forceinline__ uint32_t codes4(float4 v, float s, float qmaxf) {
  if (!(s > 0.0f)) return 0u;
  const float r = __builtin_amdgcn_rcpf(s);
  const float e[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed = 0u;
  bool exact = !(r > 1.0e-37f && r < 1.0e37f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = e[i] * r;
    const float rq_ = __builtin_rintf(p);
    // runs above the clamp may take the exact path too; both sides clamp
    exact |= fabsf(__builtin_fmaf(e[i], r, -rq_)) > 0.5f - 6.103515625e-05f;
    const float q = __builtin_amdgcn_fmed3f(rq_, -qmaxf, qmaxf);
    packed |= (uint32_t)((int)q & 0xff) << (8 * i);
  }
  if (exact) {  // rare: near a rounding boundary, or s extreme
    packed = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float q = __builtin_rintf(e[i] / s);  // ties to even
      q = fminf(fmaxf(q, -qmaxf), qmaxf);
      packed |= (uint32_t)((int)q & 0xff) << (8 * i);
    }
  }
  return packed;
}

// Quantize 4 consecutive elements of one 32-group whose 8 lanes are
// consecutive in the wave (lane % 8 = position of the 4-element run).
// Returns the 4 codes packed as int8 bytes; writes the step to *step.
__device__ __forceinline__ uint32_t quantize4(float4 v, float clip, float qmaxf, float rq, float* step) {
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = group8_max(amax);
  const float s = step_of(amax, clip, qmaxf, rq);
  *step = s;
  return codes4(v, s, qmaxf);
}

// LDS strides (elements) of P1, P2 and the X rows, so the lanes of an MFMA
// operand read fall on distinct banks: stage 1 reads P2 rows b, b + 1, b + 2,
// b + 3 (one per 16-lane group), so P2 rows are padded to 16 mod 32; stage 2
// reads P1 rows a, a + 4, a + 8, a + 12 (the rows the stage-1 result holds
// per lane group), so P1 rows are padded to 4 mod 16 (4 rows = 16 banks
// apart); X rows to 2 mod 32.  For compile-time factor shapes the kernel uses
// these constants (every LDS offset then folds into the instruction); the
// host plan uses the same values for those shapes.
constexpr int stride_to(int n, int rem) { return n + ((rem - n) % 32 + 32) % 32; }
constexpr int p_stride(int n) { return n <= 16 ? 16 : stride_to(n, 16); }
constexpr int p1_stride(int n) { return n + ((4 - n) % 16 + 16) % 16; }
constexpr int x_stride(int n2) { return stride_to(n2, 2); }
template <int N1, int N2>
struct XStrides {
  static constexpr int sp1 = N1 > 0 ? p1_stride(N1) : 0;
  static constexpr int sp2 = N2 > 0 ? p_stride(N2) : 0;
  static constexpr int sx = N2 > 0 ? x_stride(N2) : 0;
};

// Ends a branch whose MFMA accumulators are read only after the branch has
// joined another one.  The compiler's hazard count across such a join has
// come out short on gfx950 (the last element of a 16x16x4 f32 accumulator
// read 8 wait states after its MFMA, where straight-line code gets 10, and
// seen without that MFMA's contribution); 16 wait states of the branch's own
// make the read safe whatever the count.
__device__ __forceinline__ void mfma_settle_before_join() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// Stage 1 of the transform on the bf16 MFMA, for bf16 inputs: T = X * P2 with
// X exactly bf16 and P2 split into three bf16 planes whose sum is P2 exactly
// (hi = P2 truncated to bf16, mid = the remainder truncated, lo = what is
// left, which has at most 8 significant bits).  Every product of an X value
// and a plane value is exact in fp32; only the fp32 accumulation rounds, as
// on the fp32 MFMA, so x~ keeps the fp32-class bound.
//
// LDS layouts (bf16 elements): P2 planes transposed, plane p, column j < n2,
// K index b at p * plane + j * sb + b; X rows i of the n1 x n2 grid at i * sb,
// K index b.  K indices b >= n2 of P2 and of X are zero.  A column tile that
// runs past n2 reads column n2 - 1 in place of the missing ones (those
// columns of T are never used).  The row stride sb = kb + 8 puts the 16 rows
// one 16-byte read per lane touches on distinct LDS banks.
// ---------------------------------------------------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int N2>
struct BfLayout {
  static constexpr int kb = (N2 + 31) / 32 * 32;  // K extent, in steps of 32
  static constexpr int jp = (N2 + 15) / 16 * 16;  // column extent, in tiles of 16
  static constexpr int sb = kb + 8;               // row stride (elements)
  static constexpr int plane = N2 * sb;           // elements per plane (columns j < n2)
  static constexpr int p2_bytes = 3 * plane * 2;
};

// v = hi + mid + lo exactly, each the bits of a bf16 (truncations)
__device__ __forceinline__ void split3_bf16(float v, uint32_t* h, uint32_t* m, uint32_t* l) {
  const uint32_t hu = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(hu);  // exact: the low 16 mantissa bits of v
  const uint32_t mu = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mu);  // exact, at most 8 significant bits
  *h = hu >> 16;
  *m = mu >> 16;
  *l = __float_as_uint(r2) >> 16;
}

// NI items of T = X * P2, each one 16-column tile of T over NRT consecutive
// 16-row tiles starting at tile rt0[ii].  Item ii reads the X grid whose row
// i is at xgrid[ii] + i * sb (rows >= N1 read as zero) and the planes of the
// lane's column at pcol[ii] (plane p at + p * plane; the caller points lanes
// past n2 at column n2 - 1).  Lane l takes A row l % 16, B column l % 16 and K slots
// 8 (l / 16) .. + 7 of each step of 32; result element e of lane l is T row
// 16 (rt0 + q) + 4 (l / 16) + e, column l % 16 (the fp32 MFMA's layout).
// Every tile accumulates in the same order (K steps, then planes hi, mid,
// lo), so a tile's value does not depend on which kernel or wave forms it.
// SA: all items share item 0's X grid and row tiles, whose A operands are
// then read once per step for all of them.
template <int N1, int N2, int NI, int NRT, bool SA = false>
__device__ __forceinline__ void stage1_bf16(const uint16_t* const (&xgrid)[NI], const int (&rt0)[NI],
                                            const uint16_t* const (&pcol)[NI], int plane, int li, int lk,
                                            v4f (&T)[NI][NRT]) {
  using L = BfLayout<N2>;
  constexpr int NA = SA ? 1 : NI;
#pragma unroll
  for (int ks = 0; ks < L::kb / 32; ++ks) {
    v4u a[NA][NRT], b[NI][3];
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
#pragma unroll
      for (int p = 0; p < 3; ++p)
        b[ii][p] = *reinterpret_cast<const v4u*>(pcol[ii] + p * plane + 32 * ks + 8 * lk);
    }
#pragma unroll
    for (int ia = 0; ia < NA; ++ia) {
#pragma unroll
      for (int q = 0; q < NRT; ++q) {
        const int i = (rt0[ia] + q) * 16 + li;
        a[ia][q] = *reinterpret_cast<const v4u*>(xgrid[ia] + (i < N1 ? i : N1 - 1) * L::sb + 32 * ks + 8 * lk);
        if (i >= N1) a[ia][q] = v4u{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int ii = 0; ii < NI; ++ii)
#pragma unroll
        for (int q = 0; q < NRT; ++q)
          T[ii][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[SA ? 0 : ii][q]),
                                                           __builtin_bit_cast(v8bf, b[ii][p]), T[ii][q], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Stage 2 of the transform on the bf16 MFMA, for bf16 inputs: x~ = P1^T * T,
// with T (the fp32 stage-1 result) and P1 each split into three exact bf16
// planes (split3_bf16), and the six plane products of order <= 2 taken (hi,
// mid, lo = 0, 1, 2; the three dropped ones are below 2^-20 of |P1| |T|).
// Per 16x16 tile of x~ and step q of 32 reduction indices the six MFMAs run
// in one fixed order, smallest first: (P1 lo, T hi), (mid, mid), (hi, lo),
// (mid, hi), (hi, mid), (hi, hi); every kernel takes the steps in order, so a
// tile's value does not depend on which kernel or wave forms it.
//
// Reduction order.  The fp32 stage-1 result gives lane l the T rows
// 16 rt + 4 (l / 16) + e in element e of tile rt; step q of the bf16 MFMA
// wants 8 consecutive K slots 8 (l / 16) .. + 7 per lane.  Slot 8 g + 4 h + e
// of step q takes T row a = 32 q + 16 h + 4 g + e, so a lane's slots are
// tile 2q's elements then tile 2q + 1's, straight from its registers; the P1
// planes are stored with their reduction index in the same order.
//
// P1 plane layout (bf16): plane p, output row i < 16 NRT, slot a' at
// p * plane + i * sb + a' (a' = slot of row a; zeros for a, i >= n1).
// ---------------------------------------------------------------------------
template <int N1>
struct P1Layout {
  static constexpr int rows = (N1 + 15) / 16 * 16;  // output rows, in tiles of 16
  static constexpr int ka = (N1 + 31) / 32 * 32;    // reduction extent, in steps of 32
  static constexpr int sb = ka + 8;                 // row stride (elements): spreads the banks
  static constexpr int plane = rows * sb;
  static constexpr int bytes = 3 * plane * 2;
};
// slot of reduction index a, and back
__host__ __device__ constexpr int p1_slot(int a) {
  return (a & ~31) | (((a >> 2) & 3) << 3) | (((a >> 4) & 1) << 2) | (a & 3);
}
__host__ __device__ constexpr int p1_row_of_slot(int s) {
  return (s & ~31) | (((s >> 2) & 1) << 4) | (((s >> 3) & 3) << 2) | (s & 3);
}

// The planes of split3_bf16 are the upper halves of fp32 words: hi of v, mid
// of r1 = v - hi, lo of r2 = r1 - mid (each difference exact).  top_halves
// packs the upper halves of two words (the first in the low half) in one
// byte permute; minus_top is the exact difference that uncovers the next
// plane.
__device__ __forceinline__ uint32_t top_halves(float lo_slot, float hi_slot) {
  return __builtin_amdgcn_perm(__float_as_uint(hi_slot), __float_as_uint(lo_slot), 0x07060302u);
}
__device__ __forceinline__ float minus_top(float v) {
  return v - __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
}

// the three bf16 planes of 8 fp32 values, packed two per register (element
// 2k in the low half of register k): split3_bf16 of each value
__device__ __forceinline__ void planes8(const float (&v)[8], v4u (&b)[3]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float v0 = v[2 * k], v1 = v[2 * k + 1];
    const float m0 = minus_top(v0), m1 = minus_top(v1);
    b[0][k] = top_halves(v0, v1);
    b[1][k] = top_halves(m0, m1);
    b[2][k] = top_halves(minus_top(m0), minus_top(m1));
  }
}

// A operands of tile it, step q (lane's row 16 it + li, slots 32 q + 8 lk ..)
template <int N1>
__device__ __forceinline__ void p1_planes_at(const uint16_t* sP1b, int it, int q, int li, int lk, v4u (&a)[3]) {
  using L = P1Layout<N1>;
#pragma unroll
  for (int p = 0; p < 3; ++p)
    a[p] = *reinterpret_cast<const v4u*>(sP1b + p * L::plane + (it * 16 + li) * L::sb + 32 * q + 8 * lk);
}

// Product k = 0..5 of a tile and step multiplies P1 plane s2_pa(k) by T plane
// s2_pb(k): (2,0), (1,1), (0,2), (1,0), (0,1), (0,0).  Callers run k outermost
// across their independent tiles, so every tile takes the same sequence.
__host__ __device__ constexpr int s2_pa(int k) { return k == 0 ? 2 : (k == 1 || k == 3) ? 1 : 0; }
__host__ __device__ constexpr int s2_pb(int k) { return k == 0 ? 0 : (k == 1 || k == 4) ? 1 : k == 2 ? 2 : 0; }
__device__ __forceinline__ v4f s2_mm(const v4u& a, const v4u& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// The P1 planes from fp32 P1 ([n1][n1], row a, column i) in global memory,
// threads t, t + NT, ...: two slots (a pair of consecutive reduction rows)
// per 32-bit store and plane; loads first.
template <int N1, int NT>
__device__ __forceinline__ void stage_p1_planes(const float* __restrict__ P1, uint16_t* dst, int t) {
  using L = P1Layout<N1>;
  constexpr int NP = L::rows * (L::ka / 2);
  constexpr int U = (NP + NT - 1) / NT;
  float v[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = t + u * NT;
    const int i = idx / (L::ka / 2), s = 2 * (idx - i * (L::ka / 2));
    const int a = p1_row_of_slot(s);
    v[u][0] = (idx < NP && i < N1 && a < N1) ? P1[a * N1 + i] : 0.0f;
    v[u][1] = (idx < NP && i < N1 && a + 1 < N1) ? P1[(a + 1) * N1 + i] : 0.0f;
  }
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = t + u * NT;
    if (idx < NP) {
      const int i = idx / (L::ka / 2), s = 2 * (idx - i * (L::ka / 2));
      uint32_t h0, m0, l0, h1, m1, l1;
      split3_bf16(v[u][0], &h0, &m0, &l0);
      split3_bf16(v[u][1], &h1, &m1, &l1);
      const int o = (i * L::sb + s) >> 1;  // sb and s are even
      d[o] = h0 | (h1 << 16);
      d[o + L::plane / 2] = m0 | (m1 << 16);
      d[o + L::plane] = l0 | (l1 << 16);
    }
  }
}

// Stage the planes of columns j0 .. j0 + nj - 1 of P2 (fp32 [N2][N2] in
// global memory) into dst (plane stride nj * sb, local column j - j0), zeros
// outside the factor; threads tid, tid + nthr, ...  Loads are issued in
// batches of 8 before their stores (coalesced along j).
template <int N2>
__device__ __forceinline__ void stage_p2_planes(const float* __restrict__ P2, uint16_t* dst, int j0, int nj, int tid,
                                                int nthr) {
  using L = BfLayout<N2>;
  const int n = nj * L::kb;
  const int pl = nj * L::sb;
  for (int base = tid; base < n; base += 8 * nthr) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * nthr;
      const int b = idx / nj, j = j0 + (idx - (idx / nj) * nj);
      v[u] = (idx < n && b < N2 && j < N2) ? P2[b * N2 + j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * nthr;
      if (idx < n) {
        const int b = idx / nj, jj = idx - b * nj;
        uint32_t h, m, l;
        split3_bf16(v[u], &h, &m, &l);
        dst[jj * L::sb + b] = (uint16_t)h;
        dst[pl + jj * L::sb + b] = (uint16_t)m;
        dst[2 * pl + jj * L::sb + b] = (uint16_t)l;
      }
    }
  }
}

// Factor shapes of the Kronecker transforms in use (K = 256, 2048, 5632,
// 2560, 6912, and a 32-wide test shape), each with its rows per chunk, the
// most work items a wave then takes, and the inputs for which the transform
// kernel runs them in its two-role form (512 threads, MFMA stages beside the
// quantizer) rather than as 256 threads doing one phase at a time: bit 0 for
// bf16 input, bit 1 for fp32 input (set where it measured faster: the shapes
// whose one-phase form fits one work-group per CU, and the small ones; (32,
// 64) and (40, 64) run two one-phase work-groups per CU, which overlap their
// phases as well).  Chunk sizes
// make rows * ceil(n2 / 16) items a multiple of the 4 stage waves where that
// fits (3 items per wave for (64, 88) at 2 rows; (64, 108) has 7 per row and
// stays at one row).
#define LOOPQ_SHAPES(X) \
  X(16, 16, 16, 4, 3)   \
  X(32, 64, 4, 4, 0)    \
  X(64, 88, 2, 3, 3)    \
  X(40, 64, 3, 3, 0)    \
  X(64, 108, 1, 2, 3)   \
  X(4, 8, 16, 4, 3)

}  // namespace loopq
