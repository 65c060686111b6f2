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

// LDS strides (elements) of P1, P2 and the X rows: P rows padded to 16 mod
// 32 and X rows to 2 mod 32 so the 16 lanes of an MFMA operand read fall on
// distinct banks.  For compile-time factor shapes the kernel uses these
// constants (every LDS offset then folds into the instruction); the host plan
// uses the same values for those shapes.
constexpr int stride_to(int n, int rem) { return n + ((rem - n) % 32 + 32) % 32; }
constexpr int p_stride(int n) { return n <= 16 ? 16 : stride_to(n, 16); }
constexpr int x_stride(int n2) { return stride_to(n2, 2); }
template <int N1, int N2>
struct XStrides {
  static constexpr int sp1 = N1 > 0 ? p_stride(N1) : 0;
  static constexpr int sp2 = N2 > 0 ? p_stride(N2) : 0;
  static constexpr int sx = N2 > 0 ? x_stride(N2) : 0;
};

// Factor shapes of the Kronecker transforms in use (K = 256, 2048, 5632,
// 2560, 6912, and a 32-wide test shape), each with its rows per chunk and the
// most work items a wave then takes.  Chunk sizes make rows * ceil(n2 / 16)
// items a multiple of the 4 waves where that fits (3 items per wave for
// (64, 88) at 2 rows; (64, 108) has 7 per row and stays at one row).
#define LOOPQ_SHAPES(X) \
  X(16, 16, 16, 4)      \
  X(32, 64, 4, 4)       \
  X(64, 88, 2, 3)       \
  X(40, 64, 3, 3)       \
  X(64, 108, 1, 2)      \
  X(4, 8, 16, 4)

}  // namespace loopq
