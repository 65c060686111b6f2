// Few-row (decode) form of the quantized linear (gfx950): for at most 16
// token rows, the Kronecker transform, the Eq.(4) group quantizer with the
// loop's LAS clip, and the integer product with per-group rescale
//
//   y[m][n] = sum_j s_a[m][j] * s_w[n][32j / group_w] * d[m][n][j],
//   d[m][n][j] = sum_{k in group j} q_a[m][k] * q_w[n][k]   (exact int32)
//
// in one launch.  Method: Eq.(4) ("paper_specification.yaml",
// lq1_quantization), LAS (loopq_components.las, lq2), the shared Kronecker
// transform (lq3); the product is the integer form of the reproduction's
// simulated quantize-dequantize linear (README of the LoopQ reproduction,
// "Protocol").
//
// With a handful of rows the call is bound by streaming the packed INT4
// weights once and by latency.  Each work-group owns one block of CPW output
// columns over all of K and needs no other work-group: it issues the loads of
// its first weight slice into registers, forms the rows' codes while they
// arrive, then dots, with the next slice's loads in flight.
//   * Transform instances compute x~ of every row themselves (the same
//     operands and MFMA order as the chunked transform kernel, so the same x~
//     bit for bit), quantize each row into LDS with the quantizer the other
//     kernels use, and keep all rows' codes in LDS.  Every work-group repeats
//     the transform, so its latency is the call's: these instances run 8
//     waves (4 for K = 6912), which split the factor staging, the MFMA tiles
//     and the quantizer between them; the host takes this form only while the
//     transform costs about as much as the weight fetch it overlaps.
//   * Other instances quantize x (no transform) or copy canonical codes for
//     all rows and all of K into LDS (one weight slice at a time if that does
//     not fit), with every thread's loads of the next round in flight while
//     it quantizes the current one.
// Group dots: thread (column c, lane group gq) takes groups gq, gq + GL, ...
// of each slice, unpacks the column's 32 nibbles and dots them with every
// row's codes on V_DOT4_I32_I8 (exact), folding with fl32(s_w * s_a); a
// column's partial sums are added by a butterfly across the lanes of each
// wave that hold it, then in wave order through LDS, so y is deterministic.
#include "loopq_internal.h"
#include "quant_core.h"

#include <cstring>
#include <type_traits>

namespace loopq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// A work-group of NTH threads (NW = NTH / 64 waves) owns CPW consecutive
// output columns (8, 16 or 32, so that a call has about as many work-groups
// as the chip has CUs) over all of K.  Each thread holds KP groups of packed
// weights per slice in flight (at most 8, 128 bytes): in the VALU form thread
// (column c, lane group gq) takes groups gq + GL i (i < KP) of a slice; in the
// MFMA form a wave takes groups wave + NW i of a slice for all 16-column
// halves of the work-group's columns.  Where K is compiled in, KP is the
// fewest slots that cover K in one slice.
constexpr int kPer = 8;  // most groups of a slice per thread (VALU form)
template <int CPW, int NTH = 256, int KP = kPer>
struct Cols {
  static constexpr int NW = NTH / 64;                  // waves
  static constexpr int GL = NTH / CPW;                 // lane groups per column (VALU form)
  static constexpr int kSlice = KP * GL;               // groups per weight slice
  static constexpr int NH = CPW >= 16 ? CPW / 16 : 1;  // 16-column halves (MFMA form)
  static constexpr int kMPer = kSlice / NW;            // groups per wave and slice (MFMA form)
  static_assert(kSlice % NW == 0, "a slice splits evenly over the waves");
};
// slots per thread for a compiled-in K of ga groups
constexpr int slots_for(int ga, int gl) { return (ga + gl - 1) / gl < kPer ? (ga + gl - 1) / gl : kPer; }
constexpr int kLdsBudget = 160 * 1024;

struct DecodeArgs {
  const void* x;          // [R][K] fp32 or bf16 (in_codes == 0)
  int bf16;
  const int8_t* a_codes;  // canonical codes [R][K] (in_codes == 1)
  const float* a_steps;   // row-major steps [R][K/32] (in_codes == 1, mode 0)
  int in_codes;
  const float* P1;        // factors (transform instances)
  const float* P2;
  int R, K, N;
  ClipTable clips;
  int rows_per_clip;
  int qmax;
  const uint8_t* w;       // packed nibbles
  const __half* sw;       // packed steps [Npad/32][Gw][32] (mode 0)
  int gshift;
  float* y;               // [R][N] (mode 0)
  int32_t* dots;          // [R][N][K/32] (mode 1)
  int whole;              // non-transform instances: all codes fit LDS at once
  int wide_codes;         // canonical codes 16-byte aligned (copied 16 at a time)
  int8_t* codes_out;      // nullable: the codes formed from x, canonical [R][K]
  float* steps_out;       // with codes_out: their steps, row-major [R][K/32]
};

// The codes and steps of groups [j0, j0 + G) of every row, held in LDS (codes
// of group j0 + gi of row m at sA + m * a_ld + gi * 32, its step at
// sS[m * s_ld + gi]), written to the canonical output.  Every work-group holds
// the same codes, so the work-groups share the writes out between them.
template <int NTH>
__device__ __forceinline__ void dump_codes(const DecodeArgs& g, int j0, int G, const int8_t* sA, int a_ld,
                                           const float* sS, int s_ld) {
  const int K = g.K, Ga = K >> 5;
  const int stride = (int)gridDim.x * NTH;
  const int n16 = g.R * G * 2;  // 16-code pieces
  for (int q = (int)blockIdx.x * NTH + (int)threadIdx.x; q < n16; q += stride) {
    const int m = q / (2 * G), rem = q - m * 2 * G;
    *reinterpret_cast<uint4*>(g.codes_out + (int64_t)m * K + (j0 + (rem >> 1)) * 32 + (rem & 1) * 16) =
        *reinterpret_cast<const uint4*>(sA + m * a_ld + (rem >> 1) * 32 + (rem & 1) * 16);
  }
  for (int q = (int)blockIdx.x * NTH + (int)threadIdx.x; q < g.R * G; q += stride) {
    const int m = q / G;
    g.steps_out[(int64_t)m * Ga + j0 + (q - m * G)] = sS[m * s_ld + q - m * G];
  }
}

// 8 biased nibbles (q + 8) per dword -> 16 int8 codes, in K order
__device__ __forceinline__ v4i unpack16(uint2 p) {
  v4i r;
  r[0] = (int)(((p.x & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[1] = (int)((((p.x >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[2] = (int)(((p.y & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  r[3] = (int)((((p.y >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
  return r;
}

// The weights of one slice held by one thread: groups sl * kSlice + gq + GL i.
template <int KP>
struct WSlice {
  uint2 lo[KP], hi[KP];
  float s[KP];
};

// Packed weights are loaded non-temporal: a call reads each weight line once,
// and the hint leaves the caches to the factors, rows and codes that every
// call reads again (decode 3-4% faster per loop-step; the adapter recurrence
// at one row, whose weights stay in the last-level cache across its loops,
// 3% slower).
__device__ __forceinline__ uint2 weight_load2(const uint8_t* p) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return uint2{v.x, v.y};
}

// Load a thread's part of slice `sl`; groups past Ga re-read group Ga - 1
// and are not used.
template <int CPW, int MODE, int NTH, int KP>
__device__ __forceinline__ void load_slice(const DecodeArgs& g, int cb, int sl, int c, int gq,
                                           WSlice<KP>& ws) {
  using C = Cols<CPW, NTH, KP>;
  const int Ga = g.K >> 5;
  const int Gw = (Ga + (1 << g.gshift) - 1) >> g.gshift;
  const int n = cb * CPW + c;  // padded column: block n / 32, column n % 32 of it
  const int nb = n >> 5, cc = n & 31;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int j = min(sl * C::kSlice + gq + C::GL * i, Ga - 1);
    const uint8_t* blk = g.w + ((int64_t)nb * Ga + j) * kBlockBytes + cc * 8;
    ws.lo[i] = weight_load2(blk);        // K 32 j + 0..15
    ws.hi[i] = weight_load2(blk + 256);  // K 32 j + 16..31
    ws.s[i] = MODE == 0 ? __half2float(g.sw[((int64_t)nb * Gw + (j >> g.gshift)) * 32 + step_slot(cc)]) : 0.0f;
  }
}

// Dots of the thread's groups of slice `sl` that lie in [jlo, jhi) with every
// row's codes: codes of group j of row m at sA + m * a_ld + (j - a_j0) * 32
// (bytes), its step at sS[m * s_ld + j - a_j0].
template <int CPW, int RM, int MODE, int NTH, int KP>
__device__ __forceinline__ void dot_slice(const DecodeArgs& g, int cb, int sl, int c, int gq,
                                          const WSlice<KP>& ws, int jlo, int jhi, const int8_t* sA,
                                          int a_ld, int a_j0, const float* sS, int s_ld,
                                          float (&acc)[RM]) {
  using C = Cols<CPW, NTH, KP>;
  const int Ga = g.K >> 5;
  const int n = cb * CPW + c;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int j = sl * C::kSlice + gq + C::GL * i;
    if (j >= jlo && j < jhi && j < Ga) {
      const v4i w0 = unpack16(ws.lo[i]);
      const v4i w1 = unpack16(ws.hi[i]);
#pragma unroll
      for (int m = 0; m < RM; ++m) {
        if (m < g.R) {
          const v4i* ap = reinterpret_cast<const v4i*>(sA + m * a_ld + (j - a_j0) * 32);
          const v4i a0 = ap[0], a1 = ap[1];
          int d = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) d = __builtin_amdgcn_sdot4(a0[e], w0[e], d, false);
#pragma unroll
          for (int e = 0; e < 4; ++e) d = __builtin_amdgcn_sdot4(a1[e], w1[e], d, false);
          if (MODE == 0) {
            const float coef = ws.s[i] * sS[m * s_ld + j - a_j0];  // fl32(s_w * s_a)
            acc[m] = __builtin_fmaf((float)d, coef, acc[m]);
          } else if (n < g.N) {
            g.dots[((int64_t)m * g.N + n) * Ga + j] = d;
          }
        }
      }
    }
  }
}

// ---- MFMA form of the dots (up to 16 rows): V_MFMA_I32_16X16X32_I8 takes
// 16 rows (activation codes, rows >= R zero) x one 32-element group x 16
// weight columns and returns the 256 exact int32 dots.  Operand lanes: A row
// l % 16 and B column l % 16 hold K 8 (l / 16) .. + 7 of the group as 8 bytes;
// result element e of lane l is row 4 (l / 16) + e, column l % 16.  A wave
// takes groups wave, wave + 4, ... of a slice and both 16-column halves of
// the block; its nibbles for one (half, group) are one dword of the packed
// layout (K-half (l / 16) / 2, run (l / 16) % 2).

// The weights of one slice held by one lane: groups sl * kSlice + wave + NW i,
// for each 16-column half of the work-group's columns.
template <int CPW, int NTH, int KP>
struct MSlice {
  using C = Cols<CPW, NTH, KP>;
  uint32_t w[C::kMPer][C::NH];  // packed nibbles, [group][column half]
  float s[C::kMPer][C::NH];     // fp16 steps of the lane's column
};

template <int CPW, int MODE, int NTH, int KP>
__device__ __forceinline__ void load_mslice(const DecodeArgs& g, int cb, int sl, MSlice<CPW, NTH, KP>& ms) {
  using C = Cols<CPW, NTH, KP>;
  const int Ga = g.K >> 5;
  const int Gw = (Ga + (1 << g.gshift) - 1) >> g.gshift;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4;
#pragma unroll
  for (int i = 0; i < C::kMPer; ++i) {
    const int j = min(sl * C::kSlice + wave + C::NW * i, Ga - 1);  // past Ga: re-read, unused
#pragma unroll
    for (int tt = 0; tt < C::NH; ++tt) {
      const int n = cb * CPW + tt * 16 + (lane & 15);
      const int nb = n >> 5, cc = n & 31;
      ms.w[i][tt] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(
          g.w + ((int64_t)nb * Ga + j) * kBlockBytes + (q >> 1) * 256 + cc * 8 + (q & 1) * 4));
      ms.s[i][tt] = MODE == 0 ? __half2float(g.sw[((int64_t)nb * Gw + (j >> g.gshift)) * 32 + step_slot(cc)]) : 0.0f;
    }
  }
}

// 8 biased nibbles (q + 8) of one dword -> 8 int8 codes in K order (low
// nibbles first), as the 64-bit MFMA operand
__device__ __forceinline__ long unpack8(uint32_t p) {
  const uint32_t lo = ((p & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
  const uint32_t hi = (((p >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
  return (long)(((uint64_t)hi << 32) | lo);
}

// Dots of the wave's groups of slice `sl` lying in [jlo, jhi), codes and
// steps addressed as in dot_slice; acc[half][e] is row 4 (l / 16) + e of
// column half * 16 + l % 16.
template <int CPW, int MODE, int NTH, int KP>
__device__ __forceinline__ void mfma_slice(const DecodeArgs& g, int cb, int sl, const MSlice<CPW, NTH, KP>& ms,
                                           int jlo, int jhi, const int8_t* sA, int a_ld, int a_j0,
                                           const float* sS, int s_ld, float (&acc)[Cols<CPW>::NH][4]) {
  using C = Cols<CPW, NTH, KP>;
  typedef int v4i_t __attribute__((ext_vector_type(4)));
  const int Ga = g.K >> 5;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int ra = lane & 15;           // A row of the lane
  const int rac = min(ra, g.R - 1);   // rows past R read row R - 1, then zeroed
#pragma unroll
  for (int i = 0; i < C::kMPer; ++i) {
    const int j = sl * C::kSlice + wave + C::NW * i;
    if (j >= jlo && j < jhi && j < Ga) {  // wave-uniform
      long a = *reinterpret_cast<const long*>(sA + rac * a_ld + (j - a_j0) * 32 + q * 8);
      if (ra >= g.R) a = 0;
      float sa[4];
      if (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sa[e] = sS[min(4 * q + e, g.R - 1) * s_ld + j - a_j0];
      }
#pragma unroll
      for (int tt = 0; tt < C::NH; ++tt) {
        const v4i_t d = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, unpack8(ms.w[i][tt]), v4i_t{0, 0, 0, 0}, 0, 0, 0);
        if (MODE == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[tt][e] = __builtin_fmaf((float)d[e], ms.s[i][tt] * sa[e], acc[tt][e]);  // coef fl32(s_w * s_a)
        } else {
          const int n = cb * CPW + tt * 16 + (lane & 15);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 4 * q + e;
            if (m < g.R && n < g.N) g.dots[((int64_t)m * g.N + n) * Ga + j] = d[e];
          }
        }
      }
    }
  }
}

// Copy an NN x NN fp32 matrix into LDS rows of stride SP.  All of a
// thread's loads are issued before any store, so the copy costs one memory
// round trip rather than one per element.
template <int NN, int NTH = 256>
struct MatRegs {
  static constexpr int T = (NN * NN + NTH - 1) / NTH;
  float v[T];
};
template <int NN, int NTH>
__device__ __forceinline__ void stage_matrix_issue(const float* __restrict__ src, MatRegs<NN, NTH>& m) {
#pragma unroll
  for (int i = 0; i < MatRegs<NN, NTH>::T; ++i) {
    const int idx = threadIdx.x + NTH * i;
    m.v[i] = idx < NN * NN ? src[idx] : 0.0f;
  }
}
template <int NN, int SP, int NTH>
__device__ __forceinline__ void stage_matrix_commit(const MatRegs<NN, NTH>& m, float* dst) {
#pragma unroll
  for (int i = 0; i < MatRegs<NN, NTH>::T; ++i) {
    const int idx = threadIdx.x + NTH * i;
    if (idx < NN * NN) dst[(idx / NN) * SP + idx % NN] = m.v[i];
  }
}
template <int NN, int SP>
__device__ __forceinline__ void stage_matrix(const float* __restrict__ src, float* dst) {
  MatRegs<NN> m;
  stage_matrix_issue<NN>(src, m);
  stage_matrix_commit<NN, SP>(m, dst);
}

// Row r of x (K elements, bf16 or fp32) held in registers between the issue
// of its loads and their commit to LDS: bf16 in .x .y of each entry, fp32 in
// all four.
template <int K, int NTH = 256>
struct RowRegs {
  static constexpr int T = (K / 4 + NTH - 1) / NTH;
  uint4 v[T];
};
template <int K, int NTH>
__device__ __forceinline__ void x_row_issue(const DecodeArgs& g, int r, RowRegs<K, NTH>& x) {
#pragma unroll
  for (int i = 0; i < RowRegs<K, NTH>::T; ++i) {
    const int q = threadIdx.x + NTH * i;
    if (q < K / 4) {
      if (g.bf16) {
        const uint2 u = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.x) + (int64_t)r * K)[q];
        x.v[i] = uint4{u.x, u.y, 0u, 0u};
      } else {
        x.v[i] = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(g.x) + (int64_t)r * K)[q];
      }
    }
  }
}
template <int K, int N2, int SX, int NTH>
__device__ __forceinline__ void x_row_commit(const DecodeArgs& g, const RowRegs<K, NTH>& x, float* sX) {
#pragma unroll
  for (int i = 0; i < RowRegs<K, NTH>::T; ++i) {
    const int q = threadIdx.x + NTH * i;
    if (q < K / 4) {
      const int k = q * 4;
      float* dst = sX + (k / N2) * SX + k % N2;
      if (g.bf16) {
        dst[0] = bf16_bits_to_float(x.v[i].x & 0xffffu);
        dst[1] = bf16_bits_to_float(x.v[i].x >> 16);
        dst[2] = bf16_bits_to_float(x.v[i].y & 0xffffu);
        dst[3] = bf16_bits_to_float(x.v[i].y >> 16);
      } else {
        dst[0] = __uint_as_float(x.v[i].x);
        dst[1] = __uint_as_float(x.v[i].y);
        dst[2] = __uint_as_float(x.v[i].z);
        dst[3] = __uint_as_float(x.v[i].w);
      }
    }
  }
}

// Row r of x (K elements, bf16 or fp32) into LDS as the n1 x n2 grid with
// row stride SX, loads first as above.
template <int K, int N2, int SX, int NTH = 256>
__device__ __forceinline__ void stage_x_row(const DecodeArgs& g, int r, float* sX) {
  constexpr int T = (K / 4 + NTH - 1) / NTH;
  auto put = [&](int q, const float4& v) {
    const int k = q * 4;
    float* dst = sX + (k / N2) * SX + k % N2;
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  };
  if (g.bf16) {
    const uint2* src = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.x) + (int64_t)r * K);
    uint2 u[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int q = threadIdx.x + NTH * i;
      u[i] = q < K / 4 ? src[q] : uint2{0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int q = threadIdx.x + NTH * i;
      if (q < K / 4)
        put(q, float4{bf16_bits_to_float(u[i].x & 0xffffu), bf16_bits_to_float(u[i].x >> 16),
                      bf16_bits_to_float(u[i].y & 0xffffu), bf16_bits_to_float(u[i].y >> 16)});
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(g.x) + (int64_t)r * K);
    float4 v[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int q = threadIdx.x + NTH * i;
      v[i] = q < K / 4 ? src[q] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int q = threadIdx.x + NTH * i;
      if (q < K / 4) put(q, v[i]);
    }
  }
}

// LDS plan of the transform instances (bytes): P1 and P2 with bank-spread
// strides, the X row (later the x~ row), T = X * P2 for all column tiles,
// all rows' codes and steps, and the partial sums.
template <int N1, int N2>
struct XPlan {
  static constexpr int K = N1 * N2;
  static constexpr int sp1 = XStrides<N1, N2>::sp1, sp2 = XStrides<N1, N2>::sp2, sx = XStrides<N1, N2>::sx;
  static constexpr int njt = (N2 + 15) / 16;
  static constexpr int st = njt * 16;  // T row stride
  // P2 as fp32 (fp32 input) or as the bf16 planes (bf16 input); the X region
  // holds the fp32 or bf16 X grid and later the fp32 x~ row
  using BL = BfLayout<N2>;
  static constexpr int p2_bytes = N2 * sp2 * 4 > BL::p2_bytes ? N2 * sp2 * 4 : BL::p2_bytes;
  // P1 as fp32 rows (fp32 input) or as its bf16 stage-2 planes (bf16 input)
  static constexpr int p1_bytes = N1 * sp1 * 4 > P1Layout<N1>::bytes ? N1 * sp1 * 4 : P1Layout<N1>::bytes;
  static constexpr int off_p2 = (p1_bytes + 15) / 16 * 16;
  static constexpr int off_x = off_p2 + (p2_bytes + 15) / 16 * 16;
  static constexpr int x_f32 = N1 * sx * 4 > K * 4 ? N1 * sx * 4 : K * 4;
  static constexpr int x_bytes = x_f32 > N1 * BL::sb * 2 ? x_f32 : N1 * BL::sb * 2;
  static constexpr int off_t = off_x + (x_bytes + 15) / 16 * 16;
  static constexpr int off_codes = off_t + N1 * st * 4;
  static constexpr int codes_bytes(int R) { return (R * K + 15) / 16 * 16; }
  static constexpr int lds(int R, int RM, int nth) { return off_codes + codes_bytes(R) + R * (K / 32) * 4 + nth * RM * 4; }
};

// ---- transform work items (rows the one-launch form does not take): one
// work-group per (row r, 16-column tile jt of the n1 x n2 grid) writes that
// tile of x~ to xt[r][K] (fp32); the decode kernel then quantizes xt as
// plain input.  Wave w computes the stage-1 tile T[16 w ..][tile] with the
// full reduction over b, stores it in LDS, and after a barrier the stage-2
// tile x~[16 w ..][tile]; operands and MFMA order are those of the chunked
// kernel, so x~ is bitwise the same.
template <int N1, int N2>
struct ItemPlan {
  using BL = BfLayout<N2>;
  static constexpr int sp1 = XStrides<N1, N2>::sp1, sx = XStrides<N1, N2>::sx;
  static constexpr int p2_f32 = N2 * 16 * 4;          // the tile's fp32 columns [n2][16]
  static constexpr int p2_bf = 3 * 16 * BL::sb * 2;   // or its bf16 planes (16 columns)
  static constexpr int p1_bytes = N1 * sp1 * 4 > P1Layout<N1>::bytes ? N1 * sp1 * 4 : P1Layout<N1>::bytes;
  static constexpr int off_p2 = (p1_bytes + 15) / 16 * 16;
  static constexpr int off_x = off_p2 + ((p2_f32 > p2_bf ? p2_f32 : p2_bf) + 15) / 16 * 16;
  static constexpr int x_bytes = N1 * sx * 4 > N1 * BL::sb * 2 ? N1 * sx * 4 : N1 * BL::sb * 2;
  static constexpr int off_t = (off_x + x_bytes + 15) / 16 * 16;
  static constexpr int lds = off_t + N1 * 16 * 4;
};

// The factors staged in quads: four consecutive reduction indices of one
// output column (P2: K indices b = 4 bq .. + 3 of column j; P1: reduction
// indices a = 4 aq .. + 3 of output row i), loaded first and committed either
// as the bf16 planes, one 8-byte store per plane and quad (the four indices
// sit in consecutive slots of both plane layouts, at a row stride that spreads
// the lanes of a store over the banks), or as the fp32 rows.  Quads of the
// planes' padding are zeroed without loads.  The plane contents are those of
// the chunked kernel's staging (split3_bf16 of each element), so x~ is the
// same bit for bit.
inline __device__ uint2 pack4_bf16(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return uint2{a | (b << 16), c | (d << 16)};
}
// the three planes of four values, as 8-byte words at dst + o (+ plane, + 2 plane)
inline __device__ void planes_quad_store(const float4& v, uint16_t* dst, int o, int plane) {
  uint32_t h[4], m[4], l[4];
  split3_bf16(v.x, &h[0], &m[0], &l[0]);
  split3_bf16(v.y, &h[1], &m[1], &l[1]);
  split3_bf16(v.z, &h[2], &m[2], &l[2]);
  split3_bf16(v.w, &h[3], &m[3], &l[3]);
  *reinterpret_cast<uint2*>(dst + o) = pack4_bf16(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint2*>(dst + plane + o) = pack4_bf16(m[0], m[1], m[2], m[3]);
  *reinterpret_cast<uint2*>(dst + 2 * plane + o) = pack4_bf16(l[0], l[1], l[2], l[3]);
}

// P2 (n2 x n2, row b, column j): quad q = bq * N2 + j
template <int N2, int NTH>
struct P2Quads {
  static_assert(N2 % 4 == 0, "quads of K indices");
  static constexpr int NQ = N2 * (N2 / 4);
  static constexpr int T = (NQ + NTH - 1) / NTH;
  float4 v[T];
};
template <int N2, int NTH>
__device__ __forceinline__ void p2_quads_issue(const float* __restrict__ P2, P2Quads<N2, NTH>& m) {
#pragma unroll
  for (int i = 0; i < P2Quads<N2, NTH>::T; ++i) {
    const int q = threadIdx.x + NTH * i;
    if (q < P2Quads<N2, NTH>::NQ) {
      const int bq = q / N2, j = q - bq * N2;
      const float* src = P2 + 4 * bq * N2 + j;
      m.v[i] = float4{src[0], src[N2], src[2 * N2], src[3 * N2]};
    }
  }
}
// as the bf16 planes (BfLayout: plane p, column j, K slot b at p * plane +
// j * sb + b), K slots n2 .. kb - 1 zeroed
template <int N2, int NTH>
__device__ __forceinline__ void p2_quads_commit_bf(const P2Quads<N2, NTH>& m, uint16_t* dst) {
  using L = BfLayout<N2>;
#pragma unroll
  for (int i = 0; i < P2Quads<N2, NTH>::T; ++i) {
    const int q = threadIdx.x + NTH * i;
    if (q < P2Quads<N2, NTH>::NQ) {
      const int bq = q / N2, j = q - bq * N2;
      planes_quad_store(m.v[i], dst, j * L::sb + 4 * bq, L::plane);
    }
  }
  constexpr int NZ = N2 * ((L::kb - N2) / 4);  // padding quads
  for (int z = threadIdx.x; z < NZ; z += NTH) {
    const int zq = z / N2, j = z - zq * N2;
    const int o = j * L::sb + N2 + 4 * zq;
#pragma unroll
    for (int p = 0; p < 3; ++p) *reinterpret_cast<uint2*>(dst + p * L::plane + o) = uint2{0u, 0u};
  }
}
// as fp32 rows: element (b, j) at dst[b * SP + j]
template <int N2, int SP, int NTH>
__device__ __forceinline__ void p2_quads_commit_f32(const P2Quads<N2, NTH>& m, float* dst) {
#pragma unroll
  for (int i = 0; i < P2Quads<N2, NTH>::T; ++i) {
    const int q = threadIdx.x + NTH * i;
    if (q < P2Quads<N2, NTH>::NQ) {
      const int bq = q / N2, j = q - bq * N2;
      float* d = dst + 4 * bq * SP + j;
      d[0] = m.v[i].x;
      d[SP] = m.v[i].y;
      d[2 * SP] = m.v[i].z;
      d[3 * SP] = m.v[i].w;
    }
  }
}

// P1 (n1 x n1, row a, column i): quad q = aq * N1 + i
template <int N1, int NTH>
struct P1Quads {
  static_assert(N1 % 4 == 0, "quads of reduction indices");
  static constexpr int NQ = N1 * (N1 / 4);
  static constexpr int T = (NQ + NTH - 1) / NTH;
  float4 v[T];
};
template <int N1, int NTH>
__device__ __forceinline__ void p1_quads_issue(const float* __restrict__ P1, P1Quads<N1, NTH>& m) {
#pragma unroll
  for (int u = 0; u < P1Quads<N1, NTH>::T; ++u) {
    const int q = threadIdx.x + NTH * u;
    if (q < P1Quads<N1, NTH>::NQ) {
      const int aq = q / N1, i = q - aq * N1;
      const float* src = P1 + 4 * aq * N1 + i;
      m.v[u] = float4{src[0], src[N1], src[2 * N1], src[3 * N1]};
    }
  }
}
// as the bf16 stage-2 planes (P1Layout: element (a, i) at row i, slot
// p1_slot(a); the slots of a quad are consecutive), with zeros at the rows i
// and slots of reduction rows a past n1
template <int N1, int NTH>
__device__ __forceinline__ void p1_quads_commit_bf(const P1Quads<N1, NTH>& m, uint16_t* dst) {
  using L = P1Layout<N1>;
#pragma unroll
  for (int u = 0; u < P1Quads<N1, NTH>::T; ++u) {
    const int q = threadIdx.x + NTH * u;
    if (q < P1Quads<N1, NTH>::NQ) {
      const int aq = q / N1, i = q - aq * N1;
      planes_quad_store(m.v[u], dst, i * L::sb + p1_slot(4 * aq), L::plane);
    }
  }
  constexpr int NZ = L::rows * (L::ka / 4);  // every quad of the planes; the data ones are skipped
  if constexpr (L::rows > N1 || L::ka > N1) {
    for (int z = threadIdx.x; z < NZ; z += NTH) {
      const int i = z / (L::ka / 4), sq = z - i * (L::ka / 4);
      if (i >= N1 || p1_row_of_slot(4 * sq) >= N1) {
#pragma unroll
        for (int p = 0; p < 3; ++p) *reinterpret_cast<uint2*>(dst + p * L::plane + i * L::sb + 4 * sq) = uint2{0u, 0u};
      }
    }
  }
}
// as fp32 rows: element (a, i) at dst[a * SP + i]
template <int N1, int SP, int NTH>
__device__ __forceinline__ void p1_quads_commit_f32(const P1Quads<N1, NTH>& m, float* dst) {
#pragma unroll
  for (int u = 0; u < P1Quads<N1, NTH>::T; ++u) {
    const int q = threadIdx.x + NTH * u;
    if (q < P1Quads<N1, NTH>::NQ) {
      const int aq = q / N1, i = q - aq * N1;
      float* d = dst + 4 * aq * SP + i;
      d[0] = m.v[u].x;
      d[SP] = m.v[u].y;
      d[2 * SP] = m.v[u].z;
      d[3 * SP] = m.v[u].w;
    }
  }
}

template <int N1, int N2, int NTH>
__device__ __forceinline__ void x_row_commit_bf(const RowRegs<N1 * N2, NTH>& x, uint16_t* sXb) {
  using L = BfLayout<N2>;
  constexpr int K = N1 * N2;
#pragma unroll
  for (int i = 0; i < RowRegs<K, NTH>::T; ++i) {
    const int q = threadIdx.x + NTH * i;
    if (q < K / 4) *reinterpret_cast<uint2*>(sXb + (4 * q / N2) * L::sb + (4 * q) % N2) = uint2{x.v[i].x, x.v[i].y};
  }
  if constexpr (L::kb > N2) {
    constexpr int pad = L::kb - N2;
    for (int idx = threadIdx.x; idx < N1 * pad; idx += NTH) sXb[(idx / pad) * L::sb + N2 + idx % pad] = 0;
  }
}

// Row r of bf16 x as the n1 x n2 grid of bf16 rows with stride sb (the bf16
// stage-1 layout), K columns n2 .. kb - 1 zeroed; loads first.
template <int N1, int N2, int NTH = 256>
__device__ __forceinline__ void stage_x_row_bf(const DecodeArgs& g, int r, uint16_t* sXb) {
  using L = BfLayout<N2>;
  constexpr int K = N1 * N2;
  constexpr int T = (K / 4 + NTH - 1) / NTH;
  const uint2* src = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.x) + (int64_t)r * K);
  uint2 u[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const int q = threadIdx.x + NTH * i;
    u[i] = q < K / 4 ? src[q] : uint2{0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const int q = threadIdx.x + NTH * i;
    if (q < K / 4) *reinterpret_cast<uint2*>(sXb + (4 * q / N2) * L::sb + (4 * q) % N2) = u[i];
  }
  if constexpr (L::kb > N2) {
    constexpr int pad = L::kb - N2;
    for (int idx = threadIdx.x; idx < N1 * pad; idx += NTH) sXb[(idx / pad) * L::sb + N2 + idx % pad] = 0;
  }
}

template <int NRT, int N1, int N2>
__global__ __launch_bounds__(256) void xform_items_kernel(DecodeArgs g, float* __restrict__ xt) {
  extern __shared__ __align__(16) unsigned char lds[];
  using P = ItemPlan<N1, N2>;
  constexpr int n1 = N1, n2 = N2, K = N1 * N2;
  constexpr int njt = (N2 + 15) / 16;
  float* sP1 = reinterpret_cast<float*>(lds);
  float* sP2 = reinterpret_cast<float*>(lds + P::off_p2);
  float* sX = reinterpret_cast<float*>(lds + P::off_x);
  float* sT = reinterpret_cast<float*>(lds + P::off_t);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;
  const int lk = lane >> 4;
  const int r = blockIdx.x / njt;
  const int jt = blockIdx.x - r * njt;

  if (g.bf16)
    stage_p1_planes<N1, 256>(g.P1, reinterpret_cast<uint16_t*>(lds), tid);
  else
    stage_matrix<N1, P::sp1>(g.P1, sP1);
  if (g.bf16) {  // bf16 stage 1: the tile's P2 planes and the bf16 X grid
    using BL = BfLayout<N2>;
    uint16_t* sP2b = reinterpret_cast<uint16_t*>(lds + P::off_p2);
    uint16_t* sXb = reinterpret_cast<uint16_t*>(lds + P::off_x);
    stage_p2_planes<N2>(g.P2, sP2b, jt * 16, 16, tid, 256);
    stage_x_row_bf<N1, N2>(g, r, sXb);
    __syncthreads();
    for (int rt = wave; rt < NRT; rt += 4) {
      const uint16_t* xg[1] = {sXb};
      const uint16_t* pc[1] = {sP2b + li * BL::sb};
      const int rt0[1] = {rt};
      v4f T[1][1] = {{v4f{0.0f, 0.0f, 0.0f, 0.0f}}};
      stage1_bf16<N1, N2, 1, 1>(xg, rt0, pc, 16 * BL::sb, li, lk, T);
      mfma_settle_before_join();
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // element e of lane l: row 16 rt + 4 (l / 16) + e
        const int row = rt * 16 + 4 * lk + e;
        if (row < n1) sT[row * 16 + li] = T[0][0][e];
      }
    }
  } else {
  {  // the tile's P2 columns [n2][16] (zero past n2), loads first
    constexpr int T = (N2 * 16 + 255) / 256;
    float v[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int idx = tid + 256 * i;
      const int b = idx >> 4, j = jt * 16 + (idx & 15);
      v[i] = (idx < N2 * 16 && j < n2) ? g.P2[b * n2 + j] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const int idx = tid + 256 * i;
      if (idx < N2 * 16) sP2[idx] = v[i];
    }
  }
  stage_x_row<K, N2, P::sx>(g, r, sX);
  __syncthreads();

  // stage 1: T[rt] = X_r * P2[:, tile], steps of b in order (as the chunked kernel)
  for (int rt = wave; rt < NRT; rt += 4) {
    v4f T = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* xa = sX + min(rt * 16 + li, n1 - 1) * P::sx;
    const uint32_t mrow = (rt * 16 + li < n1) ? 0xffffffffu : 0u;
#pragma unroll
    for (int st = 0; st < N2 / 4; ++st) {
      const int b = 4 * st + lk;
      T = __builtin_amdgcn_mfma_f32_16x16x4f32(masked(xa[b], mrow), sP2[b * 16 + li], T, 0, 0, 0);
    }
    mfma_settle_before_join();
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // element e of lane l: row 16 rt + 4 (l / 16) + e
      const int row = rt * 16 + 4 * lk + e;
      if (row < n1) sT[row * 16 + li] = T[e];
    }
  }
  }
  __syncthreads();

  // stage 2: x~[it][tile] = sum_a P1[a][it] T[a][tile], a in the chunked kernel's order
  if (g.bf16) {  // bf16 input: the six plane products per step (quant_core.h)
    const uint16_t* sP1b = reinterpret_cast<const uint16_t*>(lds);
    for (int it = wave; it < NRT; it += 4) {
      v4f o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < P1Layout<N1>::ka / 32; ++q) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {  // slot 8 lk + u: T row 32 q + 16 (u / 4) + 4 lk + u % 4
          const int a = 32 * q + 16 * (u >> 2) + 4 * lk + (u & 3);
          v[u] = a < n1 ? sT[a * 16 + li] : 0.0f;
        }
        v4u b[3], ap[3];
        planes8(v, b);
        p1_planes_at<N1>(sP1b, it, q, li, lk, ap);
#pragma unroll
        for (int k = 0; k < 6; ++k) o = s2_mm(ap[s2_pa(k)], b[s2_pb(k)], o);
      }
      mfma_settle_before_join();
      const int j = jt * 16 + li;
      if (j < n2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int io = it * 16 + 4 * lk + e;
          if (io < n1) xt[(int64_t)r * K + io * n2 + j] = o[e];
        }
      }
    }
    return;
  }
  for (int it = wave; it < NRT; it += 4) {
    v4f o = {0.0f, 0.0f, 0.0f, 0.0f};
    const int i = it * 16 + li;
    const uint32_t mi = i < n1 ? 0xffffffffu : 0u;
#pragma unroll
    for (int st = 0; st < 4 * NRT; ++st) {
      const int ar = 16 * (st >> 2) + 4 * lk + (st & 3);
      const int ac = min(ar, n1 - 1);
      o = __builtin_amdgcn_mfma_f32_16x16x4f32(masked(sP1[ac * P::sp1 + min(i, n1 - 1)], ar < n1 ? mi : 0u),
                                               sT[ac * 16 + li], o, 0, 0, 0);
    }
    mfma_settle_before_join();
    const int j = jt * 16 + li;
    if (j < n2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int io = it * 16 + 4 * lk + e;
        if (io < n1) xt[(int64_t)r * K + io * n2 + j] = o[e];
      }
    }
  }
}

// x~ of row r (bitwise the chunked kernel's) into the X region, then its codes
// and steps into sC / sS.  Ends with a barrier.
template <int NRT, int N1, int N2, int NTH>
__device__ __forceinline__ void transform_row(const DecodeArgs& g, int r, unsigned char* lds,
                                              int8_t* sC, float* sS, bool staged) {
  using P = XPlan<N1, N2>;
  constexpr int n1 = N1, n2 = N2, K = P::K, Ga = K / 32;
  const float* sP1 = reinterpret_cast<const float*>(lds);
  const float* sP2 = reinterpret_cast<const float*>(lds + P::off_p2);
  float* sX = reinterpret_cast<float*>(lds + P::off_x);
  float* sT = reinterpret_cast<float*>(lds + P::off_t);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;
  const int lk = lane >> 4;

  using BL = BfLayout<N2>;
  const uint16_t* sP2b = reinterpret_cast<const uint16_t*>(lds + P::off_p2);
  uint16_t* sXb = reinterpret_cast<uint16_t*>(lds + P::off_x);
  if (!staged) {  // (row 0 is staged with the factors)
    if (g.bf16)
      stage_x_row_bf<N1, N2, NTH>(g, r, sXb);
    else
      stage_x_row<K, N2, P::sx, NTH>(g, r, sX);
  }
  __syncthreads();

  // stage 1: tile (rt, jt) of T = X[16 rt .., :] * P2[:, 16 jt ..], steps of b
  // in order.  Wave w takes tiles w, w + NW, ... (task t: rt = t % NRT, jt =
  // t / NRT), all at once as independent accumulators; the operands of step
  // s + 1 are read before step s multiplies.
  constexpr int NW = NTH / 64;
  constexpr int ntask = NRT * P::njt;
  constexpr int NT = (ntask + NW - 1) / NW;  // tiles per wave
  int rt[NT], jc[NT];
  bool has[NT];
  uint32_t mrow[NT], mj[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int t0 = wave + NW * u;
    has[u] = t0 < ntask;
    const int t = min(t0, ntask - 1);
    rt[u] = t % NRT;
    jc[u] = (t / NRT) * 16 + li;
    mrow[u] = rt[u] * 16 + li < n1 ? 0xffffffffu : 0u;
    mj[u] = jc[u] < n2 ? 0xffffffffu : 0u;
  }
  if (g.bf16) {
    // bf16 input: the bf16 MFMA on the X grid and the P2 planes (the tile
    // sequence of every other kernel, so x~ is bitwise the same)
    const uint16_t* xg[NT];
    const uint16_t* pc[NT];
    int rt0[NT];
    v4f acc[NT][1];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      xg[u] = sXb;
      pc[u] = sP2b + min(jc[u], N2 - 1) * BL::sb;  // columns past n2 read n2 - 1
      rt0[u] = rt[u];
      acc[u][0] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    stage1_bf16<N1, N2, NT, 1>(xg, rt0, pc, BL::plane, li, lk, acc);
    mfma_settle_before_join();
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (has[u]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rt[u] * 16 + 4 * lk + e;
          if (row < n1) sT[row * P::st + jc[u]] = acc[u][0][e];
        }
      }
    }
  } else {
    v4f acc[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float av[2][NT], bv[2][NT];
    auto fetch1 = [&](int s, float (&a)[NT], float (&bb)[NT]) {
      const int b = 4 * s + lk;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        a[u] = masked(sX[min(rt[u] * 16 + li, n1 - 1) * P::sx + b], mrow[u]);
        bb[u] = masked(sP2[b * P::sp2 + min(jc[u], n2 - 1)], mj[u]);
      }
    };
    fetch1(0, av[0], bv[0]);
#pragma unroll
    for (int s = 0; s < N2 / 4; ++s) {
      if (s + 1 < N2 / 4) fetch1(s + 1, av[(s + 1) & 1], bv[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NT; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s & 1][u], bv[s & 1][u], acc[u], 0, 0, 0);
    }
    mfma_settle_before_join();
    // element e of lane l: row 16 rt + 4 (l / 16) + e, column jc
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (has[u]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rt[u] * 16 + 4 * lk + e;
          if (row < n1) sT[row * P::st + jc[u]] = acc[u][e];
        }
      }
    }
  }
  __syncthreads();

  // stage 2: tile (it, jt) of x~ = sum_a P1[a][i] T[a][j], the same tiles per
  // wave (it = t % NRT), over a in the chunked kernel's order (a = 16 (s / 4)
  // + 4 (l / 16) + s % 4, rows >= n1 masked), into the flat x~ row in the X
  // region (no longer read)
  float* sXt = sX;
  if (g.bf16) {
    // bf16 input: the six plane products per step (quant_core.h), the B
    // planes split from T (rows past n1 as zero), tasks interleaved per product
    const uint16_t* sP1b = reinterpret_cast<const uint16_t*>(lds);
    constexpr int GT = NT < 2 ? NT : 2;  // tasks interleaved at a time (registers)
#pragma unroll
    for (int u0 = 0; u0 < NT; u0 += GT) {
      v4f acc[GT];
#pragma unroll
      for (int g2 = 0; g2 < GT; ++g2) acc[g2] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < P1Layout<N1>::ka / 32; ++q) {
        v4u b[GT][3], ap[GT][3];
#pragma unroll
        for (int g2 = 0; g2 < GT; ++g2) {
          const int u = u0 + g2 < NT ? u0 + g2 : NT - 1;
          float v[8];
#pragma unroll
          for (int w = 0; w < 8; ++w) {  // slot 8 lk + w: T row 32 q + 16 (w / 4) + 4 lk + w % 4
            const int a = 32 * q + 16 * (w >> 2) + 4 * lk + (w & 3);
            v[w] = a < n1 ? sT[a * P::st + jc[u]] : 0.0f;
          }
          planes8(v, b[g2]);
          p1_planes_at<N1>(sP1b, rt[u], q, li, lk, ap[g2]);
        }
#pragma unroll
        for (int k = 0; k < 6; ++k)
#pragma unroll
          for (int g2 = 0; g2 < GT; ++g2) acc[g2] = s2_mm(ap[g2][s2_pa(k)], b[g2][s2_pb(k)], acc[g2]);
      }
      mfma_settle_before_join();
#pragma unroll
      for (int g2 = 0; g2 < GT; ++g2) {
        const int u = u0 + g2;
        if (u < NT && has[u] && jc[u] < n2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int io = rt[u] * 16 + 4 * lk + e;
            if (io < n1) sXt[io * n2 + jc[u]] = acc[g2][e];
          }
        }
      }
    }
  } else {
    v4f acc[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float av[2][NT], bv[2][NT];
    auto fetch2 = [&](int s, float (&a)[NT], float (&bb)[NT]) {
      const int ar = 16 * (s >> 2) + 4 * lk + (s & 3);
      const int ac = min(ar, n1 - 1);
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int i = rt[u] * 16 + li;
        a[u] = masked(sP1[ac * P::sp1 + min(i, n1 - 1)], (ar < n1 && i < n1) ? 0xffffffffu : 0u);
        bb[u] = sT[ac * P::st + jc[u]];
      }
    };
    fetch2(0, av[0], bv[0]);
#pragma unroll
    for (int s = 0; s < 4 * NRT; ++s) {
      if (s + 1 < 4 * NRT) fetch2(s + 1, av[(s + 1) & 1], bv[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NT; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s & 1][u], bv[s & 1][u], acc[u], 0, 0, 0);
    }
    mfma_settle_before_join();  // (this branch of the input type joins the bf16 one)
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (has[u] && jc[u] < n2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int io = rt[u] * 16 + 4 * lk + e;
          if (io < n1) sXt[io * n2 + jc[u]] = acc[u][e];
        }
      }
    }
  }
  __syncthreads();

  // quantize row r: 8 lanes per group
  const float qmaxf = (float)g.qmax;
  const float rq = 1.0f / qmaxf;
  const float clip = g.clips.c[r / g.rows_per_clip];
  for (int base = 0; base < Ga * 8; base += NTH) {
    const int q = base + tid;
    const bool valid = q < Ga * 8;
    const int qc = valid ? q : base;  // keep the group's shuffle partners active
    const int j = qc >> 3, l8 = qc & 7;
    const float4 v = *reinterpret_cast<const float4*>(sXt + j * 32 + l8 * 4);
    float s;
    const uint32_t packed = quantize4(v, clip, qmaxf, rq, &s);
    if (valid) {
      *reinterpret_cast<uint32_t*>(sC + r * K + j * 32 + l8 * 4) = packed;
      if (l8 == 0) sS[r * Ga + j] = s;
    }
  }
  __syncthreads();
}

// Canonical codes (16-byte aligned rows) and steps of every row for groups
// [j0, j0 + G) into LDS as make_codes lays them out, 16 codes per load, all
// of a round's loads (8 per thread) issued before its stores.
// kick() runs once, right after the first round of loads is issued (the
// caller issues its weight loads there, behind the activation loads, so that
// waiting for these does not wait for the weights).
template <int MODE, int NTH, typename Kick>
__device__ __forceinline__ void copy_codes(const DecodeArgs& g, int j0, int G, int8_t* sA, int a_ld,
                                           float* sS, int s_ld, Kick kick) {
  const int K = g.K, Ga = K >> 5;
  const int nch = g.R * G * 2;  // 16-code chunks
  for (int base = 0; base < nch; base += NTH * 8) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = base + (int)threadIdx.x + NTH * i;
      v[i] = uint4{0u, 0u, 0u, 0u};
      if (t < nch) {
        const int m = t / (2 * G), rem = t - m * 2 * G;
        v[i] = *reinterpret_cast<const uint4*>(g.a_codes + (int64_t)m * K + (j0 + (rem >> 1)) * 32 + (rem & 1) * 16);
      }
    }
    if (base == 0) kick();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = base + (int)threadIdx.x + NTH * i;
      if (t < nch) {
        const int m = t / (2 * G), rem = t - m * 2 * G;
        *reinterpret_cast<uint4*>(sA + m * a_ld + (rem >> 1) * 32 + (rem & 1) * 16) = v[i];
      }
    }
  }
  if (MODE == 0) {
    const int ns = g.R * G;
    for (int base = 0; base < ns; base += NTH * 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = base + (int)threadIdx.x + NTH * i;
        if (t < ns) {
          const int m = t / G;
          v[i] = g.a_steps[(int64_t)m * Ga + j0 + (t - m * G)];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = base + (int)threadIdx.x + NTH * i;
        if (t < ns) {
          const int m = t / G;
          sS[m * s_ld + t - m * G] = v[i];
        }
      }
    }
  }
}

// Codes and steps of every row for groups [j0, j0 + G) into LDS: codes of
// group j0 + gi of row m at sA + m * a_ld + gi * 32, its step at
// sS[m * s_ld + gi].  Task t = 8 (m G + gi) + l8 covers 4 elements; thread
// tid takes tasks tid + NTH i, kU per round, and the loads of round q + 1
// are issued before round q is quantized.  A group's 8 lanes are consecutive
// and aligned, and R G 8 is a multiple of 8, so a group is wholly valid or
// wholly past the end (then it quantizes a copy of the round's first task
// and stores nothing).
constexpr int kU = 4;
struct CodeRaw {
  uint4 v[kU];  // fp32: 4 elements; bf16: 4 elements in .x .y; codes: .x codes, .y step bits
};
template <int MODE, int NTH, typename Kick>
__device__ __forceinline__ void make_codes(const DecodeArgs& g, int j0, int G, int8_t* sA, int a_ld,
                                           float* sS, int s_ld, Kick kick) {
  const int K = g.K, Ga = K >> 5;
  const int ntask = g.R * G * 8;
  const int per_round = NTH * kU;
  const int nround = (ntask + per_round - 1) / per_round;
  const float qmaxf = (float)g.qmax;
  const float rq = 1.0f / qmaxf;
  auto task_of = [&](int q, int i, int* m, int* gi, int* l8) {
    const int base = q * per_round + NTH * i;
    const int t = base + (int)threadIdx.x < ntask ? base + (int)threadIdx.x : base;
    const int grp = t >> 3;
    *l8 = t & 7;
    *m = grp / G;
    *gi = grp - *m * G;
  };
  auto issue = [&](int q, CodeRaw& raw) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      int m, gi, l8;
      task_of(q, i, &m, &gi, &l8);
      const int64_t e = (int64_t)m * K + (j0 + gi) * 32 + l8 * 4;
      if (q * per_round + NTH * i >= ntask) {  // uniform: nothing of this pass exists
        raw.v[i] = uint4{0u, 0u, 0u, 0u};
      } else if (g.in_codes) {
        raw.v[i].x = *reinterpret_cast<const uint32_t*>(g.a_codes + e);
        raw.v[i].y = MODE == 0 ? __float_as_uint(g.a_steps[(int64_t)m * Ga + j0 + gi]) : 0u;
      } else if (g.bf16) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.x) + e);
        raw.v[i].x = u.x;
        raw.v[i].y = u.y;
      } else {
        raw.v[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(g.x) + e);
      }
    }
  };
  auto process = [&](int q, const CodeRaw& raw) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int base = q * per_round + NTH * i;
      if (base >= ntask) continue;  // uniform
      int m, gi, l8;
      task_of(q, i, &m, &gi, &l8);
      uint32_t packed;
      float st;
      if (g.in_codes) {
        packed = raw.v[i].x;
        st = __uint_as_float(raw.v[i].y);
      } else {
        float4 v;
        if (g.bf16)
          v = float4{bf16_bits_to_float(raw.v[i].x & 0xffffu), bf16_bits_to_float(raw.v[i].x >> 16),
                     bf16_bits_to_float(raw.v[i].y & 0xffffu), bf16_bits_to_float(raw.v[i].y >> 16)};
        else
          v = float4{__uint_as_float(raw.v[i].x), __uint_as_float(raw.v[i].y),
                     __uint_as_float(raw.v[i].z), __uint_as_float(raw.v[i].w)};
        packed = quantize4(v, g.clips.c[m / g.rows_per_clip], qmaxf, rq, &st);
      }
      if (base + (int)threadIdx.x < ntask) {
        *reinterpret_cast<uint32_t*>(sA + m * a_ld + gi * 32 + l8 * 4) = packed;
        if (l8 == 0) sS[m * s_ld + gi] = st;
      }
    }
  };
  CodeRaw ra, rb;
  issue(0, ra);
  kick();
  for (int q = 0; q < nround; q += 2) {  // two register buffers, unrolled by two
    if (q + 1 < nround) issue(q + 1, rb);
    process(q, ra);
    if (q + 1 < nround) {
      if (q + 2 < nround) issue(q + 2, ra);
      process(q + 1, rb);
    }
  }
}

// N1 = N2 = 0: no transform (x quantized as it is, or codes given).
// RM: rows bound (4 or 16).  MODE 0: y; MODE 1: int32 group dots.  CPW:
// output columns per work-group (8, 16 or 32; 16 or 32 for RM = 16).  NTH:
// threads per work-group (256 or 512).
template <int NRT, int N1, int N2, int RM, int MODE, int CPW, int NTH>
__global__ __launch_bounds__(NTH) void decode_kernel(DecodeArgs g) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int KP = N1 > 0 ? slots_for(N1 * N2 / 32, NTH / CPW) : kPer;
  using C = Cols<CPW, NTH, KP>;
  constexpr int NW = C::NW;
  constexpr int kSlice = C::kSlice;
  constexpr int NH = C::NH;
  const int tid = threadIdx.x;
  // columns cb * CPW .. + CPW - 1.  Consecutive work-groups land on the 8
  // XCDs in turn; each XCD takes a contiguous range of column blocks instead,
  // so the 128-byte lines of packed weights (16 columns) and of their steps,
  // which neighbouring blocks of 8 columns share, are fetched through one L2.
  const int G = (int)gridDim.x;
  const int xcd = (int)(blockIdx.x & 7);
  const int cb = xcd * (G >> 3) + min(xcd, G & 7) + (int)(blockIdx.x >> 3);
  const int c = tid & (CPW - 1);   // column of the work-group
  const int gq = tid / CPW;        // lane group: groups gq + GL i of each slice
  const int K = g.K;
  const int Ga = K >> 5;
  const int R = g.R;
  const int nsl = (Ga + kSlice - 1) / kSlice;

  // the first weight slice is in flight while the codes are formed (the
  // second follows once they are: both would crowd the transform's registers)
  constexpr bool kMfma = RM > 4;  // up to 16 rows: MFMA dots; up to 4: VALU dots
  static_assert(!kMfma || CPW >= 16, "the MFMA form takes 16 columns per instruction");
  typedef typename std::conditional<kMfma, MSlice<CPW, NTH, KP>, WSlice<KP>>::type Slice;
  Slice wa, wb;
  auto load = [&](int sl, Slice& buf) {
    if constexpr (kMfma) load_mslice<CPW, MODE, NTH, KP>(g, cb, sl, buf);
    else load_slice<CPW, MODE, NTH, KP>(g, cb, sl, c, gq, buf);
  };
  float acc[RM];
  float accm[NH][4];
#pragma unroll
  for (int m = 0; m < RM; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int tt = 0; tt < NH; ++tt)
#pragma unroll
    for (int e = 0; e < 4; ++e) accm[tt][e] = 0.0f;
  auto dots = [&](int sl, const Slice& buf, int jlo, int jhi, const int8_t* sA, int a_ld, int a_j0,
                  const float* sS, int s_ld) {
    if constexpr (kMfma) mfma_slice<CPW, MODE, NTH, KP>(g, cb, sl, buf, jlo, jhi, sA, a_ld, a_j0, sS, s_ld, accm);
    else dot_slice<CPW, RM, MODE, NTH, KP>(g, cb, sl, c, gq, buf, jlo, jhi, sA, a_ld, a_j0, sS, s_ld, acc);
  };
  // slices alternate between the two register buffers (unrolled by two so
  // each buffer stays in registers); `body(sl, buf)` consumes slice sl
  auto sweep = [&](auto body) {
    for (int sl = 0; sl < nsl; sl += 2) {
      body(sl, wa);
      if (sl + 2 < nsl) load(sl + 2, wa);
      if (sl + 1 < nsl) {
        body(sl + 1, wb);
        if (sl + 3 < nsl) load(sl + 3, wb);
      }
    }
  };
  // The activation-side loads (factors and the first row, or the first round
  // of x / codes) are issued before the weight loads: a wait for them then
  // leaves the weights in flight, so the weight fetch overlaps the transform
  // or the quantizer instead of preceding it.
  float* red;

  if constexpr (N1 > 0) {
    using P = XPlan<N1, N2>;
    // the first weight slice is requested with the factors, except where its
    // registers, live across the transform, would spill ((64, 88), (64, 108)):
    // there it is requested once the codes are formed (measured faster than
    // spilling, whose stores wait for every load in flight)
    constexpr bool late = N1 * N2 > 4096;
    float* sP1 = reinterpret_cast<float*>(lds);
    float* sP2 = reinterpret_cast<float*>(lds + P::off_p2);
    int8_t* sC = reinterpret_cast<int8_t*>(lds + P::off_codes);
    float* sS = reinterpret_cast<float*>(lds + P::off_codes + P::codes_bytes(R));
    red = sS + R * (P::K / 32);
    {
      P1Quads<N1, NTH> m1;
      P2Quads<N2, NTH> m2;
      RowRegs<P::K, NTH> x0;
      p1_quads_issue<N1>(g.P1, m1);
      p2_quads_issue<N2>(g.P2, m2);
      x_row_issue<P::K>(g, 0, x0);
      if constexpr (!late) load(0, wa);
      if (g.bf16)
        p1_quads_commit_bf<N1>(m1, reinterpret_cast<uint16_t*>(lds));
      else
        p1_quads_commit_f32<N1, P::sp1>(m1, sP1);
      if (g.bf16) {
        p2_quads_commit_bf<N2>(m2, reinterpret_cast<uint16_t*>(lds + P::off_p2));
        x_row_commit_bf<N1, N2>(x0, reinterpret_cast<uint16_t*>(lds + P::off_x));
      } else {
        p2_quads_commit_f32<N2, P::sp2>(m2, sP2);
        x_row_commit<P::K, N2, P::sx>(g, x0, reinterpret_cast<float*>(lds + P::off_x));
      }
    }
    // (transform_row's first barrier orders these stores)
    for (int r = 0; r < R; ++r) transform_row<NRT, N1, N2, NTH>(g, r, lds, sC, sS, r == 0);
    if (g.codes_out) dump_codes<NTH>(g, 0, Ga, sC, K, sS, Ga);
    if constexpr (late) load(0, wa);
    if (nsl > 1) load(1, wb);
    sweep([&](int sl, const Slice& buf) { dots(sl, buf, 0, Ga, sC, K, 0, sS, Ga); });
  } else if (g.whole) {
    // every row's codes for all of K in LDS, then the dots of every slice
    int8_t* sA = reinterpret_cast<int8_t*>(lds);                                    // [R][K]
    float* sSt = reinterpret_cast<float*>(lds + ((R * K + 15) & ~15));            // [R][Ga]
    red = sSt + R * Ga;
    auto kick = [&]() {
      load(0, wa);
      if (nsl > 1) load(1, wb);
    };
    if (g.in_codes && g.wide_codes)
      copy_codes<MODE, NTH>(g, 0, Ga, sA, K, sSt, Ga, kick);
    else
      make_codes<MODE, NTH>(g, 0, Ga, sA, K, sSt, Ga, kick);
    __syncthreads();
    if (g.codes_out && !g.in_codes) dump_codes<NTH>(g, 0, Ga, sA, K, sSt, Ga);
    sweep([&](int sl, const Slice& buf) { dots(sl, buf, 0, Ga, sA, K, 0, sSt, Ga); });
  } else {
    // too many codes for LDS: one weight slice of codes at a time
    int8_t* sA = reinterpret_cast<int8_t*>(lds);                          // [RM][kSlice * 32]
    float* sSt = reinterpret_cast<float*>(lds + RM * kSlice * 32);       // [RM][kSlice]
    red = sSt + RM * kSlice;
    load(0, wa);
    if (nsl > 1) load(1, wb);
    auto none = [] {};
    sweep([&](int sl, const Slice& buf) {
      const int j0 = sl * kSlice;
      const int GS = min(kSlice, Ga - j0);
      __syncthreads();  // the previous slice's codes are no longer read
      if (g.in_codes && g.wide_codes)
        copy_codes<MODE, NTH>(g, j0, GS, sA, kSlice * 32, sSt, kSlice, none);
      else
        make_codes<MODE, NTH>(g, j0, GS, sA, kSlice * 32, sSt, kSlice, none);
      __syncthreads();
      if (g.codes_out && !g.in_codes) dump_codes<NTH>(g, j0, GS, sA, kSlice * 32, sSt, kSlice);
      dots(sl, buf, j0, j0 + GS, sA, kSlice * 32, j0, sSt, kSlice);
    });
  }
  if (MODE != 0) return;

  // partial sums of each (row, column) added in a fixed order through LDS
  if constexpr (kMfma) {
    // the NW waves' sums: red[((wave * NH + half) * 4 + e) * 64 + lane]
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int tt = 0; tt < NH; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave * NH + tt) * 4 + e) * 64 + lane] = accm[tt][e];
    __syncthreads();
    for (int o = tid; o < R * CPW; o += NTH) {  // row o / CPW, column o % CPW
      const int m = o / CPW, col = o - m * CPW;
      const int n = cb * CPW + col;
      if (n < g.N) {
        const int ln = (m >> 2) * 16 + (col & 15);
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += red[((w * NH + (col >> 4)) * 4 + (m & 3)) * 64 + ln];
        g.y[(int64_t)m * g.N + n] = tot;
      }
    }
  } else {
    // the GL lane groups' sums: the 64 / CPW lanes of a wave that hold one
    // column (lanes c + CPW k) by an xor butterfly, then the NW waves'
    // totals in wave order through LDS (a fixed order: y is deterministic)
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int m = 0; m < RM; ++m)
#pragma unroll
      for (int o = CPW; o < 64; o <<= 1) acc[m] += __shfl_xor(acc[m], o);
    if (lane < CPW) {
#pragma unroll
      for (int m = 0; m < RM; ++m) red[(wave * RM + m) * CPW + lane] = acc[m];
    }
    __syncthreads();
    for (int o = tid; o < R * CPW; o += NTH) {  // row o / CPW, column o % CPW
      const int m = o / CPW, col = o - m * CPW;
      const int n = cb * CPW + col;
      if (n < g.N) {
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += red[(w * RM + m) * CPW + col];
        g.y[(int64_t)m * g.N + n] = tot;
      }
    }
  }
}

// the kernel of a factor shape (N1 = N2 = 0: none) for CPW columns per work-group
template <int NRT, int N1, int N2, int RM, int MODE, int NTH>
const void* decode_fn(int cpw) {
  if (cpw == 8) {
    if constexpr (RM <= 4) return reinterpret_cast<const void*>(decode_kernel<NRT, N1, N2, RM, MODE, 8, NTH>);
    return nullptr;
  }
  if (cpw == 16) return reinterpret_cast<const void*>(decode_kernel<NRT, N1, N2, RM, MODE, 16, NTH>);
  return reinterpret_cast<const void*>(decode_kernel<NRT, N1, N2, RM, MODE, 32, NTH>);
}

// Threads per work-group of a transform instance: the factor staging, the
// row transform and the quantizer, which every work-group repeats, split over
// 8 waves; 4 for K = 6912, whose 8-wave form spills registers (2 waves per
// SIMD leave 256 each).  The other instances take 4 waves.
constexpr int xform_threads(int n1, int n2) { return n1 * n2 > 6000 ? 256 : 512; }

// LDS of the non-transform instances: all rows' codes and steps, or one
// weight slice of them; then the partial sums (RM * 1 KiB: 256 threads x RM
// floats in the VALU form, at most 8 KiB in the MFMA form)
int whole_lds(int R, int K, int RM) { return ((R * K + 15) & ~15) + R * (K / 32) * 4 + 8 * RM * 32 * 4; }
int slice_lds(int RM, int cpw) {
  const int ks = 2048 / cpw;
  return RM * ks * 32 + RM * ks * 4 + 8 * RM * 32 * 4;
}

// Columns per work-group.  Where every work-group repeats a fixed chain
// before its weight sweep (the row transform of the fused instances, or the
// codes of up to 16 rows over all of K in the MFMA form): the largest of 32,
// 16, 8 that still gives at least 60% of the CUs a work-group (16 at least
// for the MFMA form).  More work-groups than CUs put two on some CUs, which
// then finish about one chain later than the rest; 32 columns per work-group
// and 60-100% of the CUs busy cost only a longer weight sweep (measured at
// N = 6144 and 5632, one row: 192 and 176 work-groups of 32 columns end
// 0.7 us sooner than 384 and 352 of 16; 16 rows of codes: 1.94 against
// 2.28 ms per decode loop-step).  Otherwise (at most 4 rows quantized in
// place or copied, no transform) the sweep is the work, and every CU gets a
// work-group (the adapter recurrence at one row, K = 10560: 19.9 against
// 24.0 us per loop with 165 work-groups of 32 columns).
int pick_cpw(int64_t n_padded, int R, int ncu, bool repeats) {
  const int lo = R > 4 ? 16 : 8;
  for (int cpw = 32; cpw >= lo; cpw >>= 1)
    if (repeats ? n_padded / cpw * 5 >= (int64_t)ncu * 3 : n_padded / cpw >= ncu) return cpw;
  return lo;
}

}  // namespace

bool decode_transform_fused(int R, int n1, int n2) {
  // every work-group repeats the transform of all rows; keep that near the
  // time of the weight fetch it overlaps: at most 1.25M multiply-adds
  if (R <= 0 || R > kDecodeMaxRows) return false;
  if ((int64_t)R * n1 * n2 * (n1 + n2) > 1250000) return false;
  const int RM = R <= 4 ? 4 : kDecodeMaxRows;
#define LOOPQ_DECODE_FITS(n1_, n2_, rs_, nim_, ws_) \
  if (n1 == n1_ && n2 == n2_) return XPlan<n1_, n2_>::lds(R, RM, xform_threads(n1_, n2_)) <= kLdsBudget;
  LOOPQ_SHAPES(LOOPQ_DECODE_FITS)
#undef LOOPQ_DECODE_FITS
  return false;
}

bool decode_transform_items(int n1, int n2) {
#define LOOPQ_ITEM_SHAPE(n1_, n2_, rs_, nim_, ws_) \
  if (n1 == n1_ && n2 == n2_) return true;
  LOOPQ_SHAPES(LOOPQ_ITEM_SHAPE)
#undef LOOPQ_ITEM_SHAPE
  return false;
}

hipError_t launch_decode(const DecodeCall& c, hipStream_t s) {
  if (c.R <= 0) return hipSuccess;
  if (c.R > kDecodeMaxRows || c.K % 32 != 0) return hipErrorInvalidValue;
  const bool xform = c.P1 != nullptr;
  if (xform && (c.a_codes != nullptr || c.mode != 0)) return hipErrorInvalidValue;
  if (xform && !decode_transform_fused(c.R, c.n1, c.n2)) return hipErrorInvalidValue;
  DecodeArgs g;
  memset(&g, 0, sizeof(g));
  g.x = c.x;
  g.bf16 = c.bf16;
  g.a_codes = c.a_codes;
  g.a_steps = c.a_steps;
  g.in_codes = c.a_codes != nullptr;
  g.P1 = c.P1;
  g.P2 = c.P2;
  g.R = c.R;
  g.K = c.K;
  g.N = c.N;
  g.clips = c.clips;
  g.rows_per_clip = c.rows_per_clip > 0 ? c.rows_per_clip : 1;
  g.qmax = c.qmax;
  g.w = c.w;
  g.sw = c.sw;
  g.gshift = c.gw == 128 ? 2 : 0;
  g.y = c.y;
  g.dots = c.dots;
  g.wide_codes = c.a_codes != nullptr && (reinterpret_cast<uintptr_t>(c.a_codes) & 15) == 0 && (c.K & 15) == 0;
  if (c.codes_out != nullptr && c.a_codes == nullptr && c.mode == 0) {
    if ((reinterpret_cast<uintptr_t>(c.codes_out) & 15) != 0 || c.steps_out == nullptr) return hipErrorInvalidValue;
    g.codes_out = c.codes_out;
    g.steps_out = c.steps_out;
  }
  const void* fn = nullptr;
  int lds = 0, threads = 256;
  const bool small = c.R <= 4;
  const int RM = small ? 4 : kDecodeMaxRows;
  const int cpw = pick_cpw(padded_cols(c.N), c.R, device_cu_count(), xform || c.R > 4);
  if (xform) {
#define LOOPQ_DECODE_KERNEL(n1_, n2_, rs_, nim_, ws_)                                                   \
    if (c.n1 == n1_ && c.n2 == n2_) {                                                              \
      constexpr int nrt = (n1_ + 15) / 16;                                                         \
      constexpr int nth = xform_threads(n1_, n2_);                                                 \
      fn = small ? decode_fn<nrt, n1_, n2_, 4, 0, nth>(cpw) : decode_fn<nrt, n1_, n2_, kDecodeMaxRows, 0, nth>(cpw); \
      lds = XPlan<n1_, n2_>::lds(c.R, RM, nth);                                                    \
      threads = nth;                                                                               \
    }
    LOOPQ_SHAPES(LOOPQ_DECODE_KERNEL)
#undef LOOPQ_DECODE_KERNEL
  } else {
    fn = small ? (c.mode == 0 ? decode_fn<1, 0, 0, 4, 0, 256>(cpw) : decode_fn<1, 0, 0, 4, 1, 256>(cpw))
               : (c.mode == 0 ? decode_fn<1, 0, 0, kDecodeMaxRows, 0, 256>(cpw)
                              : decode_fn<1, 0, 0, kDecodeMaxRows, 1, 256>(cpw));
    g.whole = whole_lds(c.R, c.K, RM) <= kLdsBudget;
    lds = g.whole ? whole_lds(c.R, c.K, RM) : slice_lds(RM, cpw);
  }
  if (fn == nullptr || lds > kLdsBudget) return hipErrorInvalidValue;
  hipError_t e = prepare_launch(fn, lds, threads);
  if (e != hipSuccess) return e;
  void* args[] = {&g};
  e = hipLaunchKernel(fn, dim3((unsigned)(padded_cols(c.N) / cpw)), dim3((unsigned)threads), args, lds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_decode_items(const void* x, int bf16, const float* P1, int n1, const float* P2, int n2,
                               int R, float* xt, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (!decode_transform_items(n1, n2)) return hipErrorInvalidValue;
  DecodeArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.x = x;
  ga.bf16 = bf16;
  ga.P1 = P1;
  ga.P2 = P2;
  const void* fi = nullptr;
  int ilds = 0, items = 0;
#define LOOPQ_ITEM_KERNEL(n1_, n2_, rs_, nim_, ws_)                                                \
  if (n1 == n1_ && n2 == n2_) {                                                               \
    fi = reinterpret_cast<const void*>(xform_items_kernel<(n1_ + 15) / 16, n1_, n2_>);       \
    ilds = ItemPlan<n1_, n2_>::lds;                                                           \
    items = R * ((n2_ + 15) / 16);                                                            \
  }
  LOOPQ_SHAPES(LOOPQ_ITEM_KERNEL)
#undef LOOPQ_ITEM_KERNEL
  hipError_t e = prepare_launch(fi, ilds, 256);
  if (e != hipSuccess) return e;
  void* iargs[] = {&ga, &xt};
  e = hipLaunchKernel(fi, dim3((unsigned)items), dim3(256), iargs, ilds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace loopq
