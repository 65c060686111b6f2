// Activation quantizer: Kronecker transform + dynamic group absmax + LAS clip
// + round-to-nearest codes, fused in one kernel (gfx950).
//
// Method: Eq.(4) of the LoopQ specification ("paper_specification.yaml",
// lq1_quantization), the LAS clip per module and loop (loopq_components.las,
// implementation_status lq2) and the shared Kronecker transform
// (implementation_status lq3).  Readings: the transform is formed with fp32
// products and fp32 accumulation (an fp32-class result: each element within
// a few (n1 + n2) ulps of sum |P1| |X| |P2|); the codes and steps are those of
// Eq.(4) applied to that x~ exactly; the step is fl32(c * fl32(absmax / qmax)); codes are
// clamp(rint(fl32(x / s)), -qmax, qmax) with correctly rounded division and
// ties to even; a zero step gives zero codes.
//
// Transform path.  A work-group takes a chunk of R rows.  For each row,
// X = reshape(x, n1, n2) and
//   stage 1:  T  = X * P2          (rows (r, a), columns j, reduction over b)
//   stage 2:  x~ = P1^T * T        (rows i, columns j, reduction over a)
// both on V_MFMA_F32_16X16X4_F32 with operands staged in LDS (P1, P2 and X as
// fp32; T stays in the stage-1 result registers).  x~ goes into the buffer X occupied, and the
// quantizer reads 32-element groups of the flat row from there: for the fp6
// GEMM layout one group per lane, for the other layouts 8 lanes per group, 4
// elements per lane, absmax reduced across the 8 lanes.
#include "loopq_internal.h"
#include "quant_core.h"

#include <string.h>

#include <type_traits>

namespace loopq {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v6i __attribute__((ext_vector_type(6)));

// Position of flat element f of a chunk's transformed rows in LDS: the eight
// 16-byte quarters of each 32-element group are rotated by the group index,
// so that lanes reading one whole group each spread over all LDS banks.
__device__ __forceinline__ int xt_pos(int f) {
  return (f & ~31) | ((((f >> 2) + (f >> 5)) & 7) << 2) | (f & 3);
}

// quantize4 for a whole 32-element group held by one lane, in place: the
// same absmax, step and code arithmetic (the max is order-free, and a group
// redone by exact division gives the codes the fast path gives wherever that
// is not flagged), with the near-tie test taken over the group on
// |p - rint(p)| itself (if that is at most 0.5 - 2^-14, fl32(x/s) lies within
// 0.5 - 2^-15 of rint(p)).  ev and od
// hold the group's even and odd elements on entry and their clamped codes
// (as floats) on return; reload(ev, od) brings the group back for the rare
// exact path.  A row_amax >= 0 replaces the group's absmax (one step per
// row).  Returns the step.
template <typename Reload>
__device__ __forceinline__ float quantize32(v16f& ev, v16f& od, float clip, float qmaxf, float rq,
                                            Reload reload, float row_amax) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fmaxf(fabsf(ev[i]), fabsf(od[i])));
  if (row_amax >= 0.0f) amax = row_amax;  // one step for the whole row
  const float q0 = amax * rq;
  const float base = __builtin_fmaf(__builtin_fmaf(-q0, qmaxf, amax), rq, q0);  // = fl32(amax / qmax)
  const float s = clip * base;
  if (!(s > 0.0f)) {
    ev = v16f{};
    od = v16f{};
    return s;
  }
  const float r = __builtin_amdgcn_rcpf(s);
  bool exact = !(r > 1.0e-37f && r < 1.0e37f);
  // in place: p = fl32(x * r), then its distance to rint(p) (exact in fp32)
  // against the same margin, then the clamped code
  float dmax = 0.0f;
  auto code = [&](float x) {
    const float p = x * r;
    const float rq_ = __builtin_rintf(p);
    dmax = fmaxf(dmax, fabsf(p - rq_));
    return __builtin_amdgcn_fmed3f(rq_, -qmaxf, qmaxf);
  };
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = code(ev[i]);
    od[i] = code(od[i]);
  }
  exact |= dmax > 0.5f - 6.103515625e-05f;
  if (exact) {  // rare: near a rounding boundary, or s extreme
    reload(ev, od);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ev[i] = __builtin_amdgcn_fmed3f(__builtin_rintf(ev[i] / s), -qmaxf, qmaxf);
      od[i] = __builtin_amdgcn_fmed3f(__builtin_rintf(od[i] / s), -qmaxf, qmaxf);
    }
  }
  return s;
}

// Store the codes of one 4-element run in code format FMT and, for the first
// lane of the group, the step.  k0 is the first K index of the run (a
// multiple of 4).
template <int FMT>
__device__ __forceinline__ void store_run_f(const QuantArgs& a, int K, int row, int k0,
                                            uint32_t packed, float s, bool first, const float4& xt) {
  const int Ga = K >> 5;
  const int j = k0 >> 5;
  if (FMT == kCodesTiledF6) {
    // the 8 lanes of the group are consecutive and aligned, so its two
    // half-groups are whole quads of lanes
    store_f6_run(a.codes, (Ga + 1) >> 1, row, k0, e2m3_of_codes4(packed));
  } else if (FMT == kCodesTiledI8) {
    const int kk = k0 & 31;
    const int64_t off = ((int64_t)(row >> 5) * Ga + j) * 1024 + (kk >> 4) * 512 + (row & 31) * 16 +
                        (kk & 15);
    *reinterpret_cast<uint32_t*>(a.codes + off) = packed;
  } else {
    *reinterpret_cast<uint32_t*>(a.codes + (int64_t)row * K + k0) = packed;
  }
  if (first) {
    if (a.scales_gm)
      a.scales[(int64_t)j * a.scales_ld + row] = s;
    else
      a.scales[(int64_t)row * Ga + j] = s;
  }
  if (a.xt_out) *reinterpret_cast<float4*>(a.xt_out + (int64_t)row * K + k0) = xt;
}

__device__ __forceinline__ void store_run(const QuantArgs& a, int row, int k0, uint32_t packed,
                                          float s, bool first, const float4& xt) {
  if (a.codes_fmt == kCodesTiledF6)
    store_run_f<kCodesTiledF6>(a, a.K, row, k0, packed, s, first, xt);
  else if (a.codes_fmt == kCodesTiledI8)
    store_run_f<kCodesTiledI8>(a, a.K, row, k0, packed, s, first, xt);
  else
    store_run_f<kCodesCanonical>(a, a.K, row, k0, packed, s, first, xt);
}

// No transform: quantize x directly.  One wave covers 8 groups (256 elements)
// per step; each wave takes a contiguous range of the rows * K / 256 steps.
__global__ __launch_bounds__(256) void quant_plain_kernel(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int K = a.K;
  const int64_t total = (int64_t)a.rows * K;  // K % 32 == 0, so total % 256 may be 0 or 128.. handled per lane
  const float qmaxf = (float)a.qmax;
  const float rqmax = 1.0f / qmaxf;
  // each wave takes one contiguous range of 256-element steps, so the lines
  // of the tiled code layout are completed by one wave (one L2)
  const int64_t nsteps = (total + 255) / 256;
  const int64_t per_wave = (nsteps + nwaves - 1) / nwaves;
  const int64_t step_end = min(nsteps, ((int64_t)wave + 1) * per_wave);
  for (int64_t base = (int64_t)wave * per_wave * 256; base < step_end * 256; base += 256) {
    const int64_t e0 = base + lane * 4;
    // a lane group of 8 covers one 32-group; groups never straddle rows (K % 32 == 0)
    const bool valid = e0 < total;
    const int64_t ec = valid ? e0 : base;  // keep the shuffle partners active
    const int row = (int)(ec / K);
    const int k0 = (int)(ec - (int64_t)row * K);
    float4 v;
    if (a.bf16) {
      const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + ec);
      v.x = bf16_bits_to_float(u.x & 0xffffu);
      v.y = bf16_bits_to_float(u.x >> 16);
      v.z = bf16_bits_to_float(u.y & 0xffffu);
      v.w = bf16_bits_to_float(u.y >> 16);
    } else {
      v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + ec);
    }
    const float clip = a.clips.c[row / a.rows_per_clip];
    float s;
    const uint32_t packed = quantize4(v, clip, qmaxf, rqmax, &s);
    if (valid) store_run(a, row, k0, packed, s, (lane & 7) == 0, v);
  }
}

// One activation step per token ("LoopQ 4-bit quantization of Ouro-1.4B --
// raw artifacts", "The arms": rtn_w4a4_per_token): Eq.(4) over the whole row.
// One work group per row of x (fp32 or bf16; no transform here): the row's
// absolute maximum, then its step (step_of) and codes (codes4), the same
// arithmetic as the group quantizer.  The step is written to each of the
// row's K/32 group slots, so the group-wise GEMM consumes it unchanged.
// Lane l of each 1024-element window takes elements 4l..4l+3, as in the
// group kernels (whole quads and 8-lane groups for the tiled stores).
__device__ __forceinline__ float4 load_row4(const QuantArgs& a, int row, int k) {
  const int64_t e = (int64_t)row * a.K + k;
  if (a.bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + e);
    return make_float4(bf16_bits_to_float(u.x & 0xffffu), bf16_bits_to_float(u.x >> 16),
                       bf16_bits_to_float(u.y & 0xffffu), bf16_bits_to_float(u.y >> 16));
  }
  return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + e);
}

// NC > 0: the row is held in NC float4 registers per thread (K <= 1024 NC),
// all of its loads issued before the first is used; NC = 0 reads the row
// twice, one quad at a time, for any K.
template <int NC>
__global__ __launch_bounds__(256) void quant_token_kernel(QuantArgs a) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const int n4 = a.K >> 2;
  const float qmaxf = (float)a.qmax;
  const float rq = 1.0f / qmaxf;
  auto amax4 = [](const float4& v) { return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))); };
  auto row_max = [&](float m) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  };
  float m = 0.0f;
  if constexpr (NC > 0) {
    float4 v[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = threadIdx.x + 256 * c;
      v[c] = i < n4 ? load_row4(a, row, 4 * i) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) m = fmaxf(m, amax4(v[c]));
    const float s = step_of(row_max(m), a.clips.c[row / a.rows_per_clip], qmaxf, rq);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = threadIdx.x + 256 * c;
      if (i < n4) store_run(a, row, 4 * i, codes4(v[c], s, qmaxf), s, ((4 * i) & 31) == 0, v[c]);
    }
  } else {
    for (int i = threadIdx.x; i < n4; i += 256) m = fmaxf(m, amax4(load_row4(a, row, 4 * i)));
    const float s = step_of(row_max(m), a.clips.c[row / a.rows_per_clip], qmaxf, rq);
    for (int i = threadIdx.x; i < n4; i += 256) {
      const float4 v = load_row4(a, row, 4 * i);
      store_run(a, row, 4 * i, codes4(v, s, qmaxf), s, ((4 * i) & 31) == 0, v);
    }
  }
}

// Work item of slot ii of a wave.  SR (shared row): a wave's NIM slots are
// consecutive items, all in one row of the chunk (the row's column-tile count
// is a multiple of NIM, or the chunk is one row), so the stage-1 X operand is
// read once for all of them; otherwise the items are dealt to the 4 waves in
// turn.
template <bool SR, int NIM>
__device__ __forceinline__ int item_of(int wave, int ii) {
  return SR ? wave * NIM + ii : wave + 4 * ii;
}

// Stage 1 of the transform for NI work items of one wave: T[ii][rt]
// accumulates X_r * P2 over the 4-deep steps of b.
template <int NRT, int N1, int N2, int NI, int NIM, bool SR>
__device__ __forceinline__ void stage1(const QuantArgs& a, const float* sP2, const float* sX,
                                       int wave, int njt, int li, int lk, v4f (&T)[NIM][NRT]) {
  const int n1 = N1 > 0 ? N1 : a.n1;
  const int n2 = N2 > 0 ? N2 : a.n2;
  constexpr int NA = SR ? 1 : NI;  // distinct X rows among the items
  const float* pb[NI];
  const float* xa[NA][NRT];
  uint32_t mj[NI], mrow[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) mrow[rt] = (rt * 16 + li < n1) ? 0xffffffffu : 0u;
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int item = item_of<SR, NIM>(wave, ii);
    const int r = item / njt;
    const int j = (item - r * njt) * 16 + li;
    mj[ii] = j < n2 ? 0xffffffffu : 0u;
    pb[ii] = sP2 + (j < n2 ? j : 0);
    if (ii < NA) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        xa[ii][rt] = sX + (r * n1 + min(rt * 16 + li, n1 - 1)) * (N2 > 0 ? XStrides<N1, N2>::sx : a.sx);
    }
  }
  // raw (fp32) operands of one 4-deep step; the compile-time form reads the
  // next step's operands before converting and multiplying the current
  // one, so the LDS latency hides behind the MFMAs
  struct Raw {
    float b[NI];
    float a[NA][NRT];
  };
  auto fetch = [&](int s, Raw& o) {
    const int b = 4 * s + lk;
    // addresses are clamped in bounds: load unconditionally, then zero the
    // lanes outside the matrix with an integer mask (no branch)
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
      o.b[ii] = masked(pb[ii][b * (N2 > 0 ? XStrides<N1, N2>::sp2 : a.sp2)], mj[ii]);
#pragma unroll
    for (int ia = 0; ia < NA; ++ia)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) o.a[ia][rt] = masked(xa[ia][rt][b], mrow[rt]);
  };
  auto mma = [&](const Raw& o) {
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        T[ii][rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[SR ? 0 : ii][rt], o.b[ii], T[ii][rt], 0, 0, 0);
  };
  if constexpr (N2 > 0) {  // fully unrolled: the accumulators stay in place
    Raw buf[2];
    fetch(0, buf[0]);
#pragma unroll
    for (int s = 0; s < N2 / 4; ++s) {
      if (s + 1 < N2 / 4) fetch(s + 1, buf[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mma(buf[s & 1]);
    }
  } else {
    for (int s = 0; s < (n2 >> 2); ++s) {
      Raw o;
      fetch(s, o);
      mma(o);
    }
  }
}

// Stage 1 on the bf16 MFMA for the wave's NI items (bf16 input, compile-time
// factor shape): item (row r, column tile jt) covers all NRT row tiles of the
// row's X grid (bf16 rows of stride sb at sXb) against the P2 planes.
template <int NRT, int N1, int N2, int NI, int NIM, bool SR>
__device__ __forceinline__ void stage1_bf(const uint16_t* sXb, const uint16_t* sP2b, int wave, int njt, int li,
                                          int lk, v4f (&T)[NIM][NRT]) {
  using L = BfLayout<N2>;
  const uint16_t* xg[NI];
  const uint16_t* pc[NI];
  int rt0[NI];
  v4f acc[NI][NRT];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int item = item_of<SR, NIM>(wave, ii);
    const int r = item / njt;
    const int jt = item - r * njt;
    xg[ii] = sXb + r * N1 * L::sb;
    pc[ii] = sP2b + min(jt * 16 + li, N2 - 1) * L::sb;  // columns past n2 read n2 - 1
    rt0[ii] = 0;
#pragma unroll
    for (int q = 0; q < NRT; ++q) acc[ii][q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  stage1_bf16<N1, N2, NI, NRT, SR>(xg, rt0, pc, L::plane, li, lk, acc);
#pragma unroll
  for (int ii = 0; ii < NI; ++ii)
#pragma unroll
    for (int q = 0; q < NRT; ++q) T[ii][q] = acc[ii][q];
}

// Stage 2 for the same items: x~[:, tile] = P1^T * T, B operands straight
// from the stage-1 results (element e of tile rt is step s = 4 rt + e);
// writes fp32 x~ into the flat rows of the X region.
template <int NRT, int N1, int N2, int NI, int NIM, bool SR>
__device__ __forceinline__ void stage2(const QuantArgs& a, const float* sP1, float* sX, int wave,
                                       int njt, int li, int lk, const v4f (&T)[NIM][NRT]) {
  const int n1 = N1 > 0 ? N1 : a.n1;
  const int n2 = N2 > 0 ? N2 : a.n2;
  const int K = n1 * n2;
  v4f o[NI][NRT];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii)
#pragma unroll
    for (int it = 0; it < NRT; ++it) o[ii][it] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // step s = 4 rt + e reduces over rows a = 16 rt + 4 (l/16) + e (the rows
  // lane l holds in element e of stage-1 tile rt), for all 4 NRT steps: with
  // n1 % 16 != 0 the last tile's rows below n1 are spread over all four of
  // its steps, and the P1 operand is zero for rows a >= n1 (whose T rows are
  // zero too).  As in stage 1 the compile-time form reads the next step's P1
  // operands before multiplying.
  auto fetch = [&](int s, float (&o2)[NRT]) {
    const int ar = 16 * (s >> 2) + 4 * lk + (s & 3);
    const float* pa = sP1 + min(ar, n1 - 1) * (N1 > 0 ? XStrides<N1, N2>::sp1 : a.sp1);
#pragma unroll
    for (int it = 0; it < NRT; ++it) {
      const int i = it * 16 + li;
      o2[it] = masked(pa[min(i, n1 - 1)], (i < n1 && ar < n1) ? 0xffffffffu : 0u);
    }
  };
  auto mma = [&](int s, const float (&raw)[NRT]) {
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
      for (int it = 0; it < NRT; ++it)
        o[ii][it] = __builtin_amdgcn_mfma_f32_16x16x4f32(raw[it], T[ii][s >> 2][s & 3], o[ii][it], 0, 0, 0);
  };
  if constexpr (N1 > 0) {
    float buf[2][NRT];
    fetch(0, buf[0]);
#pragma unroll
    for (int s = 0; s < 4 * NRT; ++s) {
      if (s + 1 < 4 * NRT) fetch(s + 1, buf[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mma(s, buf[s & 1]);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 4 * NRT; ++s) {
      float raw[NRT];
      fetch(s, raw);
      mma(s, raw);
    }
  }
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int item = item_of<SR, NIM>(wave, ii);
    const int r = item / njt;
    const int j = (item - r * njt) * 16 + li;
    if (j < n2) {
#pragma unroll
      for (int it = 0; it < NRT; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int io = it * 16 + 4 * lk + e;  // result element e of lane l: row 4 (l/16) + e
          if (io < n1) sX[xt_pos(r * K + io * n2 + j)] = o[ii][it][e];
        }
    }
  }
}

// Stage 2 on the bf16 MFMA for the same items (bf16 input, compile-time
// shape): the six plane products of each 16x16 tile of x~ and step of 32
// reduction indices (quant_core.h), the B planes split from the stage-1
// result registers (step q takes tiles 2q and 2q + 1), the A planes read from
// the P1 planes in LDS.  Product k runs across all of the wave's tiles before
// product k + 1, so the six products of a tile do not wait on each other.
template <int NRT, int N1, int N2, int NI, int NIM, bool SR>
__device__ __forceinline__ void stage2_bf(const uint16_t* sP1b, float* sX, int wave, int njt, int li, int lk,
                                          const v4f (&T)[NIM][NRT]) {
  constexpr int K = N1 * N2;
  constexpr int NQ = P1Layout<N1>::ka / 32;
  v4f o[NI][NRT];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii)
#pragma unroll
    for (int it = 0; it < NRT; ++it) o[ii][it] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    v4u b[NI][3], a[NRT][3];
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = T[ii][2 * q][e];
        v[4 + e] = 2 * q + 1 < NRT ? T[ii][2 * q + 1 < NRT ? 2 * q + 1 : 0][e] : 0.0f;
      }
      planes8(v, b[ii]);
    }
#pragma unroll
    for (int it = 0; it < NRT; ++it) p1_planes_at<N1>(sP1b, it, q, li, lk, a[it]);
#pragma unroll
    for (int k = 0; k < 6; ++k)
#pragma unroll
      for (int it = 0; it < NRT; ++it)
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) o[ii][it] = s2_mm(a[it][s2_pa(k)], b[ii][s2_pb(k)], o[ii][it]);
  }
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int item = item_of<SR, NIM>(wave, ii);
    const int r = item / njt;
    const int j = (item - r * njt) * 16 + li;
    if (j < N2) {
#pragma unroll
      for (int it = 0; it < NRT; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int io = it * 16 + 4 * lk + e;  // result element e of lane l: row 4 (l/16) + e
          if (io < N1) sX[xt_pos(r * K + io * N2 + j)] = o[ii][it][e];
        }
    }
  }
}

// Absmax of chunk row r from its four per-wave partials (per-token steps).
__device__ __forceinline__ float row_amax_of(const float* sR, int r) {
  return fmaxf(fmaxf(sR[4 * r], sR[4 * r + 1]), fmaxf(sR[4 * r + 2], sR[4 * r + 3]));
}

// Quantize the flat transformed rows [rows][K] of a chunk held in LDS at sX
// (chunk row r is global row row0 + r; elements placed by xt_pos), four
// elements per lane.  Lane r of the wave holds the clip of chunk row r in cl
// (rows <= 64); a run takes it with one LDS permute, read a step ahead
// together with the run's four elements.
template <int FMT>
__device__ __forceinline__ void quant_chunk(const QuantArgs& a, const float* sX, const float* sR,
                                            int row0, int rows, int K, int wave, int lane, float cl,
                                            float qmaxf, float rqmax) {
  const int nruns = rows * K / 4;  // multiple of 8
  int q0 = wave * 64;
  if (q0 >= nruns) return;
  auto load = [&](int qb, float4& v, float& c) {
    const int q = qb + lane;
    const int qc = q < nruns ? q : qb;
    v = *reinterpret_cast<const float4*>(sX + xt_pos(qc * 4));
    c = __int_as_float(__builtin_amdgcn_ds_bpermute(((qc * 4) / K) << 2, __float_as_int(cl)));
  };
  float4 v;
  float c;
  load(q0, v, c);
  for (; q0 < nruns; q0 += 256) {
    float4 vn = v;
    float cn = c;
    if (q0 + 256 < nruns) load(q0 + 256, vn, cn);
    const int q = q0 + lane;
    const bool valid = q < nruns;
    const int e = (valid ? q : q0) * 4;
    const int r = e / K;
    float s;
    uint32_t packed;
    if (a.per_token) {
      s = step_of(row_amax_of(sR, r), c, qmaxf, rqmax);
      packed = codes4(v, s, qmaxf);
    } else {
      packed = quantize4(v, c, qmaxf, rqmax, &s);
    }
    if (valid) store_run_f<FMT>(a, K, row0 + r, e - r * K, packed, s, (lane & 7) == 0, v);
    v = vn;
    c = cn;
  }
}

// The same for the fp6 code layout, one 32-element group per lane: each
// wave takes a contiguous quarter of the chunk's groups.  The clamped codes
// go through V_CVT_SCALEF32_2XPK16_FP6_F32 (scale 1: integers -7..7 are exact
// e2m3 values), which packs its two 16-element sources interleaved, source 0
// into the even fields; fed the even and the odd elements it yields the
// group's 24 bytes in field order, stored as they are.  A zero code may come
// out as either e2m3 zero pattern.
//
// MAXT > 0 (at most MAXT groups per lane): the codes and steps are kept in
// `out` and stored later by f6_store_deferred; the x~ side output, if any,
// is still written here.
struct F6Group {
  v6i bits;
  float s;
  int row, j, ok;
};

__device__ __forceinline__ void f6_store(const QuantArgs& a, int Gp, int Ga, int row, int j, const v6i& bits,
                                         float s) {
  uint2* dst = reinterpret_cast<uint2*>(reinterpret_cast<char*>(a.codes) +
                                        ((int64_t)(row >> 5) * Gp + (j >> 1)) * kF6BlockBytes +
                                        ((row & 31) + 32 * (j & 1)) * 24);
  dst[0] = uint2{(uint32_t)bits[0], (uint32_t)bits[1]};
  dst[1] = uint2{(uint32_t)bits[2], (uint32_t)bits[3]};
  dst[2] = uint2{(uint32_t)bits[4], (uint32_t)bits[5]};
  if (a.scales_gm)
    a.scales[(int64_t)j * a.scales_ld + row] = s;
  else
    a.scales[(int64_t)row * Ga + j] = s;
}

template <int MAXT>
__device__ __forceinline__ void f6_store_deferred(const QuantArgs& a, int K, const F6Group (&out)[MAXT]) {
  const int Ga = K >> 5;
#pragma unroll
  for (int t = 0; t < MAXT; ++t)
    if (out[t].ok) f6_store(a, (Ga + 1) >> 1, Ga, out[t].row, out[t].j, out[t].bits, out[t].s);
}

template <int MAXT>
__device__ __forceinline__ void quant_groups_f6(const QuantArgs& a, const float* sX, const float* sR,
                                                int row0, int rows, int K, int wave, int lane, float cl,
                                                float qmaxf, float rqmax, F6Group (&out)[MAXT > 0 ? MAXT : 1]) {
  const int Ga = K >> 5;
  const int Gp = (Ga + 1) >> 1;
  const int ng = rows * Ga;
  const int per = (ng + 3) >> 2;
  const int g0 = wave * per;
  const int g1 = min(ng, g0 + per);
  if constexpr (MAXT > 0) {
#pragma unroll
    for (int t = 0; t < MAXT; ++t) out[t].ok = 0;
  }
  int trip = 0;
  for (int gb = g0; gb < g1; gb += 64, ++trip) {  // wave-uniform
    const int g = gb + lane;
    const bool valid = g < g1;
    const int gc = valid ? g : gb;
    // element i sits at gc * 32 + xt_pos quarter rotation; read each one
    // straight into its even / odd source register of the packing instruction
    auto load = [&](v16f& ev, v16f& od) {
      const float* gp = sX + gc * 32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ev[i] = gp[((((2 * i) >> 2) + gc) & 7) << 2 | ((2 * i) & 3)];
        od[i] = gp[((((2 * i + 1) >> 2) + gc) & 7) << 2 | ((2 * i + 1) & 3)];
      }
    };
    v16f ev, od;
    load(ev, od);
    const int r = gc / Ga;
    const int j = gc - r * Ga;
    const float clip = __int_as_float(__builtin_amdgcn_ds_bpermute(r << 2, __float_as_int(cl)));
    const float s = quantize32(ev, od, clip, qmaxf, rqmax, load, a.per_token ? row_amax_of(sR, r) : -1.0f);
    if (!valid) continue;
    // The instruction's result must not share registers with its sources
    // (measured: a result placed inside the second source comes out wrong in
    // one dword per lane).  The register allocator may place it there, and a
    // fence that only keeps the sources live can be scheduled ahead of the
    // instruction, so it is issued here with an early-clobber result, which
    // no input may overlap.
    v6i bits;
    asm volatile("s_nop 1\n\tv_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, 1.0" : "=&v"(bits) : "v"(ev), "v"(od));
    const int row = row0 + r;
    if constexpr (MAXT > 0) {
#pragma unroll
      for (int t = 0; t < MAXT; ++t)
        if (t == trip) out[t] = F6Group{bits, s, row, j, 1};
    } else {
      f6_store(a, Gp, Ga, row, j, bits, s);
    }
    if (a.xt_out) {
      load(ev, od);
      float4* xo = reinterpret_cast<float4*>(a.xt_out + (int64_t)row * K + j * 32);
#pragma unroll
      for (int c = 0; c < 8; ++c) xo[c] = float4{ev[2 * c], od[2 * c], ev[2 * c + 1], od[2 * c + 1]};
    }
  }
}

// Copy an n x n factor into LDS rows of stride sp.  Each thread issues a
// batch of loads before its first LDS write, so the copy takes a few memory
// round trips rather than one per element it moves.
__device__ __forceinline__ void stage_factor(float* dst, const float* src, int n, int sp, int tid) {
  constexpr int kBatch = 16;
  const int nn = n * n;
  for (int base = tid; base < nn; base += 256 * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int idx = base + 256 * i;
      v[i] = idx < nn ? src[idx] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int idx = base + 256 * i;
      if (idx < nn) dst[(idx / n) * sp + idx % n] = v[i];
    }
  }
}

// P1 (fp32 rows of stride sp1) and P2 (its three bf16 planes when BFS, else
// fp32 rows of stride sp2) into LDS for a compile-time factor shape, with
// every global load issued before the first LDS write, so that the staging
// takes one memory round trip.  NT threads take part; thread t is t.  The
// planes are written two K rows at a time (one 32-bit store per plane).
template <int N1, int N2, bool BFS, int NT>
__device__ __forceinline__ void stage_factors_once(const float* __restrict__ P1, const float* __restrict__ P2,
                                                   float* sP1, unsigned char* p2, int t) {
  using S = XStrides<N1, N2>;
  constexpr int U1 = BFS ? 1 : (N1 * N1 + NT - 1) / NT;
  float v1[U1];
  if constexpr (!BFS) {
#pragma unroll
    for (int u = 0; u < U1; ++u) {
      const int idx = t + u * NT;
      v1[u] = idx < N1 * N1 ? P1[idx] : 0.0f;
    }
  }
  if constexpr (BFS) {
    using L = BfLayout<N2>;
    constexpr int NP = N2 * (L::kb / 2);  // (pair of K rows b, b + 1; column j < n2)
    constexpr int U2 = (NP + NT - 1) / NT;
    float v2[U2][2];
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int idx = t + u * NT;
      const int b = 2 * (idx / N2), j = idx % N2;
      v2[u][0] = (idx < NP && b < N2) ? P2[b * N2 + j] : 0.0f;
      v2[u][1] = (idx < NP && b + 1 < N2) ? P2[(b + 1) * N2 + j] : 0.0f;
    }
    // P1 as its bf16 planes (loads issued behind P2's, one round trip for both)
    stage_p1_planes<N1, NT>(P1, reinterpret_cast<uint16_t*>(sP1), t);
    uint32_t* d = reinterpret_cast<uint32_t*>(p2);
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int idx = t + u * NT;
      if (idx < NP) {
        const int b = 2 * (idx / N2), j = idx % N2;
        uint32_t h0, m0, l0, h1, m1, l1;
        split3_bf16(v2[u][0], &h0, &m0, &l0);
        split3_bf16(v2[u][1], &h1, &m1, &l1);
        const int o = (j * L::sb + b) >> 1;  // sb and b are even
        d[o] = h0 | (h1 << 16);
        d[o + L::plane / 2] = m0 | (m1 << 16);
        d[o + L::plane] = l0 | (l1 << 16);
      }
    }
  } else {
    constexpr int U2 = (N2 * N2 + NT - 1) / NT;
    float v2[U2];
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int idx = t + u * NT;
      v2[u] = idx < N2 * N2 ? P2[idx] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U1; ++u) {
      const int idx = t + u * NT;
      if (idx < N1 * N1) sP1[(idx / N1) * S::sp1 + idx % N1] = v1[u];
    }
    float* d = reinterpret_cast<float*>(p2);
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int idx = t + u * NT;
      if (idx < N2 * N2) d[(idx / N2) * S::sp2 + idx % N2] = v2[u];
    }
  }
}

// Work-groups per CU the register allocation is held to: two (at most 256
// registers a lane, two waves a SIMD) where the instance fits in them without
// spilling, which hides one wave's LDS and MFMA latency behind the other's;
// one for the fp32-input instances with four row tiles and the generic ones.
constexpr int xform_min_blocks(int nrt, int n1, int bf) { return n1 > 0 && (bf || nrt < 4) ? 2 : 1; }

// Transform + quantize, NRT = ceil(n1 / 16) row tiles.  N1, N2 > 0 fix the
// factor sizes at compile time (the k-loops then unroll fully, which keeps the
// accumulators in place); N1 = N2 = 0 takes them from the arguments.
// RS > 0 fixes the rows per chunk (the host plan uses the same value) and
// enables the prefetch of the next chunk's X into registers; BF is the input
// type when RS > 0 (1 bf16, 0 fp32).  NIM bounds the work items per wave.
//
// Dynamic LDS: P1 [n1][sp1] f32 at 0, P2 [n2][sp2] f32 at off_p2, and
// X [R*n1][sx] f32 at off_x; after stage 1 the same region holds x~ as flat
// fp32 rows [R][K] (WS: x~ has a region of its own at off_t).
//
// WS (compile-time shapes): 512 threads in two roles, so that each SIMD runs
// one wave of MFMA stages beside one wave of quantizing.  Waves 0-3 run both
// stages of chunk c; waves 4-7 meanwhile quantize chunk c - G (the previous
// chunk of this work-group) from the x~ region, then copy the next chunk's X
// into the X region and prefetch the one after.  Each step has two phases,
// (stage 1 | quantize) and (stage 2 | next X), with a barrier after each:
// stage 2 writes x~ only after the quantizer has read the previous chunk's,
// and the next X lands only after stage 1 has read the current one.
//
// Work item = (row r of the chunk, 16-column tile jt of the n1 x n2 grid);
// item_of gives each wave its items.  Stage 1 computes T[:, jt] = X_r * P2[:, jt]
// as NRT independent 16x16 accumulators (the reduction over b runs in 4-deep
// MFMA steps).  In the result, lane l holds T[16 rt + 4 (l/16) + e][16 jt +
// l%16] in element e of tile rt, which is exactly the B operand stage 2 needs
// from lane l at step s = 4 rt + e once stage 2 takes its reduction over a in
// that order (rows a = 16 rt + 4 (l/16) + e at step s), so T stays in
// registers.  Stage 2 then forms x~[:, jt] = P1^T * T with NRT accumulators
// over the i tiles.
template <int NRT, int N1, int N2, int RS, int NIM, int BF, int WS>
__global__ __launch_bounds__(WS ? 512 : 256, WS ? 1 : xform_min_blocks(NRT, N1, BF)) void quant_xform_kernel(
    QuantArgs a) {
  static_assert(!WS || RS > 0, "the two-role form needs a compile-time shape");
  extern __shared__ __align__(16) unsigned char lds[];
  float* sP1 = reinterpret_cast<float*>(lds);
  float* sP2 = reinterpret_cast<float*>(lds + a.off_p2);
  float* sX = reinterpret_cast<float*>(lds + a.off_x);
  float* sXt = WS ? reinterpret_cast<float*>(lds + a.off_t) : sX;  // the x~ rows
  float* sR = reinterpret_cast<float*>(lds + a.off_rmax);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ltid = tid & 255;  // thread within its role (WS), else tid
  const int qwave = wave & 3;  // wave within its role
  const int n1 = N1 > 0 ? N1 : a.n1;
  const int n2 = N2 > 0 ? N2 : a.n2;
  const int K = n1 * n2;
  const int R = RS > 0 ? RS : a.R;
  const bool bf16 = RS > 0 ? BF == 1 : a.bf16 != 0;
  const float qmaxf = (float)a.qmax;
  const float rqmax = 1.0f / qmaxf;
  const int njt = (n2 + 15) >> 4;
  constexpr bool SR = N2 > 0 && (((N2 + 15) / 16) % NIM == 0 || RS == 1);  // a wave's items share one row

  const int sp1 = N1 > 0 ? XStrides<N1, N2>::sp1 : a.sp1;
  const int sp2 = N2 > 0 ? XStrides<N1, N2>::sp2 : a.sp2;
  const int sx = N2 > 0 ? XStrides<N1, N2>::sx : a.sx;
  // bf16 input of a compile-time shape: stage 1 on the bf16 MFMA (X rows and
  // the P2 planes as bf16 in LDS); otherwise fp32 operands on the fp32 MFMA
  constexpr bool BFS = BF == 1 && N2 > 0 && RS > 0;
  using BL = BfLayout<(N2 > 0 ? N2 : 16)>;
  uint16_t* sP2b = reinterpret_cast<uint16_t*>(lds + a.off_p2);
  uint16_t* sXb = reinterpret_cast<uint16_t*>(lds + a.off_x);
  const int li = lane & 15;  // row of A / column of B and of the result
  const int lk = lane >> 4;  // k within a 4-deep step; result rows lk + 4 e
  const int nchunks = (a.rows + R - 1) / R;

  // X of a chunk: 4 consecutive b per thread-step (n2 % 4 == 0), element q
  // of the chunk's rows*K/4 runs
  auto x_src = [&](int row0, int q) -> int64_t { return (int64_t)row0 * K + (int64_t)q * 4; };
  auto x_dst = [&](int q) -> float* {
    const int e = q * 4;
    const int r = e / K;
    const int k = e - r * K;
    return sX + (r * n1 + k / n2) * sx + k % n2;
  };
  auto put = [&](float* dst, const float4& v) {
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  };
  auto widen = [&](const uint2& u) {
    return float4{bf16_bits_to_float(u.x & 0xffffu), bf16_bits_to_float(u.x >> 16),
                  bf16_bits_to_float(u.y & 0xffffu), bf16_bits_to_float(u.y >> 16)};
  };
  // prefetch buffer for the next chunk's X (compile-time chunk shapes only)
  constexpr int PF = RS > 0 ? (RS * N1 * N2 / 4 + 255) / 256 : 1;
  typedef typename std::conditional<BF == 1, uint2, float4>::type raw_t;
  raw_t pre[PF];
  // Every lane issues all PF loads (past the chunk's end it re-reads its last
  // run), so the loads are counted in program order and the stash waits for
  // them alone, not for the code stores issued after them.
  auto fetch = [&](int chunk) {
    const int row0 = chunk * R;
    const int nq = min(R, a.rows - row0) * K / 4;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int q = min(ltid + 256 * i, nq - 1);
      if constexpr (BF == 1)
        pre[i] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + x_src(row0, q));
      else
        pre[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + x_src(row0, q));
    }
  };
  auto stash = [&](int chunk, bool pad_k) {
    const int row0 = chunk * R;
    const int nq = min(R, a.rows - row0) * K / 4;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int q = ltid + 256 * i;
      if (q < nq) {
        if constexpr (BFS) {
          // four bf16 values as they are, into the bf16 X grid
          const int e = q * 4;
          const int r = e / K;
          const int k = e - r * K;
          *reinterpret_cast<uint2*>(sXb + (r * n1 + k / n2) * BL::sb + k % n2) = pre[i];
        } else if constexpr (BF == 1) {
          put(x_dst(q), widen(pre[i]));
        } else {
          put(x_dst(q), pre[i]);
        }
      }
    }
    if constexpr (BFS && BL::kb > (N2 > 0 ? N2 : 16)) {  // zero K columns n2 .. kb - 1 of every X row
      constexpr int pad = BL::kb - N2;
      if (!pad_k) return;
      for (int idx = ltid; idx < R * N1 * pad; idx += 256) {
        const int row = idx / pad;
        sXb[row * BL::sb + N2 + (idx - row * pad)] = 0;
      }
    }
  };

  // The clip of each chunk row, kept by lane r for row r (rows <= 16): the
  // table indices are wave-uniform, so these are scalar loads, whose wait
  // does not hold up the vector-memory traffic in flight.
  auto clip_lanes = [&](int row0, int rows) {
    float cl = 0.0f;
    int idx = row0 / a.rows_per_clip, pos = row0 - idx * a.rows_per_clip;
#pragma unroll
    for (int r = 0; r < (RS > 0 ? RS : 16); ++r) {
      if (r < rows) {
        const float c = a.clips.c[idx];
        cl = (lane == r || (r == rows - 1 && lane > r)) ? c : cl;  // lanes past the rows: the last row's
        if (++pos == a.rows_per_clip) {
          pos = 0;
          ++idx;
        }
      }
    }
    return cl;
  };

  // Each pass of the grid covers gridDim.x consecutive chunks.  Work-groups
  // land on the 8 XCDs in turn; slot numbering gives each XCD one run of
  // consecutive chunks per pass, so the rows sharing a 128-byte line of the
  // tiled code layout are written at about the same time into one L2.
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int slot = xcd * (G >> 3) + min(xcd, G & 7) + (int)(blockIdx.x >> 3);
  // the first chunk's X is in flight while the factors are staged
  const bool xrole = !WS || wave >= 4;  // this wave moves X and quantizes
  if (RS > 0 && xrole && slot < nchunks) fetch(slot);
  if constexpr (RS > 0) {
    stage_factors_once<N1, N2, BFS, WS ? 512 : 256>(a.P1, a.P2, sP1, lds + a.off_p2, tid);
  } else {
    stage_factor(sP1, a.P1, n1, sp1, tid);
    stage_factor(sP2, a.P2, n2, sp2, tid);
  }
  if constexpr (WS) {
    // the two-role pipeline (see above); x~ of chunk cq waits in its region
    // for the quantizer while the stages run on chunk c
    if (xrole && slot < nchunks) {
      stash(slot, true);
      if (slot + G < nchunks) fetch(slot + G);
    }
    __syncthreads();
    // steps of this work-group: one per chunk, and one more that quantizes
    // the last; each role runs its own loop (so that neither keeps the
    // other's registers live), both meeting the same two barriers a step
    const int nsteps = slot < nchunks ? (nchunks - 1 - slot) / G + 2 : 0;
    if (!xrole) {
      v4f T[NIM][NRT];
      for (int i = 0, c = slot; i < nsteps; ++i, c += G) {
        const bool st = c < nchunks;
        int nmine = 0;
        if (st) {
          const int items = min(R, a.rows - c * R) * njt;
#pragma unroll
          for (int ii = 0; ii < NIM; ++ii) nmine += (item_of<SR, NIM>(wave, ii) < items) ? 1 : 0;
#pragma unroll
          for (int ii = 0; ii < NIM; ++ii)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) T[ii][rt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (BFS) {
            switch (nmine) {
              case 4: if constexpr (NIM >= 4) stage1_bf<NRT, N1, N2, 4, NIM, SR>(sXb, sP2b, wave, njt, li, lk, T); break;
              case 3: if constexpr (NIM >= 3) stage1_bf<NRT, N1, N2, 3, NIM, SR>(sXb, sP2b, wave, njt, li, lk, T); break;
              case 2: if constexpr (NIM >= 2) stage1_bf<NRT, N1, N2, 2, NIM, SR>(sXb, sP2b, wave, njt, li, lk, T); break;
              case 1: stage1_bf<NRT, N1, N2, 1, NIM, SR>(sXb, sP2b, wave, njt, li, lk, T); break;
              default: break;
            }
          } else {
            switch (nmine) {
              case 4: if constexpr (NIM >= 4) stage1<NRT, N1, N2, 4, NIM, SR>(a, sP2, sX, wave, njt, li, lk, T); break;
              case 3: if constexpr (NIM >= 3) stage1<NRT, N1, N2, 3, NIM, SR>(a, sP2, sX, wave, njt, li, lk, T); break;
              case 2: if constexpr (NIM >= 2) stage1<NRT, N1, N2, 2, NIM, SR>(a, sP2, sX, wave, njt, li, lk, T); break;
              case 1: stage1<NRT, N1, N2, 1, NIM, SR>(a, sP2, sX, wave, njt, li, lk, T); break;
              default: break;
            }
          }
        }
        __syncthreads();  // stage 1 done with X; the quantizer done with the x~ rows
        if constexpr (BFS) {
          const uint16_t* sP1b = reinterpret_cast<const uint16_t*>(lds);
          switch (nmine) {
            case 4: if constexpr (NIM >= 4) stage2_bf<NRT, N1, N2, 4, NIM, SR>(sP1b, sXt, wave, njt, li, lk, T); break;
            case 3: if constexpr (NIM >= 3) stage2_bf<NRT, N1, N2, 3, NIM, SR>(sP1b, sXt, wave, njt, li, lk, T); break;
            case 2: if constexpr (NIM >= 2) stage2_bf<NRT, N1, N2, 2, NIM, SR>(sP1b, sXt, wave, njt, li, lk, T); break;
            case 1: stage2_bf<NRT, N1, N2, 1, NIM, SR>(sP1b, sXt, wave, njt, li, lk, T); break;
            default: break;
          }
        } else {
          switch (nmine) {
            case 4: if constexpr (NIM >= 4) stage2<NRT, N1, N2, 4, NIM, SR>(a, sP1, sXt, wave, njt, li, lk, T); break;
            case 3: if constexpr (NIM >= 3) stage2<NRT, N1, N2, 3, NIM, SR>(a, sP1, sXt, wave, njt, li, lk, T); break;
            case 2: if constexpr (NIM >= 2) stage2<NRT, N1, N2, 2, NIM, SR>(a, sP1, sXt, wave, njt, li, lk, T); break;
            case 1: stage2<NRT, N1, N2, 1, NIM, SR>(a, sP1, sXt, wave, njt, li, lk, T); break;
            default: break;
          }
        }
        __syncthreads();  // x~ of chunk c and X of chunk c + G are in place
      }
    } else {
      // fp6 codes of the chunk being quantized, stored in phase B after the
      // next X is copied in (the prefetch loads are then the newest memory
      // operations, so copying X waits for them alone)
      constexpr int MAXT = (((RS * (N1 * N2 / 32) + 3) / 4) + 63) / 64;
      F6Group fout[MAXT];
#pragma unroll
      for (int t = 0; t < MAXT; ++t) fout[t].ok = 0;
      for (int i = 0, c = slot; i < nsteps; ++i, c += G) {
        const bool st = c < nchunks;
        if (i > 0) {  // chunk c - G, whose x~ stage 2 wrote in the previous step
          const int row0 = (c - G) * R;
          const int qrows = min(R, a.rows - row0);
          const float cl = clip_lanes(row0, qrows);
          if (a.codes_fmt == kCodesTiledF6)
            quant_groups_f6<MAXT>(a, sXt, sR, row0, qrows, K, qwave, lane, cl, qmaxf, rqmax, fout);
          else if (a.codes_fmt == kCodesTiledI8)
            quant_chunk<kCodesTiledI8>(a, sXt, sR, row0, qrows, K, qwave, lane, cl, qmaxf, rqmax);
          else
            quant_chunk<kCodesCanonical>(a, sXt, sR, row0, qrows, K, qwave, lane, cl, qmaxf, rqmax);
        }
        __syncthreads();  // stage 1 done with X; the quantizer done with the x~ rows
        if (st && c + G < nchunks) stash(c + G, false);
        if (i > 0 && a.codes_fmt == kCodesTiledF6) f6_store_deferred<MAXT>(a, K, fout);
        if (st && c + 2 * G < nchunks) fetch(c + 2 * G);
        __syncthreads();  // x~ of chunk c and X of chunk c + G are in place
      }
    }
  } else {
    for (int chunk = slot; chunk < nchunks; chunk += G) {
      const int row0 = chunk * R;
      const int rows = min(R, a.rows - row0);
      // clip of chunk row `lane`, loaded now and used after both stages
      const float cl = clip_lanes(row0, rows);
      __syncthreads();  // previous chunk done with the x~ rows (and P staged on the first pass)

      // ---- X rows into LDS: from the prefetch registers, or loaded here
      if constexpr (RS > 0) {
        stash(chunk, true);
      } else {
        const int nq = rows * K / 4;
        for (int q = tid; q < nq; q += 256) {
          const int64_t g = x_src(row0, q);
          float4 v;
          if (bf16)
            v = widen(*reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + g));
          else
            v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + g);
          put(x_dst(q), v);
        }
      }
      __syncthreads();
      // the next chunk's X is in flight during both MFMA stages
      if constexpr (RS > 0) {
        if (chunk + G < nchunks) fetch(chunk + G);
      }

      // ---- stage 1 for the wave's items; all of them run in one loop so
      // NI * NRT accumulator chains interleave
      const int items = rows * njt;
      int nmine = 0;
  #pragma unroll
      for (int ii = 0; ii < NIM; ++ii) nmine += (item_of<SR, NIM>(wave, ii) < items) ? 1 : 0;
      v4f T[NIM][NRT];
  #pragma unroll
      for (int ii = 0; ii < NIM; ++ii)
  #pragma unroll
        for (int rt = 0; rt < NRT; ++rt) T[ii][rt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (BFS) {
        switch (nmine) {
          case 4: if constexpr (NIM >= 4) stage1_bf<NRT, N1, N2, 4, NIM, SR>(sXb, sP2b, wave, njt, li, lk, T); break;
          case 3: if constexpr (NIM >= 3) stage1_bf<NRT, N1, N2, 3, NIM, SR>(sXb, sP2b, wave, njt, li, lk, T); break;
          case 2: if constexpr (NIM >= 2) stage1_bf<NRT, N1, N2, 2, NIM, SR>(sXb, sP2b, wave, njt, li, lk, T); break;
          case 1: stage1_bf<NRT, N1, N2, 1, NIM, SR>(sXb, sP2b, wave, njt, li, lk, T); break;
          default: break;
        }
      } else {
        switch (nmine) {
          case 4: if constexpr (NIM >= 4) stage1<NRT, N1, N2, 4, NIM, SR>(a, sP2, sX, wave, njt, li, lk, T); break;
          case 3: if constexpr (NIM >= 3) stage1<NRT, N1, N2, 3, NIM, SR>(a, sP2, sX, wave, njt, li, lk, T); break;
          case 2: if constexpr (NIM >= 2) stage1<NRT, N1, N2, 2, NIM, SR>(a, sP2, sX, wave, njt, li, lk, T); break;
          case 1: stage1<NRT, N1, N2, 1, NIM, SR>(a, sP2, sX, wave, njt, li, lk, T); break;
          default: break;
        }
      }
      __syncthreads();  // every X read is done; x~ may now overwrite the region

      // ---- stage 2: x~[i][j] = sum_a P1[a][i] T[a][j]
      if constexpr (BFS) {
        const uint16_t* sP1b = reinterpret_cast<const uint16_t*>(lds);
        switch (nmine) {
          case 4: if constexpr (NIM >= 4) stage2_bf<NRT, N1, N2, 4, NIM, SR>(sP1b, sX, wave, njt, li, lk, T); break;
          case 3: if constexpr (NIM >= 3) stage2_bf<NRT, N1, N2, 3, NIM, SR>(sP1b, sX, wave, njt, li, lk, T); break;
          case 2: if constexpr (NIM >= 2) stage2_bf<NRT, N1, N2, 2, NIM, SR>(sP1b, sX, wave, njt, li, lk, T); break;
          case 1: stage2_bf<NRT, N1, N2, 1, NIM, SR>(sP1b, sX, wave, njt, li, lk, T); break;
          default: break;
        }
      } else {
        switch (nmine) {
          case 4: if constexpr (NIM >= 4) stage2<NRT, N1, N2, 4, NIM, SR>(a, sP1, sX, wave, njt, li, lk, T); break;
          case 3: if constexpr (NIM >= 3) stage2<NRT, N1, N2, 3, NIM, SR>(a, sP1, sX, wave, njt, li, lk, T); break;
          case 2: if constexpr (NIM >= 2) stage2<NRT, N1, N2, 2, NIM, SR>(a, sP1, sX, wave, njt, li, lk, T); break;
          case 1: stage2<NRT, N1, N2, 1, NIM, SR>(a, sP1, sX, wave, njt, li, lk, T); break;
          default: break;
        }
      }
      __syncthreads();

      // ---- per-token steps: each row's absmax over its whole x~ row (the
      // max is order-free), one partial per wave, combined when used
      if (a.per_token) {
        for (int r = 0; r < rows; ++r) {
          float m = 0.0f;
          for (int q = tid; q < (K >> 2); q += 256) {
            const float4 v = *reinterpret_cast<const float4*>(sX + xt_pos(r * K + 4 * q));
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
          }
  #pragma unroll
          for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
          if (lane == 0) sR[4 * r + wave] = m;
        }
        __syncthreads();
      }

      // ---- quantize groups of the flat transformed rows
      F6Group none[1];
      if (a.codes_fmt == kCodesTiledF6)
        quant_groups_f6<0>(a, sX, sR, row0, rows, K, wave, lane, cl, qmaxf, rqmax, none);
      else if (a.codes_fmt == kCodesTiledI8)
        quant_chunk<kCodesTiledI8>(a, sX, sR, row0, rows, K, wave, lane, cl, qmaxf, rqmax);
      else
        quant_chunk<kCodesCanonical>(a, sX, sR, row0, rows, K, wave, lane, cl, qmaxf, rqmax);
    }
  }
}

}  // namespace

namespace {

constexpr int kRowMaxBytes = 16 * 4 * 4;

int x_bytes_for(int R, int n1, int sx, int K) {
  int xb = R * n1 * sx * 4;
  if (xb < R * K * 4) xb = R * K * 4;
  return (xb + 15) / 16 * 16;
}

// host copies of BfLayout<n2> (the bf16 stage-1 layouts)
int bf_sb(int n2) { return (n2 + 31) / 32 * 32 + 8; }
int bf_p2_bytes(int n2) { return 3 * n2 * bf_sb(n2) * 2; }
// host copy of P1Layout<n1>::bytes (the bf16 stage-2 planes of P1)
int bf_p1_bytes(int n1) { return 3 * ((n1 + 15) / 16 * 16) * ((n1 + 31) / 32 * 32 + 8) * 2; }


// LDS plan of the fused transform kernel: P1 and P2 with strides that put the
// 16 lanes of an MFMA operand read on distinct banks, and R rows of X with a
// stride of 2 mod 32 (the same region later holds the flat x~ rows).  R is
// the shape's chunk size above, else the largest row count whose
// R * ceil(n2/16) work items fit two per wave.  The bank padding of P1/P2 is
// dropped if that lets two work-groups share a CU.  Returns false if one row
// does not fit.
bool plan_quant(QuantArgs& a) {
  const int budget = 160 * 1024;
  const int njt = (a.n2 + 15) / 16;
  int R = 0, nim = 2, ws = 0;
#define LOOPQ_PLAN_SHAPE(n1_, n2_, rs_, nim_, ws_) \
  if (a.n1 == n1_ && a.n2 == n2_) {                \
    R = rs_;                                       \
    nim = nim_;                                    \
    ws = (ws_) & (a.bf16 ? 1 : 2);                 \
  }
  LOOPQ_SHAPES(LOOPQ_PLAN_SHAPE)
#undef LOOPQ_PLAN_SHAPE
  const bool fixed = R > 0;
  if (!fixed) {
    R = 8 / njt;
    if (R < 1) return false;  // n2 > 128 is rejected earlier
    if (R > 16) R = 16;
  }
  if (R * njt > 4 * nim) return false;  // every work item must have a wave slot
  // bf16 input of a compile-time shape: P2 as bf16 planes, X rows as bf16
  // (the X region must also hold the fp32 x~ rows)
  const bool bfs = fixed && a.bf16;
  auto p2_bytes = [&](int sp2) { return bfs ? bf_p2_bytes(a.n2) : a.n2 * sp2 * 4; };
  auto xb_for = [&](int sx, int r) {
    int xb = x_bytes_for(r, a.n1, sx, a.K);
    const int xbb = (r * a.n1 * bf_sb(a.n2) * 2 + 15) / 16 * 16;
    return bfs && xbb > xb ? xbb : xb;
  };
  // + 256 bytes of per-row absmax partials (16 rows x 4 waves) after X
  auto p1_bytes = [&](int sp1) { return bfs ? bf_p1_bytes(a.n1) : a.n1 * sp1 * 4; };
  auto lds_for = [&](int sp1, int sp2, int sx, int r) {
    const int p2 = (p1_bytes(sp1) + 15) / 16 * 16;
    const int px = (p2 + p2_bytes(sp2) + 15) / 16 * 16;
    return px + xb_for(sx, r) + kRowMaxBytes;
  };
  int sp1 = p1_stride(a.n1);
  int sp2 = p_stride(a.n2);
  int sx = x_stride(a.n2);
  if (fixed) {
    // compile-time shapes: the kernel has these strides built in
    if (lds_for(sp1, sp2, sx, R) > budget) return false;
  } else {
    if (lds_for(sp1, sp2, sx, R) > 80 * 1024 && lds_for(a.n1, a.n2, sx, R) <= 80 * 1024) {
      sp1 = a.n1;
      sp2 = a.n2;
    }
    while (R > 1 && lds_for(sp1, sp2, sx, R) > budget) --R;
    if (lds_for(sp1, sp2, sx, R) > budget) {
      sp1 = a.n1;
      sp2 = a.n2;
      sx = a.n2;
    }
    if (lds_for(sp1, sp2, sx, R) > budget) return false;
  }
  a.sp1 = sp1;
  a.sp2 = sp2;
  a.sx = sx;
  a.st = 0;
  a.R = R;
  a.off_p2 = (p1_bytes(sp1) + 15) / 16 * 16;
  a.off_x = (a.off_p2 + p2_bytes(sp2) + 15) / 16 * 16;
  a.off_t = 0;
  a.off_rmax = a.off_x + xb_for(sx, R);
  a.lds_bytes = a.off_rmax + kRowMaxBytes;
  a.ws = 0;
  // the two-role form (compile-time shapes; per-token steps need a barrier
  // among the quantizing waves alone, so they keep the one-phase form): X
  // and the x~ rows in regions of their own
  if (fixed && ws && !a.per_token) {
    const int xg = bfs ? R * a.n1 * bf_sb(a.n2) * 2 : R * a.n1 * sx * 4;
    const int off_t = a.off_x + (xg + 15) / 16 * 16;
    const int off_rmax = off_t + (R * a.K * 4 + 15) / 16 * 16;
    if (off_rmax + kRowMaxBytes <= budget) {
      a.ws = 1;
      a.off_t = off_t;
      a.off_rmax = off_rmax;
      a.lds_bytes = off_rmax + kRowMaxBytes;
    }
  }
  return true;
}

}  // namespace

bool quant_plan_fits(int K, int n1, int n2) {
  // the plan must fit for either input type (bf16 inputs of compile-time
  // shapes use the bf16 stage-1 layouts)
  for (int bf = 0; bf < 2; ++bf) {
    QuantArgs a;
    memset(&a, 0, sizeof(a));
    a.K = K;
    a.n1 = n1;
    a.n2 = n2;
    a.bf16 = bf;
    if (!plan_quant(a)) return false;
  }
  return true;
}

hipError_t launch_quant_token(QuantArgs a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.P1 != nullptr) return hipErrorInvalidValue;  // transform first, then quantize x~
  const int n4 = a.K / 4;
  void (*fn)(QuantArgs) = n4 <= 256    ? quant_token_kernel<1>
                          : n4 <= 512  ? quant_token_kernel<2>
                          : n4 <= 1024 ? quant_token_kernel<4>
                          : n4 <= 1536 ? quant_token_kernel<6>
                          : n4 <= 2048 ? quant_token_kernel<8>
                                       : quant_token_kernel<0>;
  hipLaunchKernelGGL(fn, dim3((unsigned)a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quant_act(QuantArgs a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.P1 == nullptr) {
    const int64_t waves_needed = ((int64_t)a.rows * a.K + 255) / 256;
    int64_t blocks = (waves_needed + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(quant_plain_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (!plan_quant(a)) return hipErrorInvalidConfiguration;
  const void* fn = nullptr;
#define LOOPQ_KERNEL_FORM(n1_, n2_, rs_, nim_, bf_, ws_)                                                  \
  (a.ws ? reinterpret_cast<const void*>(quant_xform_kernel<(n1_ + 15) / 16, n1_, n2_, rs_, nim_, bf_, ws_>) \
        : reinterpret_cast<const void*>(quant_xform_kernel<(n1_ + 15) / 16, n1_, n2_, rs_, nim_, bf_, 0>))
#define LOOPQ_KERNEL_SHAPE(n1_, n2_, rs_, nim_, ws_)                                     \
  if (a.n1 == n1_ && a.n2 == n2_)                                                        \
    fn = a.bf16 ? LOOPQ_KERNEL_FORM(n1_, n2_, rs_, nim_, 1, ((ws_) & 1) ? 1 : 0)         \
                : LOOPQ_KERNEL_FORM(n1_, n2_, rs_, nim_, 0, ((ws_) & 2) ? 1 : 0);
  LOOPQ_SHAPES(LOOPQ_KERNEL_SHAPE)
#undef LOOPQ_KERNEL_SHAPE
#undef LOOPQ_KERNEL_FORM
  if (fn == nullptr) {
    switch ((a.n1 + 15) / 16) {
      case 1: fn = reinterpret_cast<const void*>(quant_xform_kernel<1, 0, 0, 0, 2, 0, 0>); break;
      case 2: fn = reinterpret_cast<const void*>(quant_xform_kernel<2, 0, 0, 0, 2, 0, 0>); break;
      case 3: fn = reinterpret_cast<const void*>(quant_xform_kernel<3, 0, 0, 0, 2, 0, 0>); break;
      case 4: fn = reinterpret_cast<const void*>(quant_xform_kernel<4, 0, 0, 0, 2, 0, 0>); break;
      case 5: fn = reinterpret_cast<const void*>(quant_xform_kernel<5, 0, 0, 0, 2, 0, 0>); break;
      case 6: fn = reinterpret_cast<const void*>(quant_xform_kernel<6, 0, 0, 0, 2, 0, 0>); break;
      case 7: fn = reinterpret_cast<const void*>(quant_xform_kernel<7, 0, 0, 0, 2, 0, 0>); break;
      case 8: fn = reinterpret_cast<const void*>(quant_xform_kernel<8, 0, 0, 0, 2, 0, 0>); break;
      default: return hipErrorInvalidConfiguration;
    }
  }
  const int threads = a.ws ? 512 : 256;
  int per_cu = 1, ncu = 256;
  hipError_t e = prepare_launch(fn, a.lds_bytes, threads, &per_cu, &ncu);
  if (e != hipSuccess) return e;
  const int nchunks = (a.rows + a.R - 1) / a.R;
  int blocks = ncu * per_cu;
  if (blocks > nchunks) blocks = nchunks;
  void* args[] = {&a};
  e = hipLaunchKernel(fn, dim3(blocks), dim3(threads), args, a.lds_bytes, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace loopq
