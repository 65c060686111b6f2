// Activation quantizer: Kronecker transform + dynamic group absmax + LAS clip
// + round-to-nearest codes, fused in one kernel (gfx950).
//
// Method: Eq.(4) of the LoopQ specification ("paper_specification.yaml",
// lq1_quantization), the LAS clip per module and loop (loopq_components.las,
// implementation_status lq2) and the shared Kronecker transform
// (implementation_status lq3).  Readings: the transform is formed in fp64 and
// rounded once to fp32; the step is fl32(c * fl32(absmax / qmax)); codes are
// clamp(rint(fl32(x / s)), -qmax, qmax) with correctly rounded division and
// ties to even; a zero step gives zero codes.
//
// Transform path.  A work-group takes a chunk of R rows.  For each row,
// X = reshape(x, n1, n2) and
//   stage 1:  T  = X * P2          (rows (r, a), columns j, reduction over b)
//   stage 2:  x~ = P1^T * T        (rows i, columns j, reduction over a)
// both on V_MFMA_F64_16X16X4_F64 with operands staged in LDS (P1, P2 and X as
// fp32, T as fp64).  x~ is rounded to fp32 into the buffer X occupied, and the
// quantizer reads 32-element groups of the flat row from there: 8 lanes per
// group, 4 elements per lane, absmax reduced across the 8 lanes.
#include "loopq_internal.h"

namespace loopq {
namespace {

typedef double v4d __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Quantize 4 consecutive elements of one 32-group whose 8 lanes are
// consecutive in the wave (lane % 8 = position of the 4-element run).
// Returns the 4 codes packed as int8 bytes; writes the step to *step.
__device__ __forceinline__ uint32_t quantize4(float4 v, float clip, float qmaxf, float* step) {
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
  const float base = amax / qmaxf;  // correctly rounded fp32 division
  const float s = clip * base;      // one fp32 product
  *step = s;
  uint32_t packed = 0u;
  if (s > 0.0f) {
    float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float r = __builtin_rintf(e[i] / s);  // ties to even
      r = fminf(fmaxf(r, -qmaxf), qmaxf);
      packed |= (uint32_t)((int)r & 0xff) << (8 * i);
    }
  }
  return packed;
}

// Store the codes of one 4-element run and, for the first lane of the group,
// the step.  k0 is the first K index of the run (a multiple of 4).
__device__ __forceinline__ void store_run(const QuantArgs& a, int row, int k0, uint32_t packed,
                                          float s, bool first, const float4& xt) {
  const int K = a.K;
  const int Ga = K >> 5;
  const int j = k0 >> 5;
  if (a.codes_tiled) {
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

// No transform: quantize x directly.  One wave covers 8 groups (256 elements)
// per step; the grid strides over all rows * K / 256 wave-steps.
__global__ __launch_bounds__(256) void quant_plain_kernel(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int K = a.K;
  const int64_t total = (int64_t)a.rows * K;  // K % 32 == 0, so total % 256 may be 0 or 128.. handled per lane
  const float qmaxf = (float)a.qmax;
  for (int64_t base = (int64_t)wave * 256; base < total; base += (int64_t)nwaves * 256) {
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
    const uint32_t packed = quantize4(v, clip, qmaxf, &s);
    if (valid) store_run(a, row, k0, packed, s, (lane & 7) == 0, v);
  }
}

// Transform + quantize.  Dynamic LDS: P1 [n1][sp1] f32 at 0, P2 [n2][sp2] f32
// at off_p2, X [R*n1][sx] f32 at off_x (reused for x~, flat [R][K]), T
// [R*n1][st] f64 at off_t.
__global__ __launch_bounds__(256) void quant_xform_kernel(QuantArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  float* sP1 = reinterpret_cast<float*>(lds);
  float* sP2 = reinterpret_cast<float*>(lds + a.off_p2);
  float* sX = reinterpret_cast<float*>(lds + a.off_x);
  double* sT = reinterpret_cast<double*>(lds + a.off_t);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n1 = a.n1, n2 = a.n2, K = a.K;
  const int R = a.R;
  const float qmaxf = (float)a.qmax;

  for (int idx = tid; idx < n1 * n1; idx += 256) sP1[(idx / n1) * a.sp1 + idx % n1] = a.P1[idx];
  for (int idx = tid; idx < n2 * n2; idx += 256) sP2[(idx / n2) * a.sp2 + idx % n2] = a.P2[idx];

  const int li = lane & 15;  // row (A) / column (B, D) within a 16x16 tile
  const int lk = lane >> 4;  // k within a 4-deep step; D rows lk, lk+4, lk+8, lk+12
  const int nchunks = (a.rows + R - 1) / R;

  for (int chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int row0 = chunk * R;
    const int rows = min(R, a.rows - row0);
    __syncthreads();  // previous chunk done with sX / sT (and P staged on the first pass)

    // ---- load X rows (4 consecutive b per thread-step; n2 % 4 == 0)
    const int nq = rows * K / 4;
    for (int q = tid; q < nq; q += 256) {
      const int e = q * 4;
      const int r = e / K;
      const int k = e - r * K;
      const int ra = r * n1 + k / n2;
      const int b = k % n2;
      const int64_t g = (int64_t)(row0 + r) * K + k;
      float4 v;
      if (a.bf16) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + g);
        v.x = bf16_bits_to_float(u.x & 0xffffu);
        v.y = bf16_bits_to_float(u.x >> 16);
        v.z = bf16_bits_to_float(u.y & 0xffffu);
        v.w = bf16_bits_to_float(u.y >> 16);
      } else {
        v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + g);
      }
      float* dst = sX + ra * a.sx + b;
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    __syncthreads();

    // ---- stage 1: T[(r,a)][j] = sum_b X[(r,a)][b] * P2[b][j]
    {
      const int flat_rows = rows * n1;
      const int nrt = (flat_rows + 15) >> 4;
      const int njt = (n2 + 15) >> 4;
      const int nsteps = n2 >> 2;
      for (int tile = wave; tile < nrt * njt; tile += 4) {
        const int rt = tile / njt, jt = tile - (tile / njt) * njt;
        const int ra = rt * 16 + li;
        const int j = jt * 16 + li;
        const bool va = ra < flat_rows;
        const bool vj = j < n2;
        const float* xa = sX + (va ? ra : 0) * a.sx;
        const float* pb = sP2 + (vj ? j : 0);
        v4d acc = {0.0, 0.0, 0.0, 0.0};
        for (int s = 0; s < nsteps; ++s) {
          const int b = 4 * s + lk;
          const double av = va ? (double)xa[b] : 0.0;
          const double bv = vj ? (double)pb[b * a.sp2] : 0.0;
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
        }
        if (vj) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ro = rt * 16 + 4 * e + lk;  // D element e of lane l: row 4e + l/16
            if (ro < flat_rows) sT[ro * a.st + j] = acc[e];
          }
        }
      }
    }
    __syncthreads();

    // ---- stage 2: x~[r][i][j] = sum_a P1[a][i] * T[(r,a)][j]  -> fp32, flat in sX
    {
      const int nit = (n1 + 15) >> 4;
      const int njt = (n2 + 15) >> 4;
      const int per_row = nit * njt;
      const int nsteps = n1 >> 2;
      for (int tile = wave; tile < rows * per_row; tile += 4) {
        const int r = tile / per_row;
        const int rem = tile - r * per_row;
        const int it = rem / njt, jt = rem - (rem / njt) * njt;
        const int i = it * 16 + li;
        const int j = jt * 16 + li;
        const bool vi = i < n1;
        const bool vj = j < n2;
        const float* pa = sP1 + (vi ? i : 0);
        const double* tb = sT + (int64_t)(r * n1) * a.st + (vj ? j : 0);
        v4d acc = {0.0, 0.0, 0.0, 0.0};
        for (int s = 0; s < nsteps; ++s) {
          const int aa = 4 * s + lk;
          const double av = vi ? (double)pa[aa * a.sp1] : 0.0;
          const double bv = vj ? tb[aa * a.st] : 0.0;
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
        }
        if (vj) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int io = it * 16 + 4 * e + lk;
            if (io < n1) sX[r * K + io * n2 + j] = (float)acc[e];  // RNE to fp32
          }
        }
      }
    }
    __syncthreads();

    // ---- quantize groups of the flat transformed rows
    const int nruns = rows * K / 4;  // multiple of 8
    for (int q0 = wave * 64; q0 < nruns; q0 += 256) {
      const int q = q0 + lane;
      const bool valid = q < nruns;
      const int qc = valid ? q : q0;
      const int e = qc * 4;
      const int r = e / K;
      const int k0 = e - r * K;
      const float4 v = *reinterpret_cast<const float4*>(sX + r * K + k0);
      const int row = row0 + r;
      const float clip = a.clips.c[row / a.rows_per_clip];
      float s;
      const uint32_t packed = quantize4(v, clip, qmaxf, &s);
      if (valid) store_run(a, row, k0, packed, s, (lane & 7) == 0, v);
    }
  }
}

}  // namespace

namespace {

int stride_mod(int n, int mod, int rem) {
  int s = n;
  while (s % mod != rem) ++s;
  return s;
}

int x_bytes_for(int R, int n1, int sx, int K) {
  int xb = R * n1 * sx * 4;
  if (xb < R * K * 4) xb = R * K * 4;
  return (xb + 15) / 16 * 16;
}

// LDS plan of the fused transform kernel: strides chosen so the MFMA operand
// reads of 16 lanes fall on distinct banks, then as many rows per chunk as fit
// two work-groups per CU (at most 16).  Returns false if one row does not fit.
bool plan_quant(QuantArgs& a) {
  const int budget = 160 * 1024;
  a.sp1 = a.n1 <= 16 ? 16 : stride_mod(a.n1, 32, 16);
  a.sp2 = a.n2 <= 16 ? 16 : stride_mod(a.n2, 32, 16);
  a.sx = stride_mod(a.n2, 32, 2);
  a.st = stride_mod(a.n2, 16, 8);
  auto need = [&](int R) {
    const int p2 = (a.n1 * a.sp1 * 4 + 15) / 16 * 16;
    const int pt = (p2 + a.n2 * a.sp2 * 4 + 15) / 16 * 16;
    return pt + x_bytes_for(R, a.n1, a.sx, a.K) + R * a.n1 * a.st * 8;
  };
  if (need(1) > budget) {  // drop the bank padding
    a.sp1 = a.n1;
    a.sp2 = a.n2;
    a.sx = a.n2;
    a.st = a.n2;
  }
  if (need(1) > budget) return false;
  int R = 1;
  while (R < 16 && need(R + 1) <= 80 * 1024) ++R;
  a.R = R;
  a.off_p2 = (a.n1 * a.sp1 * 4 + 15) / 16 * 16;
  a.off_x = (a.off_p2 + a.n2 * a.sp2 * 4 + 15) / 16 * 16;
  a.off_t = a.off_x + x_bytes_for(R, a.n1, a.sx, a.K);
  a.lds_bytes = a.off_t + R * a.n1 * a.st * 8;
  return true;
}

}  // namespace

bool quant_plan_fits(int K, int n1, int n2) {
  QuantArgs a;
  a.K = K;
  a.n1 = n1;
  a.n2 = n2;
  return plan_quant(a);
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
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(quant_xform_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, a.lds_bytes);
  if (e != hipSuccess) return e;
  const int nchunks = (a.rows + a.R - 1) / a.R;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 256;
  const int per_cu = a.lds_bytes <= 80 * 1024 ? 2 : 1;
  int blocks = ncu * per_cu;
  if (blocks > nchunks) blocks = nchunks;
  hipLaunchKernelGGL(quant_xform_kernel, dim3(blocks), dim3(256), a.lds_bytes, s, a);
  return hipGetLastError();
}

}  // namespace loopq
