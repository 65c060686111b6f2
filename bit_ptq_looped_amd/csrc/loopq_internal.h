// Internal declarations shared by the HIP translation units of libloopq.
// Layouts, argument structs and the host-side launchers each kernel file
// provides.  Nothing here is part of the public C ABI (include/loopq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace loopq {

// ---------------------------------------------------------------------------
// Packed weight layout (opaque to callers).
//
// Codes: the weight [N][K] is cut into blocks of 32 output columns x 32 K.
// Block (nb, kc) starts at byte (nb * (K/32) + kc) * 512.  Inside a block the
// byte for column c (0..31), K-half h (0..1) and 16-element run i (0..15) is
//   h * 256 + c * 8 + (i / 8) * 4 + (i % 4),
// low nibble for i % 8 < 4, high nibble for i % 8 >= 4.  A nibble holds the
// code biased by 8 (q + 8 in 1..15).  One wave reads a block as 64 lanes x 8
// contiguous bytes; lane l gets column l % 32 and K-half l / 32, which is the
// B-operand layout of V_MFMA_I32_32X32X32_I8.
//
// Steps: fp16, [ceil(N/32)][G_w][32] (column block, weight group, slot);
// column c of a block sits in slot step_slot(c) = ((c >> 2) & 1) * 16 +
// (c >> 3) * 4 + (c & 3), so the 16 columns 8q + 4h + r (q, r in 0..3) that
// one half-wave holds in a 32x32 MFMA result are 32 contiguous bytes.
// Columns past N (padding to a multiple of 32) hold code 0 and step 0.
// ---------------------------------------------------------------------------
constexpr int kColBlock = 32;
constexpr int kChunkK = 32;
constexpr int kBlockBytes = 512;

inline int64_t padded_cols(int64_t N) { return (N + 31) / 32 * 32; }
__host__ __device__ inline int step_slot(int c) { return ((c >> 2) & 1) * 16 + (c >> 3) * 4 + (c & 3); }
inline int64_t weight_groups(int64_t K, int64_t gw) { return (K + gw - 1) / gw; }

// ---------------------------------------------------------------------------
// Internal activation layout used between the quantizer and the GEMM.
//
// Codes: rows padded to a multiple of 32; block (mb, j) of 32 rows x one
// 32-group starts at byte (mb * (K/32) + j) * 1024; inside, row r (0..31),
// K-half h and byte i (0..15) sit at h * 512 + r * 16 + i.  Lane l of a wave
// loads 16 contiguous bytes = the A operand of V_MFMA_I32_32X32X32_I8 for
// row l % 32, K-half l / 32.
// Steps: fp32 group-major [K/32][ld] with ld >= padded rows.
//
// bf16 variant (operands of V_MFMA_F32_32X32X16_BF16): the same blocks at
// 2048 bytes each; row r, K-half h and element i (0..15) sit at
// h * 1024 + r * 32 + 2 i, so lane l loads 32 contiguous bytes (row l % 32,
// K-half l / 32) and feeds elements 0..7 and 8..15 to two MFMAs.  Codes are
// small integers, exact in bf16.  Expanded weights use the identical layout
// with output columns in place of rows.
// ---------------------------------------------------------------------------
enum CodeFormat { kCodesCanonical = 0, kCodesTiledI8 = 1, kCodesTiledBf16 = 2 };
inline int64_t padded_rows(int64_t M) { return (M + 31) / 32 * 32; }

struct ClipTable {
  float c[64];
};

struct QuantArgs {
  const void* x;     // [rows][K], fp32 or bf16
  int rows;          // number of rows (T*M for the looped forms)
  int K;
  int bf16;          // 1 if x is bf16
  const float* P1;   // [n1][n1] or null
  const float* P2;   // [n2][n2] or null
  int n1, n2;
  int rows_per_clip; // row r uses clips.c[r / rows_per_clip]
  ClipTable clips;
  int qmax;
  int8_t* codes;     // canonical [rows][K] or a tiled GEMM layout
  int codes_fmt;     // CodeFormat
  float* scales;     // row-major [rows][K/32] or group-major [K/32][scales_ld]
  int scales_gm;
  int scales_ld;
  float* xt_out;     // nullable, [rows][K]
  // transform kernel LDS plan (set by the host launcher)
  int R;             // rows per work chunk
  int sp1, sp2, sx, st;  // LDS strides (elements) of P1, P2, X, T
  int off_p2, off_x, off_t;  // byte offsets in dynamic LDS
  int lds_bytes;
};

// host launchers -------------------------------------------------------------
hipError_t launch_quant_act(QuantArgs a, hipStream_t s);
// true if the fused transform kernel's LDS plan fits one work-group
bool quant_plan_fits(int K, int n1, int n2);

hipError_t launch_pack_weights(const float* w, int K, int N, int gw, uint8_t* codes,
                               __half* scales, hipStream_t s);
hipError_t launch_export_weights(const uint8_t* codes, const __half* scales, int K, int N, int gw,
                                 int8_t* out_codes, uint16_t* out_scales, hipStream_t s);
hipError_t launch_fold(const float* w, int K, int N, const float* P1, int n1, const float* P2,
                       int n2, float* out, void* ws, hipStream_t s);

hipError_t launch_tile_codes(const int8_t* canon_codes, const float* canon_scales, int M, int K,
                             void* tiled_codes, int fmt, float* gm_scales, int ld, hipStream_t s);

// packed nibbles -> bf16 weight operands in the tiled bf16 layout
hipError_t launch_expand_weights_bf16(const uint8_t* w_codes, int K, int N, uint16_t* out,
                                      hipStream_t s);

// bf16-operand GEMM (codes and expanded weights in the bf16 tiled layout);
// same modes as launch_gemm
hipError_t launch_gemm_bf16(const uint16_t* a_tiled, const float* a_scales_gm, int ld_sa, int M,
                            int K, int N, const uint16_t* w_bf16, const __half* w_scales, int gw,
                            float* y, int32_t* dots, int mode, hipStream_t s);

// GEMM over the internal activation layout.  mode 0: y = rescaled sum;
// mode 1: write int32 per-group dots [M][N][K/32].
hipError_t launch_gemm(const int8_t* a_tiled, const float* a_scales_gm, int ld_sa, int M, int K,
                       int N, const uint8_t* w_codes, const __half* w_scales, int gw, float* y,
                       int32_t* dots, int mode, hipStream_t s);

// status word shared by the synchronizing offline calls
hipError_t reset_status(hipStream_t s);
hipError_t read_status(int* host_status, hipStream_t s);

}  // namespace loopq
