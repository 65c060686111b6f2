// Internal declarations shared by the HIP translation units of libloopq.
// Layouts, argument structs and the host-side launchers each kernel file
// provides.  Nothing here is part of the public C ABI (include/loopq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <string.h>

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
// fp6 variant, W4A4 only (operands of V_MFMA_SCALE_F32_32X32X64_F8F6F4 in
// the e2m3 format, which holds the codes -7..7 exactly): block (mb, p) of 32
// rows x one pair of groups (2p, 2p + 1) starts at byte (mb * Gp + p) * 1536,
// Gp = ceil(Ga / 2); lane slot l = row % 32 + 32 * (group % 2) holds that
// row's 32 codes of the group in 24 bytes at l * 24, code i at bits 6i..6i+5
// (little endian).  A wave's 24-byte-per-lane load of a block is the MFMA
// operand whose K-halves are the two groups.  Expanded weights use the same
// layout with output columns in place of rows.  With Ga odd the second half
// of the last pair is never multiplied by anything but zero; it may hold any
// bits (every e2m3 pattern is finite).
// ---------------------------------------------------------------------------
enum CodeFormat { kCodesCanonical = 0, kCodesTiledI8 = 1, kCodesTiledF6 = 2 };
constexpr int kF6BlockBytes = 1536;
__host__ __device__ inline int64_t group_pairs(int64_t K) { return (K / 32 + 1) / 2; }

// e2m3 patterns of four codes in [-7, 7] given one per byte (two's
// complement; only the low nibble of each byte is read), packed as 4 x 6
// bits.  Nibbles 0..7 are the codes 0..7; nibbles 9..15 are -7..-1.  Two byte
// lookups (v_perm) by the low 3 bits, then a per-byte select on bit 3.
__device__ __forceinline__ uint32_t e2m3_of_codes4(uint32_t codes) {
  const uint32_t n = codes & 0x0F0F0F0Fu;
  const uint32_t sel = n & 0x07070707u;
  // v_perm picks byte s of {first operand : second operand}, bytes 0..3 from
  // the second.  Codes 0..7: 00 08 10 14 18 1A 1C 1E.
  const uint32_t pos = __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, sel);
  // nibble 8 + i is the code i - 8: i = 1..7 -> -7..-1 (i = 0 does not occur)
  const uint32_t neg = __builtin_amdgcn_perm(0x28303438u, 0x3A3C3E00u, sel);
  const uint32_t b3 = (n >> 3) & 0x01010101u;
  const uint32_t mask = (b3 << 8) - b3;  // 0xFF in the bytes whose code is negative
  const uint32_t f = (neg & mask) | (pos & ~mask);
  return (f & 0x3Fu) | ((f >> 2) & 0xFC0u) | ((f >> 4) & 0x3F000u) | ((f >> 6) & 0xFC0000u);
}

// Store the 24 bits of one 4-code run of row `row`, starting at K index k0,
// into the fp6 tiled layout.  Must be called by all four lanes of an aligned
// quad of lanes holding the four consecutive runs of one 16-code half-group
// (lane % 4 == run position): each of three lanes stores one dword of the
// quad's 12 bytes, taking the next lane's bits through a DPP quad permute.
__device__ __forceinline__ void store_f6_run(void* tiled, int Gp, int row, int k0, uint32_t bits24) {
  const int i = (k0 >> 2) & 3;
  // quad_perm(1, 2, 3, 3): lane i reads lane i + 1
  const uint32_t nxt = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits24, 0xF9, 0xF, 0xF, false);
  if (i == 3) return;
  const uint32_t dw = (bits24 >> (8 * i)) | (nxt << (24 - 8 * i));
  const int j = k0 >> 5;
  const int64_t off = ((int64_t)(row >> 5) * Gp + (j >> 1)) * kF6BlockBytes +
                      ((row & 31) + 32 * (j & 1)) * 24 + ((k0 & 31) >> 4) * 12 + 4 * i;
  *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(tiled) + off) = dw;
}
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
  int per_token;     // 1: one step per row from the row's absmax, written to every group slot
  // transform kernel LDS plan (set by the host launcher)
  int R;             // rows per work chunk
  int sp1, sp2, sx, st;  // LDS strides (elements) of P1, P2, X, T
  int off_p2, off_x, off_t;  // byte offsets in dynamic LDS
  int off_rmax;      // byte offset of the per-row, per-wave absmax partials (per_token)
  int lds_bytes;
  int ws;            // 1: the two-role kernel form (512 threads)
};

// host launchers -------------------------------------------------------------
hipError_t launch_quant_act(QuantArgs a, hipStream_t s);
// one step per row (no transform: a.P1 must be null); the step fills every
// group slot of the row in a.scales
hipError_t launch_quant_token(QuantArgs a, hipStream_t s);
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

// Codes in layout `fmt` (ld: padded rows of the tiled layouts) and steps
// (group-major [K/32][ld] if steps_gm, else row-major [rows][K/32]) back to
// canonical int8 [rows][K] and row-major fp32 steps.  fp6 fields that are not
// a code -7..7 come back as -128.
hipError_t launch_export_act(const void* codes, const float* steps, int rows, int K, int fmt, int ld,
                             int steps_gm, int8_t* out_codes, float* out_steps, hipStream_t s);

// packed nibbles -> fp6 weight operands in the fp6 tiled layout
// (padded_cols(N) / 32 * group_pairs(K) blocks of kF6BlockBytes)
hipError_t launch_expand_weights_f6(const uint8_t* w_codes, int K, int N, void* out, hipStream_t s);

// fp6-operand GEMM (W4A4: codes and expanded weights in the fp6 tiled
// layout); same modes as launch_gemm
// Grouped GEMM: rows [s * rows_per_set, (s + 1) * rows_per_set) take weight
// set s (rows_per_set a multiple of 64, at most 64 sets).
struct GemmSets {
  int rows_per_set = 0;
  int n = 0;
  const void* w[64];
  const __half* sw[64];
};

hipError_t launch_gemm_f6(const void* a_tiled, const float* a_scales_gm, int ld_sa, int M, int K,
                          int N, const void* w_f6, const __half* w_scales, int gw, float* y,
                          int32_t* dots, int mode, hipStream_t s, const GemmSets* sets = nullptr);

// GEMM over the internal activation layout.  mode 0: y = rescaled sum;
// mode 1: write int32 per-group dots [M][N][K/32].
hipError_t launch_gemm(const int8_t* a_tiled, const float* a_scales_gm, int ld_sa, int M, int K,
                       int N, const uint8_t* w_codes, const __half* w_scales, int gw, float* y,
                       int32_t* dots, int mode, hipStream_t s, const GemmSets* sets = nullptr);

// Few-row (decode) linear in one launch: at most kDecodeMaxRows token rows
// of x (quantized in the launch, after an optional transform of one of the
// compiled-in factor shapes) or of canonical codes and steps, times the
// packed weights.  mode 0: y [R][N]; mode 1 (codes only): int32 group dots
// [R][N][K/32].  No workspace.
constexpr int kDecodeMaxRows = 16;
struct DecodeCall {
  const void* x;          // [R][K] fp32 or bf16, or null with codes
  int bf16;
  const int8_t* a_codes;  // canonical codes [R][K] (instead of x)
  const float* a_steps;   // row-major steps [R][K/32]
  const float* P1;        // factors or null
  const float* P2;
  int n1, n2;
  int R, K, N;
  ClipTable clips;        // row r uses clips.c[r / rows_per_clip]
  int rows_per_clip;
  int qmax;
  const uint8_t* w;       // packed weights
  const __half* sw;
  int gw;
  float* y;
  int32_t* dots;
  int mode;
  // nullable: when the launch forms the codes itself (from x), it also
  // writes them here, canonical [R][K], with row-major steps [R][K/32]
  int8_t* codes_out;
  float* steps_out;
};
// true if one launch takes this transform for R rows (a compiled-in factor
// shape, and the transform repeated per work-group cheap enough)
bool decode_transform_fused(int R, int n1, int n2);
// true if the factor shape is compiled in; then launch_decode_items writes x~
// of R rows ([R][K] fp32, bitwise the chunked kernel's) with one work-group
// per (row, 16-column tile of the n1 x n2 grid)
bool decode_transform_items(int n1, int n2);
hipError_t launch_decode_items(const void* x, int bf16, const float* P1, int n1, const float* P2, int n2,
                               int R, float* xt, hipStream_t s);
hipError_t launch_decode(const DecodeCall& c, hipStream_t s);

// status word shared by the synchronizing offline calls
// Trajectory Hessian: H [K][K] += x^T x over `rows` rows of x [rows][K] fp32
// (K % 32 == 0, rows >= 1); `part` holds hessian_workspace_bytes(K) bytes.
constexpr int kHessianMaxK = 65536;
constexpr int kHessianMaxRows = 1 << 30;
size_t hessian_workspace_bytes(int K);
// Raises fn's dynamic-LDS limit on the current device to lds_bytes if it is
// below (never lowers it, so every earlier launch size stays valid) and, if
// asked, reports the device's CU count and fn's resident work-groups per CU
// for blocks of `block` threads at that LDS size (256 CUs and 1 if a query
// fails).  Kept per device and kernel, so only a kernel's first launch at a
// given size pays for the runtime queries.
hipError_t prepare_launch(const void* fn, int lds_bytes, int block, int* per_cu = nullptr, int* ncu = nullptr);
// CU count of the current device (queried once per device; 256 if the query fails)
int device_cu_count();

// Tile form of a rescale-mode GEMM launch (both kernels): 0 whole 128x128
// tiles, 1 the two-way split-K form, 2 the four-way form (gemm_f6.hip).
int gemm_form(int M, int N, int K);

hipError_t launch_hessian(const float* x, int rows, int K, float* H, float* part, hipStream_t s);

// x [M][2N] = cat(s [M][N], e [M][N]) per row (fp32, N % 4 == 0, 16-byte aligned)
hipError_t launch_concat_state(const float* s, const float* e, float* x, int M, int N, hipStream_t st);

// CTA over `rows` rows of K: row i takes transition i / rows_per_tr + first
// (a negative transition copies the row unchanged); a, b [ntr][K], eta [ntr]
// (host), U, V [K][r], 1 <= r <= cta_max_rank(), K % 32 == 0
hipError_t launch_cta(const void* h, int bf16, int64_t rows, int K, const float* U, const float* V, int r,
                      const float* a, const float* b, const float* eta, int ntr, int64_t rows_per_tr, int first,
                      void* out, hipStream_t s);
int cta_max_rank();

hipError_t reset_status(hipStream_t s);
hipError_t read_status(int* host_status, hipStream_t s);

}  // namespace loopq
