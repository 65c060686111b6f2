/*
 * loopq.h -- C ABI of the looped W4A4 / W4A8 group-quantized linear layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (sources are the pages' titles and the passage used):
 *   - "paper_specification.yaml" of the LoopQ reproduction, lq1_quantization:
 *     Eq.(4) Q_a(x; c) = c * clip(round(x / c), q_min, q_max); symmetric
 *     round-to-nearest; 4-bit weights with 4- or 8-bit activations; group-wise
 *     weights and activations with group size 32.
 *   - the same file, loopq_components: a shared quantized backbone with an
 *     invertible transform folded into the activation and weight sides; LAS
 *     replaces the shared activation clip with one clip per module and loop.
 *   - implementation_status lq2 (clips multiply dynamic token/group absmax
 *     steps) and lq3 (one Kronecker transform shared by all loops, folded
 *     into the weights through its exact inverse transpose, unquantized).
 *   - "LoopQ 4-bit quantization of Ouro-1.4B -- raw artifacts", "The arms":
 *     random orthogonal Kronecker transforms; Ouro-1.4B applies one set of 24
 *     layers four times to every token.
 *   - "Quantizing Looped Transformers: Feedback Exposure and Calibration
 *     Blindness", Figure 3 and Table 6: grouped INT4 weights with g = 128.
 *
 * Readings where the pages are silent: codes are symmetric in
 * [-(2^(b-1)-1), 2^(b-1)-1]; ties round to even; the step of a group is
 * fl32(c * fl32(absmax / qmax)) (weights: fl16(fl32(absmax / 7)), codes use
 * the fp16 step); division is correctly rounded; an all-zero group has step 0
 * and codes 0; groups run along K over the flat row-major index; the
 * transform is x~ = x (P1 kron P2) = vec_r(P1^T X P2), formed with fp32
 * products and fp32 accumulation (within 8 (n1 + n2) 2^-24 |P1|^T |X| |P2| of
 * the exact value per element); codes and steps are Eq.(4) of that x~ exactly.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without waiting, except
 *     where a call says it synchronizes.
 *   - The caller owns every buffer.  Compute calls allocate nothing; scratch
 *     memory comes in through `workspace` (size from loopq_workspace_bytes).
 *   - Arguments are validated on the host before any HIP call; a failed
 *     check returns a negative loopq_status and enqueues nothing.  The
 *     library is fail-closed: an unsupported shape is an error, never a
 *     slower fallback.  A device fault surfaces at the caller's next
 *     synchronization.
 *   - Calls on different streams may run concurrently; they share no
 *     mutable library state except the status word of the synchronizing
 *     offline calls (pack, fold), which must not overlap on one device, and
 *     the auxiliary stream of the pipelined loop-sequential schedule, whose
 *     enqueueing is serialized (its work can then queue behind another
 *     call's).
 *   - Matrices are row-major.  x is [M][K] (one token per row), weights are
 *     stored one output column per row, [N][K]; y is [M][N] fp32.
 */
#ifndef LOOPQ_H
#define LOOPQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOOPQ_ABI_VERSION 2
#define LOOPQ_GROUP_A 32   /* activation group size (lq1_quantization) */
#define LOOPQ_MAX_LOOPS 64 /* largest T accepted by loopq_looped_forward */

typedef enum {
  LOOPQ_OK = 0,
  LOOPQ_ERR_INVALID_ARG = -1, /* null pointer, size <= 0, clip <= 0 or not finite */
  LOOPQ_ERR_UNSUPPORTED = -2, /* K % 32 != 0, n1*n2 != K, n1 or n2 not a multiple of 4
                                 or above 128, bits not 4/8, group_w not 32/128, T > 64,
                                 or a GEMM whose activation steps (rows x K/32 x 4 B) or
                                 weight steps (padded N x groups x 2 B) reach 2 GiB */
  LOOPQ_ERR_ALIGNMENT = -3,   /* a pointer breaks the alignment a call states */
  LOOPQ_ERR_RANGE = -4,       /* a weight step overflows fp16 */
  LOOPQ_ERR_HIP = -5,         /* the HIP runtime reported an error */
  LOOPQ_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required */
  LOOPQ_ERR_SINGULAR = -7     /* a transform factor is not invertible (fold) */
} loopq_status;

typedef enum { LOOPQ_F32 = 0, LOOPQ_BF16 = 1 } loopq_dtype;

typedef enum {
  LOOPQ_SCHED_AUTO = 0,
  LOOPQ_SCHED_LOOP_SEQUENTIAL = 1, /* per t: quantize x_t, then the GEMM */
  LOOPQ_SCHED_WEIGHT_STATIONARY = 2 /* quantize all T*M rows, one pass over the weights */
} loopq_schedule;

typedef enum {
  LOOPQ_OP_LINEAR = 1,
  LOOPQ_OP_LOOPED_FORWARD = 2,
  LOOPQ_OP_FOLD = 3,
  LOOPQ_OP_LOOPED_FORWARD_EX = 4, /* bits_a ignored: enough for 4- and 8-bit loops */
  LOOPQ_OP_HESSIAN = 5,           /* rows as M; T, N and bits_a ignored */
  LOOPQ_OP_QUANT_PER_TOKEN = 6,   /* M, K; T, N and bits_a ignored */
  LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN = 7, /* T, M, K, N, bits_a */
  LOOPQ_OP_RECURRENT_ADAPTER = 8, /* M, N, bits_a (K = 2N implied); T and K ignored */
  LOOPQ_OP_LOOPED_FORWARD_CTA = 9, /* T, M, K, N, bits_a; dtype bytes taken as 4 */
  LOOPQ_OP_LOOPED_FORWARD_HESSIAN = 10 /* T, M, K, N, bits_a */
} loopq_op;

/* ABI version of the loaded library (LOOPQ_ABI_VERSION it was built with). */
int32_t loopq_abi_version(void);

/* Static text for a status code; never NULL. */
const char* loopq_status_string(int32_t status);

/* Bytes of the packed weight codes and steps for a K x N weight with weight
 * group size group_w (32 or 128).  Host only, touches no GPU.  Codes take
 * ceil(N/32)*32 * K/2 bytes; steps ceil(N/32)*32 * ceil(K/group_w) fp16. */
int32_t loopq_packed_weight_bytes(int32_t K, int32_t N, int32_t group_w,
                                  size_t* codes_bytes_host, size_t* scales_bytes_host);

/* Workspace bytes an op needs (host only).  LINEAR: T ignored.
 * LOOPED_FORWARD: T loops.  FOLD: pass n1 as M and n2 as N; T, K and bits_a
 * are ignored.  The size is a multiple of 256. */
int32_t loopq_workspace_bytes(int32_t op, int32_t T, int32_t M, int32_t K, int32_t N,
                              int32_t bits_a, size_t* bytes_host);

/* a0 -- fold the transform into the weights (offline).
 * Page: paper_specification.yaml, loopq_components.shared_transformed_backbone
 * and implementation_status lq3 (the weights absorb the exact inverse
 * transpose of the transform, before any quantization).  w [N][K] fp32 holds one output column per row; for each row
 * w_folded[n] = vec_r(P1^-1 * reshape(w[n], n1, n2) * P2^-T), computed in
 * fp64 with the factors inverted on the GPU (Gauss-Jordan, partial pivoting)
 * and rounded once to fp32.  P1 is n1 x n1 and P2 is n2 x n2 fp32, n1*n2 = K,
 * n1, n2 <= 128.  Needs loopq_workspace_bytes(LOOPQ_OP_FOLD, 0, n1, K, n2, 0, ...).
 * Synchronizes `stream`; returns LOOPQ_ERR_SINGULAR for a singular factor. */
int32_t loopq_fold_weights(const float* w, int32_t K, int32_t N,
                           const float* P1, int32_t n1, const float* P2, int32_t n2,
                           float* w_folded, void* workspace, size_t workspace_bytes,
                           void* stream);

/* a1 -- INT4 weight packing (offline).
 * Page: Eq.(4) with clip 1 (lq1_quantization), group-wise W4; g = 128 from
 * "Quantizing Looped Transformers", Figure 3.  For output column n and K-group
 * j of size group_w (the last group may be short): s = fl16(fl32(absmax / 7)),
 * q = clamp(rint(fl32(w / s)), -7, 7), 0 when s == 0.
 * w_folded [N][K] fp32 (K % 32 == 0).  w_codes and w_scales receive an opaque,
 * kernel-tiled layout (sizes from loopq_packed_weight_bytes, 16-byte aligned);
 * loopq_export_weights recovers canonical codes and steps.
 * Synchronizes `stream`; returns LOOPQ_ERR_RANGE if a step overflows fp16. */
int32_t loopq_pack_weights(const float* w_folded, int32_t K, int32_t N, int32_t group_w,
                           void* w_codes, void* w_scales, void* stream);

/* a2-a4 -- transform + dynamic group absmax + LAS clip + RTN of activations.
 * Page: Eq.(4) (lq1_quantization); LAS (loopq_components.las, lq2); the
 * Kronecker transform (lq3).  x [M][K] in `dtype` (fp32 or bf16, 4-byte
 * aligned); P1 [n1][n1], P2 [n2][n2] fp32 or both NULL for no transform.
 * For row m and group j of 32: s = fl32(clip * fl32(absmax / qmax)),
 * codes[m][k] = clamp(rint(fl32(x~ / s)), -qmax, qmax) (0 when s == 0),
 * scales[m][j] = s; qmax = 7 (bits_a 4) or 127 (bits_a 8).
 * codes int8 [M][K]; scales fp32 [M][K/32]; xt_out (nullable) receives x~
 * [M][K] fp32, the values that were quantized. */
int32_t loopq_quant_act(const void* x, int32_t dtype, int32_t M, int32_t K,
                        const float* P1, int32_t n1, const float* P2, int32_t n2,
                        float clip, int32_t bits_a,
                        int8_t* codes, float* scales, float* xt_out, void* stream);

/* a2-a5 -- one quantized linear: quant_act, then the integer GEMM with the
 * per-group rescale y[m][n] = sum_j s_a[m][j] * s_w[n][32j/group_w] * d[m][n][j],
 * d the exact int32 dot of group j.  bits_a 4 is W4A4, 8 is W4A8.
 * w_codes/w_scales from loopq_pack_weights with the same K, N, group_w.
 * y [M][N] fp32.  Workspace: loopq_workspace_bytes(LOOPQ_OP_LINEAR, ...). */
int32_t loopq_w4a4_linear(const void* x, int32_t dtype, int32_t M, int32_t K, int32_t N,
                          const float* P1, int32_t n1, const float* P2, int32_t n2,
                          float clip, int32_t bits_a,
                          const void* w_codes, const void* w_scales, int32_t group_w,
                          float* y, void* workspace, size_t workspace_bytes, void* stream);

/* loopq_w4a4_linear without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It runs the kernels of
 * loopq_w4a4_linear on a fixed scratch array the library holds on each
 * device it runs on (loopq_noalloc_scratch_bytes() bytes, 64 MiB, kept
 * until the process ends) and calls no allocating routine; the timing
 * hooks record nothing for it.  The same arguments, errors and results as
 * loopq_w4a4_linear (bitwise: same kernels, same layout); a call whose
 * loopq_workspace_bytes(LOOPQ_OP_LINEAR, 1, M, K, N, bits_a) exceeds the
 * scratch returns LOOPQ_ERR_WORKSPACE before any launch (e.g. M * K above
 * roughly 40 M elements at N = K).  Every call on one device shares that
 * device's scratch and leaves the last call's contents there: calls that
 * overlap on one device (different streams or threads) race and must be
 * ordered by the caller. */
int32_t loopq_w4a4_linear_noalloc(const void* x, int32_t dtype, int32_t M, int32_t K, int32_t N,
                                  const float* P1, int32_t n1, const float* P2, int32_t n2, float clip,
                                  int32_t bits_a, const void* w_codes, const void* w_scales, int32_t group_w,
                                  float* y, void* stream);

/* Bytes of the fixed scratch of loopq_w4a4_linear_noalloc (host only). */
size_t loopq_noalloc_scratch_bytes(void);

/* Per-token activation steps: the same RTN with one step per token.
 * Page: "LoopQ 4-bit quantization of Ouro-1.4B -- raw artifacts", "The arms"
 * (rtn_w4a4_per_token: plain RTN, one step per token, a common W4A4 reference).  Eq.(4)
 * over the whole row of x~ (x with no transform): for row m,
 * s = fl32(clip * fl32(absmax_m / qmax)), codes[m][k] = clamp(rint(fl32(x~ / s)),
 * -qmax, qmax) (0 when s == 0), with the arithmetic of loopq_quant_act.
 * codes int8 [M][K]; scales fp32 [M][K/32]: the row's one step written to each
 * of its K/32 group slots, so loopq_gemm_codes consumes the pair unchanged.
 * xt_out (nullable) receives x~.  Arguments and errors as loopq_quant_act.
 * With a transform, each row's absmax is taken over the x~ row the transform
 * kernel holds on chip (one launch; x~ reaches memory only through xt_out).
 * The call needs no workspace: workspace and workspace_bytes are accepted and
 * ignored (loopq_workspace_bytes(LOOPQ_OP_QUANT_PER_TOKEN, ...) returns 0). */
int32_t loopq_quant_act_per_token(const void* x, int32_t dtype, int32_t M, int32_t K,
                                  const float* P1, int32_t n1, const float* P2, int32_t n2,
                                  float clip, int32_t bits_a, int8_t* codes, float* scales,
                                  float* xt_out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* The loop with per-token activation steps: for each loop t,
 * loopq_quant_act_per_token of x_t with the loop's clip clips_host[t], then
 * the GEMM of loopq_gemm_codes against the same packed weights,
 * y_t = sum_j s_a[m] * s_w[n][32j/group_w] * d[m][n][j] (= s_a[m] * sum_j s_w * d
 * up to fp32 rounding order).  Page as above; the loop as for
 * loopq_looped_forward.  All T*M rows run weight-stationary (one pass over
 * the weights); T = 1 is one linear.  x [T][M][K], y [T][M][N]; other
 * arguments and errors as loopq_looped_forward.  Workspace:
 * loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, T, M, K, N, bits_a, ...). */
int32_t loopq_looped_forward_per_token(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                                       int32_t N, const float* P1, int32_t n1, const float* P2,
                                       int32_t n2, const float* clips_host, int32_t bits_a,
                                       const void* w_codes, const void* w_scales, int32_t group_w,
                                       float* y, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* a6 -- the loop: the same packed weights applied at every loop t with the
 * loop's own clip.  Page: "LoopQ 4-bit quantization of Ouro-1.4B -- raw
 * artifacts" (each token passes through the same 24 layers four times); LAS,
 * one clip per module and loop.
 * x [T][M][K], y [T][M][N]; clips_host [T] (host memory, read before return).
 * schedule: a loopq_schedule.  LOOP_SEQUENTIAL quantizes and multiplies loop
 * by loop, pipelined: the quantizer of loop t + 1 runs on an auxiliary stream
 * the library keeps per device (default priority) while the GEMM of loop t
 * runs on `stream`; `stream` waits for the auxiliary work through events, so
 * the call keeps stream order for the caller (and can be captured into a HIP
 * graph).  WEIGHT_STATIONARY quantizes all T*M rows, then streams the weights
 * once for all loops; AUTO picks WEIGHT_STATIONARY.  A launch of at most 16
 * rows (T*M, or M per loop) takes the small-row (decode) kernel, which reads
 * the packed weights directly and forms the group dots on the VALU; larger
 * ones take the MFMA GEMM.  Codes and steps are the same either way; y is
 * deterministic and equal between schedules up to fp32 summation order
 * (bitwise when both launch the same kernel).
 * Workspace: loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, ...). */
int32_t loopq_looped_forward(const void* x, int32_t dtype, int32_t T, int32_t M,
                             int32_t K, int32_t N,
                             const float* P1, int32_t n1, const float* P2, int32_t n2,
                             const float* clips_host, int32_t bits_a,
                             const void* w_codes, const void* w_scales, int32_t group_w,
                             float* y, int32_t schedule,
                             void* workspace, size_t workspace_bytes, void* stream);

/* a6 with loop-dependent pieces.  Loop t uses weight/transform set
 * sets_host[t] (0 <= set < nsets) and activation bit width bits_host[t] (4 or 8).
 * Pages: SLT ("paper_specification.yaml", loopq_components.slt, Section 4.2,
 * Eqs. (5)-(6): the transform and weight groups that SLT picks vary with the
 * loop, the rest stay shared, i.e. one set for every loop) and a loop-wise
 * activation precision
 * allocation ("Quantisation errors can keep returning inside a looped model",
 * "Three components address three sources of mismatch").  x, y, clips_host and
 * the other arguments as for loopq_looped_forward.  Set s has factors
 * P1_sets_host[s] (n1 x n1) and P2_sets_host[s] (n2 x n2), device pointers held
 * in host arrays of nsets entries (both arrays NULL: no transform for any set),
 * and packed weights w_codes_sets_host[s] / w_scales_sets_host[s] from
 * loopq_pack_weights with the same K, N, group_w.  Each maximal run of
 * consecutive loops with the same set and bit width runs weight-stationary
 * (one pass over that set's weights for all of the run's rows), so one set for
 * every loop is exactly loopq_looped_forward's weight-stationary schedule.
 * When every loop has the same bit width, M % 64 == 0 and T * M > 16, the
 * runs share one grouped GEMM launch over all T * M rows instead, each loop's
 * rows multiplied by its own set's weights (the same bits as separate calls).
 * Workspace: loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD_EX, T, M, K, N, 0, ...)
 * (room for the W4A4 operands of up to T weight sets).
 * Errors: a set index outside [0, nsets), a bit width other than 4 or 8, or a
 * NULL set entry return LOOPQ_ERR_INVALID_ARG / LOOPQ_ERR_UNSUPPORTED before
 * any launch; the shape and transform checks are those of loopq_looped_forward. */
int32_t loopq_looped_forward_ex(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                                int32_t N, int32_t nsets, const float* const* P1_sets_host, int32_t n1,
                                const float* const* P2_sets_host, int32_t n2,
                                const void* const* w_codes_sets_host,
                                const void* const* w_scales_sets_host, int32_t group_w,
                                const int32_t* sets_host, const int32_t* bits_host,
                                const float* clips_host, float* y, void* workspace,
                                size_t workspace_bytes, void* stream);

/* a6 with the trajectory Hessian as a side output: the looped forward of
 * loopq_looped_forward (same arguments, schedules and results: y is bitwise
 * that call's whenever that call takes the quantizer and the GEMM, i.e. for
 * more than 16 rows per launch; here the few-row kernel is never used) whose
 * quantizer also writes the x~ it quantizes, fp32 [T][M][K], into the
 * workspace, followed by H += x~^T x~ over all T*M rows as
 * loopq_hessian_accumulate computes it (bitwise the same H), so no second
 * transform pass is made.  Page as for loopq_hessian_accumulate: the N-step
 * calibration Hessian summed over the recurrence steps.  After the call the
 * x~ rows stay in the workspace at byte offset
 * loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, bits_a) rounded
 * up to a multiple of 256.  H fp32 [K][K] (4-byte aligned), accumulated in
 * place; K <= 65536 and T*M <= 2^30 as for loopq_hessian_accumulate.
 * Workspace: loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD_HESSIAN, T, M, K, N,
 * bits_a, ...).  Other errors as loopq_looped_forward. */
int32_t loopq_looped_forward_hessian(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                                     int32_t N, const float* P1, int32_t n1, const float* P2, int32_t n2,
                                     const float* clips_host, int32_t bits_a, const void* w_codes,
                                     const void* w_scales, int32_t group_w, float* y, int32_t schedule,
                                     float* H, void* workspace, size_t workspace_bytes, void* stream);

/* CTA, one loop transition on M rows: out = a * h + b + eta * U (V^T h) per
 * row.  Page: "paper_specification.yaml", loopq_components.cta (Section 4.3,
 * Eq.(7), not printed there: an affine plus gated low-rank adapter applied
 * only at loop transitions, U and V shared, a_t, b_t and eta_t per
 * transition), experiment_hyperparameters cta_rank 8; identity (a = 1,
 * b = 0, eta = 0) is the untrained arm's CTA ("LoopQ 4-bit quantization of
 * Ouro-1.4B -- raw artifacts", "The arms").
 * h, out [M][K] in `dtype` (16-byte aligned; out may be h itself, any other
 * overlap is an error); U, V [K][rank] fp32 row-major, a, b [K] fp32 (device
 * memory, 4-byte aligned); eta a host scalar.  V^T h is accumulated in fp32
 * in a fixed order (deterministic); the result is formed as
 * fma(eta, sum_j U[k][j] z_j, fma(a_k, h_k, b_k)) and stored in `dtype`
 * (bf16: round to nearest, ties to even).  K % 32 == 0 and 1 <= rank <= 16,
 * else LOOPQ_ERR_UNSUPPORTED; M == 0 is a no-op. */
int32_t loopq_cta_apply(const void* h, int32_t dtype, int32_t M, int32_t K, const float* U,
                        const float* V, int32_t rank, const float* a, const float* b, float eta,
                        void* out, void* stream);

/* a6 with CTA at the loop transitions: loop 0 reads x_0; loop t >= 1 reads
 * transition t - 1 of loopq_cta_apply applied to x_t (a_sets + (t-1) K,
 * b_sets + (t-1) K, eta_host[t-1]), stored in the input's type.  Pages as
 * for loopq_cta_apply and loopq_looped_forward.  The adapted loop inputs
 * (and a copy of loop 0) are written to the workspace after the region
 * loopq_looped_forward uses, then that path runs on them with the same
 * schedule; a_sets, b_sets [T-1][K] and U, V as for loopq_cta_apply (unused
 * when T == 1), eta_host [T-1] host memory.  Other arguments and errors as
 * loopq_looped_forward.  Workspace:
 * loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD_CTA, T, M, K, N, bits_a, ...),
 * whose first loopq_workspace_bytes(LOOPQ_OP_LOOPED_FORWARD, ...) bytes are
 * laid out as loopq_looped_forward's (loopq_export_act_codes reads them). */
int32_t loopq_looped_forward_cta(const void* x, int32_t dtype, int32_t T, int32_t M, int32_t K,
                                 int32_t N, const float* P1, int32_t n1, const float* P2, int32_t n2,
                                 const float* clips_host, int32_t bits_a, const void* w_codes,
                                 const void* w_scales, int32_t group_w, float* y, int32_t schedule,
                                 const float* U, const float* V, int32_t rank, const float* a_sets,
                                 const float* b_sets, const float* eta_host, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* A dependent recurrence through one quantized linear (the adapter loop).
 * Page: "Quantizing Looped Transformers: Feedback Exposure and Calibration
 * Blindness", Figure 4 (the Huginn recurrence loop): the adapter reads the
 * state concatenated with the embedding, cat(s_t, e), and its output enters the
 * recurrence directly, with no skip connection around it.  With the
 * recurrent blocks between two adapter calls left out, loop t computes
 * s_{t+1} = y_t = the quantized linear (loopq_w4a4_linear, clip clips_host[t])
 * of x_t = cat(s_t, e), so every loop's input is the previous loop's output.
 * s0, e [M][N] fp32 (16-byte aligned), N % 16 == 0; the weight is [N][2N]
 * (K = 2N), packed by loopq_pack_weights; y [T][M][N] fp32 receives
 * s_1 .. s_T (loop t + 1 reads y[t] after loop t wrote it, in stream order).
 * Each loop is one call of the single-linear path (the few-row kernel up to
 * 16 rows, else quantizer and GEMM) after a device-side concatenation; no
 * host synchronization between loops, so the sequence can be captured into a
 * HIP graph.  Workspace: loopq_workspace_bytes(LOOPQ_OP_RECURRENT_ADAPTER, 0,
 * M, 0, N, bits_a, ...).  Errors as loopq_looped_forward. */
int32_t loopq_recurrent_adapter(const float* s0, const float* e, int32_t T, int32_t M, int32_t N,
                                const float* P1, int32_t n1, const float* P2, int32_t n2,
                                const float* clips_host, int32_t bits_a, const void* w_codes,
                                const void* w_scales, int32_t group_w, float* y, void* workspace,
                                size_t workspace_bytes, void* stream);

/* a5 alone -- the GEMM on activation codes and steps already formed.
 * a_codes int8 [M][K], a_scales fp32 [M][K/32] (the layouts loopq_quant_act
 * writes); same weights and output as loopq_w4a4_linear.  bits_a selects
 * the kernel as in the linear: 4 (every code must lie in [-7, 7]; codes
 * outside give unspecified results) or 8 ([-127, 127]); M <= 16 takes the
 * small-row kernel. */
int32_t loopq_gemm_codes(const int8_t* a_codes, const float* a_scales, int32_t M, int32_t K,
                         int32_t N, const void* w_codes, const void* w_scales, int32_t group_w,
                         int32_t bits_a, float* y, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Trajectory Hessian accumulation: H += xt^T xt.
 * Page: "Quantizing Looped Transformers: Feedback Exposure and Calibration
 * Blindness" -- N-step GPTQ calibration accumulates the input Hessian over the
 * recurrence steps, H = sum_t X_t^T X_t (Tables 19 and 25; Table 1 reports the
 * rank of such Hessians at a 1e-3 lambda_max threshold); the GPTQ memory note
 * of the same page set keeps one fp32 [in][in] Hessian per linear.  Passing
 * the x~ rows of every loop t (the values the forward quantizes, e.g. the
 * xt_out of loopq_quant_act) in one or several calls accumulates that sum for
 * the transformed linear.
 * xt fp32 [rows][K] (16-byte aligned); H fp32 [K][K] (4-byte aligned), read and
 * written in place: H[i][j] += sum_r xt[r][i] * xt[r][j] for all i, j.  Each
 * value is formed once for i <= j (fp32 products, fp32 accumulation) and
 * stored at both (i, j) and (j, i), so a symmetric H stays exactly symmetric.
 * The summation order depends only on (rows, K): results are deterministic.
 * rows == 0 returns LOOPQ_OK at once (any pointers).  K % 32 == 0, K <= 65536,
 * rows <= 2^30.
 * Workspace: loopq_workspace_bytes(LOOPQ_OP_HESSIAN, 0, rows, K, 0, 0, ...)
 * (64 MiB; the size depends on K only).
 * Two calls on one H must not overlap, nor two calls sharing a workspace;
 * xt must not alias H. */
int32_t loopq_hessian_accumulate(const float* xt, int32_t rows, int32_t K, float* H, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Test export: canonical weight codes int8 [N][K] and steps fp16 [N][ceil(K/group_w)]
 * (raw binary16 bits) from the packed layout. */
int32_t loopq_export_weights(const void* w_codes, const void* w_scales, int32_t K, int32_t N,
                             int32_t group_w, int8_t* codes, uint16_t* scales, void* stream);

/* Test export: canonical weight codes int8 [N][K] from the packed layout
 * (loopq_export_weights without the steps). */
int32_t loopq_export_weight_codes(const void* w_codes, int32_t K, int32_t N, int32_t group_w, int8_t* codes,
                                  void* stream);

/* Test export: the activation codes and steps that the last forward call on
 * `workspace` (the same op, T, M, K, N, bits_a and schedule) left there and its
 * product consumed, in canonical form: codes int8 [T*M][K], steps fp32
 * [T*M][K/32] (16-byte aligned codes, 4-byte aligned steps).  Page: Eq.(4)
 * (lq1_quantization) -- these are the codes and steps to compare with it.
 *   op LOOPQ_OP_LOOPED_FORWARD (loopq_looped_forward, either schedule),
 *      LOOPQ_OP_LINEAR (loopq_w4a4_linear, T = 1),
 *      LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN (loopq_looped_forward_per_token),
 *      LOOPQ_OP_RECURRENT_ADAPTER (loopq_recurrent_adapter, T = 1 here: the
 *      last loop's codes; K is ignored, 2N is used).
 * The GEMM paths keep W4A4 codes as e2m3 fp6 MFMA operands and W4A8 codes as
 * int8 tiles; both are decoded here (an fp6 field that is not a code -7..7
 * comes back as -128).  The few-row path (at most 16 rows per launch) writes
 * the codes it formed on chip to the workspace in canonical form.
 * Workspace as the forward call sized it (loopq_workspace_bytes of the op). */
int32_t loopq_export_act_codes(const void* workspace, size_t workspace_bytes, int32_t op, int32_t T, int32_t M,
                               int32_t K, int32_t N, int32_t bits_a, int32_t schedule, int8_t* codes,
                               float* scales, void* stream);

/* Test export: the exact int32 per-group dots d[m][n][j] = sum_{k in group j}
 * a_codes[m][k] * w[n][k], computed by the MFMA path of the bits_a kernel
 * (4: fp6 operands, codes in [-7, 7]; 8: INT8 operands; M <= 16: the
 * small-row kernel's VALU dots, as the forward uses), [M][N][K/32].
 * a_codes int8 [M][K]; workspace as for loopq_workspace_bytes(LOOPQ_OP_LINEAR,
 * 1, M, K, N, bits_a). */
int32_t loopq_group_dots(const int8_t* a_codes, int32_t M, int32_t K, int32_t N, int32_t bits_a,
                         const void* w_codes, int32_t* dots, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Measurement hooks (tracing).  While enabled, every hot-path kernel launch is
 * bracketed by a pair of HIP events recorded on the launch's own stream, so
 * kernel durations can be read without a profiler.  Kernel ids: */
typedef enum {
  LOOPQ_KERNEL_QUANT_TRANSFORM = 0, /* fused transform + quantizer */
  LOOPQ_KERNEL_QUANT_PLAIN = 1,     /* quantizer without transform */
  LOOPQ_KERNEL_GEMM = 2,            /* integer GEMM + rescale */
  LOOPQ_KERNEL_DECODE = 3,          /* few-row linear: transform, quantizer and product in one launch */
  LOOPQ_KERNEL_HESSIAN = 4,         /* trajectory Hessian accumulation (one record per call) */
  LOOPQ_KERNEL_QUANT_TOKEN = 5,     /* per-token quantizer */
  LOOPQ_KERNEL_CTA = 6              /* CTA loop-transition adapter */
} loopq_kernel_id;

/* Turn the hooks on (1) or off (0).  Host only; cheap. */
int32_t loopq_timing_enable(int32_t on);

/* Sum, per kernel id k < n, the elapsed milliseconds and the number of
 * launches recorded since the last read or reset, into ms_host[k] and
 * launches_host[k]; then forget the records.  Waits for the recorded events. */
int32_t loopq_timing_read(int32_t n, double* ms_host, int64_t* launches_host);

/* Forget all records (waits for outstanding events). */
int32_t loopq_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* LOOPQ_H */
