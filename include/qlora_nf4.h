/*
 * qlora_nf4.h -- C ABI of the QLoRA NF4 hot path for one AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes three things the pages define:
 *
 *  1. Blockwise NF4 quantisation with double quantisation (DQ).
 *     Page "QLoRA: NF4 storage, gradients and local integration" (dineshblog),
 *     section "Exact CPU teaching quantizer and adapter gradient path":
 *     blocks of 64 consecutive weights, scale = max|w| per block, nearest
 *     level of the 16-entry NF4 table (first one on ties), two 4-bit codes
 *     per byte with the even element in the low nibble, a zero block divided
 *     by 1.  Section "Double quantization: correct the scale arithmetic" of
 *     the same page and "QLoRA Deep Dive: 4-bit NormalFloat & Double
 *     Quantization Internals" (devtechtools), section "2. Squeezing More
 *     Memory: Double Quantization (DQ)": the fp32 block scales are stored as
 *     8-bit floats, one fp32 second-level scale per 256 of them, plus an
 *     offset.  Readings where the pages are silent: the 8-bit code is OCP FP8
 *     E4M3FN (round to nearest even, saturating at 448); one fp32 offset mu
 *     per tensor = mean of its block scales (fixed fp64 stride-halving tree:
 *     per 256 scale slots, then over the group sums padded to a power of
 *     two); s2 = C2 / 448 with C2 = max|s_b - mu| over the group.
 *
 *  2. The frozen-base QLoRA linear, row-batch form (page 2, paragraph after
 *     the listing; course notebook FT-02, "LoRALinear from scratch"):
 *        Y = X Qhat(W)^T + s (X A^T) B^T,   s = alpha / r.
 *
 *  3. Its backward (page 2, same paragraph): with upstream gradient G,
 *        dX = G Qhat(W) + s (G B) A,  dB = s G^T (X A^T),  dA = s (G B)^T X.
 *     W is frozen: no weight gradient is formed.
 *
 * Data layout (format v1, part of the ABI):
 *   W       fp32 [rows = d_out, cols = d_in], row-major; N = rows * cols.
 *   nb      = ceil(N / 64) first-level blocks, over the flattened W.
 *   ng      = ceil(nb / 256) DQ groups.
 *   packed  uint8 [32 * nb]: byte j holds code 2j (bits 0..3) and code 2j+1
 *           (bits 4..7); padding weights of the last block are zero (code 7).
 *   qscale  uint8 [nb]: E4M3FN codes of (s_b - mu) / s2_g.
 *   scale2  fp32  [ng]: s2_g.
 *   offset  fp32  [1] : mu.
 *   Dequantized weight: w' = RN32(L[c] * s'), s' = fmaf(e4m3(q), s2, mu).
 *   X, A, B, G (= dY), Y, dX are bf16 (passed as uint16_t bit patterns),
 *   row-major: X [M, cols], A [r, cols], B [rows, r], G and Y [M, rows],
 *   dX [M, cols].  u = X A^T and v = G B are fp32 [M, r]; dA fp32 [r, cols];
 *   dB fp32 [rows, r].  Accumulation is fp32; Y and dX are rounded to bf16.
 *
 * Conventions:
 *   - Every buffer argument is a device pointer owned by the caller (except
 *     the qn_nf4dq struct itself, which lives in host memory and holds
 *     device pointers).  The library allocates nothing; scratch memory comes
 *     from the caller as `workspace` (sizes from the *_workspace functions;
 *     256-byte aligned).  Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL: the null stream).  All calls are
 *     stream-ordered and asynchronous, except nf4_quantize_dq without a
 *     `nonfinite` flag pointer, which synchronizes `stream` so that it can
 *     report non-finite input in its return value.
 *   - Arguments are checked on the host before any launch; on error nothing
 *     is launched.  QN_EINVAL: bad size or null required pointer;
 *     QN_EALIGN: misaligned pointer; QN_EWORKSPACE: workspace too small;
 *     QN_EDEVICE: a HIP runtime call failed (no device, launch failure).
 *   - Calls that overlap on one stream are ordered; calls on different
 *     streams that share a workspace race.  Calls on different streams with
 *     their own workspaces are independent: the library keeps no mutable
 *     state of its own.
 *   - Linear workspaces (qlora_linear_workspace) begin with QN_ARRIVAL_BYTES
 *     of arrival counters, through which the workgroups of one launch learn
 *     which of them finishes a reduction.  They must be zero before the
 *     workspace is first used (allocate it zeroed, or clear it once); every
 *     call leaves them at zero when it completes, so a workspace may then
 *     serve any number of calls, of any shape, on one stream.  The backward
 *     also clears them in its first kernel.  nf4_quantize_dq leaves the same
 *     bytes of its workspace untouched, so one buffer may serve all calls.
 *   - Sizes the linear calls accept: M <= 2^23 rows, rows and cols <= 2^20
 *     (QN_EINVAL beyond).
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QN_ABI_VERSION 4

/* Bytes of arrival counters at the start of a linear workspace. */
#define QN_ARRIVAL_BYTES 4096

typedef enum {
  QN_OK = 0,
  QN_EINVAL = 1,
  QN_ENONFINITE = 2,
  QN_EALIGN = 3,
  QN_EWORKSPACE = 4,
  QN_EDEVICE = 5
} qn_status;

typedef enum { QN_F32 = 0, QN_BF16 = 1 } qn_dtype;

/* Codebooks of the 4-bit codes (qn_nf4dq.codebook). */
#define QN_CODE_NF4 0 /* the NF4 table above                                  */
#define QN_CODE_FP4 1 /* FP4 (course notebook FT-02, "Exercise 3: NF4 vs FP4 at
                         equal memory"): E2M1 levels {0, 0.0625, 2, 3, 4, 6, 8,
                         12} / 12 in fp32; code = sign (bit 3) | magnitude index;
                         nearest magnitude, ties to the lower                 */

/* A quantized weight (device pointers, host struct).  With absmax == NULL
 * the block scales are double quantized (qscale, scale2, offset: format v1
 * above); with absmax != NULL double quantization is off (course notebook
 * FT-02, "Guided example 3: double quantization"): absmax [nb] holds the
 * fp32 block scales and qscale, scale2, offset are ignored (4.5 bits per
 * weight against 4.127).  codebook: QN_CODE_NF4 (zero-initialised structs
 * are NF4) or QN_CODE_FP4.  Every call and every route of the linear calls
 * takes every state (only the level table and the source of the block
 * scales differ). */
typedef struct {
  const uint8_t* packed; /* [32*nb] */
  const uint8_t* qscale; /* [nb]    */
  const float* scale2;   /* [ng]    */
  const float* offset;   /* [1]     */
  int64_t rows;          /* d_out   */
  int64_t cols;          /* d_in    */
  const float* absmax;   /* [nb] fp32 block scales (double quantization off), or NULL */
  int32_t codebook;      /* QN_CODE_NF4 or QN_CODE_FP4 */
} qn_nf4dq;

/* ABI version of the loaded library (QN_ABI_VERSION). */
int qn_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* qn_status_str(qn_status s);

/* The 16 NF4 levels the library uses, as fp32, into host memory. */
void qn_nf4_codebook(float out[16]);

/* The 16 FP4 code values the library uses (QN_CODE_FP4), as fp32, into host
 * memory. */
void qn_fp4_codebook(float out[16]);

/* Workspace bytes needed by nf4_quantize_dq for a rows x cols weight. */
size_t nf4_quantize_dq_workspace(int64_t rows, int64_t cols);

/* Quantize W [rows, cols] fp32 to NF4 with double quantisation (see top of
 * file for the steps and the state layout).  rows, cols >= 1; W 16-byte
 * aligned.  Writes packed [32*nb], qscale [nb], scale2 [ng], offset [1].
 * Non-finite input (a NaN or an infinity in W; the outputs are then
 * unspecified) is reported in one of two ways:
 *   nonfinite == NULL: the call synchronizes `stream` and returns
 *     QN_ENONFINITE;
 *   nonfinite = a device int (4-byte aligned): the call stays asynchronous
 *     and writes 1 (non-finite input) or 0 there, stream-ordered; the caller
 *     must read it before trusting the state. */
qn_status nf4_quantize_dq(const float* W, int64_t rows, int64_t cols, uint8_t* packed,
                          uint8_t* qscale, float* scale2, float* offset, int* nonfinite,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Blockwise 4-bit quantization with a choice of codebook and of double
 * quantization: nf4_quantize_dq is (QN_CODE_NF4, double_quant = 1).  With
 * double_quant != 0 writes packed, qscale, scale2, offset (absmax may be
 * NULL); with double_quant == 0 writes packed and absmax [nb] fp32 (qscale,
 * scale2, offset may be NULL).  Same blocks, codes search rule, workspace
 * (nf4_quantize_dq_workspace) and non-finite reporting as nf4_quantize_dq. */
qn_status qn_quantize(const float* W, int64_t rows, int64_t cols, int codebook,
                      int double_quant, uint8_t* packed, uint8_t* qscale, float* scale2,
                      float* offset, float* absmax, int* nonfinite, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Dequantize w into out [rows, cols]: fp32 (QN_F32) or bf16 bit patterns
 * (QN_BF16, round to nearest even of the fp32 value). */
qn_status nf4_dequantize(const qn_nf4dq* w, qn_dtype out_dtype, void* out, void* stream);

/* Workspace bytes needed by qlora_linear_fwd (backward == 0) or
 * qlora_linear_bwd (backward != 0) for M rows of activations (at least
 * QN_ARRIVAL_BYTES; the first QN_ARRIVAL_BYTES must be zero before first
 * use, see the conventions above). */
size_t qlora_linear_workspace(int64_t M, int64_t rows, int64_t cols, int r, int backward);

/* Forward: y [M, rows] bf16 = X Qhat(W)^T + (alpha/r) (X A^T) B^T.
 * cols must be a multiple of 64 and rows a multiple of 8 (so that every row
 * of X, G and W starts 16-byte aligned); 1 <= r <= 64; M >= 0 (M == 0: no
 * work).
 * u_out (nullable) receives u = X A^T, fp32 [M, r], for the backward. */
qn_status qlora_linear_fwd(const qn_nf4dq* w, const uint16_t* x, int64_t M, const uint16_t* A,
                           const uint16_t* B, int r, float alpha, uint16_t* y, float* u_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* The forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, results and
 * routes as qlora_linear_fwd (bit-identical output), but its scratch memory
 * is a file-scope device array of QN_STATIC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; the call allocates
 * nothing.  Sizes whose forward needs more scratch than that (the large-
 * batch route, which keeps a bf16 copy of the weight) return QN_EWORKSPACE.
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (other streams, other threads) race.  The array keeps what the
 * last call left in it; the call clears what must start at zero. */
#define QN_STATIC_SCRATCH_BYTES (16u << 20)
qn_status qlora_linear_fwd_noalloc(const qn_nf4dq* w, const uint16_t* x, int64_t M,
                                   const uint16_t* A, const uint16_t* B, int r, float alpha,
                                   uint16_t* y, float* u_out, void* stream);

/* Options of the adapter branch for the _ex calls (a NULL pointer means
 * alpha / r and no dropout).
 *   rslora: 0 -> s = alpha / r; 1 -> s = alpha / sqrt(r) (rsLoRA; course
 *     notebook FT-02, "Exercise 4: alpha/r vs alpha/sqrt(r) scaling").
 *   dropout_mask (nullable): dropout on the adapter branch's input (FT-02,
 *     the LoraConfig's lora_dropout): a keep mask over x [M, cols],
 *     bit-packed row-major (element e kept when bit e % 8 of byte e / 8 is
 *     set), device memory, 16-byte aligned (QN_EALIGN otherwise); the
 *     caller draws it.  Kept elements pass
 *     unchanged and the branch's scale becomes s / (1 - dropout_p); the
 *     backward takes the same mask (the dA product masks x where it loads
 *     it, the branch's share of dX is masked).  Forwards with dropout take the GEMM routes,
 *     never the decode kernels.
 *   dropout_p: in [0, 1) with a mask; 0 without one. */
typedef struct {
  int rslora;
  const uint8_t* dropout_mask;
  float dropout_p;
} qn_lora_opts;

/* Workspace bytes for a linear call on this state (its format decides the
 * route) with these options (nullable). */
size_t qlora_linear_workspace_state(const qn_nf4dq* w, int64_t M, int r, int backward,
                                    const qn_lora_opts* opts);

/* Workspace bytes for the _ex calls with these options (with dropout the
 * forward of a small batch takes a GEMM route instead of a decode kernel),
 * for an NF4 state with double quantization. */
size_t qlora_linear_workspace_ex(int64_t M, int64_t rows, int64_t cols, int r, int backward,
                                 const qn_lora_opts* opts);

/* qlora_linear_fwd with adapter options (opts nullable). */
qn_status qlora_linear_fwd_ex(const qn_nf4dq* w, const uint16_t* x, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float alpha, const qn_lora_opts* opts,
                              uint16_t* y, float* u_out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Backward: from G = dY [M, rows] bf16 computes
 *   dX [M, cols] bf16 = G Qhat(W) + s (G B) A      (skipped if dX == NULL)
 *   dA [r, cols] fp32 = s (G B)^T X                 (overwritten)
 *   dB [rows, r] fp32 = s G^T u,  u = X A^T          (overwritten)
 * with s = alpha / r.  u_saved (nullable) is the forward's u_out; when NULL
 * u is recomputed from x.  Same shape rules as the forward; M == 0 writes
 * zero dA and dB. */
qn_status qlora_linear_bwd(const qn_nf4dq* w, const uint16_t* x, const uint16_t* dY, int64_t M,
                           const uint16_t* A, const uint16_t* B, int r, float alpha,
                           const float* u_saved, uint16_t* dX, float* dA, float* dB,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Adapter merged into the dequantized weight (page "QLoRA: NF4 storage,
 * gradients and local integration", section "Merge changes the operator:
 * test it explicitly"):
 *   out [rows, cols] fp32 = Qhat(W) + (alpha/r) B A
 * with A [r, cols] and B [rows, r] bf16, 1 <= r <= 64.  Rounding: per
 * element, d = sum_j B[n][j] A[j][k] in fp64 in rank order, then
 * out = RN32(RN64(w' + RN64(s d))), w' the fp32 dequantized weight and
 * s = alpha / r in fp32.  This is the operator the separate adapter path
 * computes, up to the final fp32 rounding; requantizing it (nf4_quantize_dq
 * on out) is a different operator again.  Stream-ordered, no workspace. */
qn_status nf4_merge_lora(const qn_nf4dq* w, const uint16_t* A, const uint16_t* B, int r,
                         float alpha, float* out, void* stream);

/* Hyperparameters of one AdamW step (fp32 values; step >= 1). */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;
} qn_adamw_hparams;

/* One AdamW step with 8-bit moment states, for the adapters (course notebook
 * FT-02, the training arguments' optim="paged_adamw_8bit").  State format (a
 * reading: the pages name the optimizer but not its format): each moment in
 * blocks of 256 elements, OCP E4M3FN codes m_codes/v_codes [n] of x / s_b
 * with fp32 block scales m_scales/v_scales [ceil(n/256)], s_b = max|x| / 448
 * (all zero to start).  Update in fp32, one rounding per operation:
 *   m = b1 m + (1-b1) g,  v = b2 v + ((1-b2) g) g,  p = p (1 - lr wd),
 *   p = p - lr ((m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps))
 * (1-b, 1 - b^t and 1 - lr wd formed in fp64 from the fp32 values and
 * rounded once), then both moments are stored again with new block scales.
 * p [n] fp32 is updated in place from g [n] fp32 (for instance dA or dB);
 * p_bf16 (nullable) receives bf16(p) for the next forward.  Device pointers
 * 16-byte aligned; stream-ordered. */
qn_status adamw8_step(float* p, const float* g, int64_t n, uint8_t* m_codes, float* m_scales,
                      uint8_t* v_codes, float* v_scales, uint16_t* p_bf16,
                      const qn_adamw_hparams* h, void* stream);

/* Kernel routes of the linear calls (qlora_linear_route). */
enum {
  QN_ROUTE_DECODE_ROWS = 1,  /* M <= 16: one kernel over bands of whole rows */
  QN_ROUTE_DECODE_TILES = 2, /* M <= 16: one kernel over column slices of row bands */
  QN_ROUTE_DECODE_SPLIT = 3, /* M <= 16, r > 16: partial sums, then a finishing kernel */
  QN_ROUTE_FUSED_SMALL = 4,  /* M <= 32: dequantization inside 32-row GEMM tiles */
  QN_ROUTE_FUSED = 5,        /* dequantization inside 128 x 128 GEMM tiles */
  QN_ROUTE_DENSE = 6         /* bf16 copy of Qhat(W) in the workspace + dense GEMM */
};

/* Which route qlora_linear_fwd (backward == 0) or the dX product of
 * qlora_linear_bwd (backward != 0) takes for these sizes on the current
 * device (the same for every state format); -1 for sizes the calls reject.
 * For tests and profiling: every route computes the same function. */
int qlora_linear_route(int64_t M, int64_t rows, int64_t cols, int r, int backward);

/* qlora_linear_bwd with adapter options (opts nullable; the same options as
 * the forward whose u_saved is passed). */
qn_status qlora_linear_bwd_ex(const qn_nf4dq* w, const uint16_t* x, const uint16_t* dY,
                              int64_t M, const uint16_t* A, const uint16_t* B, int r, float alpha,
                              const qn_lora_opts* opts, const float* u_saved, uint16_t* dX,
                              float* dA, float* dB, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Dense LoRA linear on an already dequantized weight -- the forward's product
 * once Qhat(W) is held in bf16 (page 2, paragraph after the listing):
 *   y [M, rows] bf16 = X W^T + (alpha/r) V L^T
 * with X bf16 [M, cols], W bf16 [rows, cols] (e.g. from nf4_dequantize),
 * V fp32 [M, r] (u = X A^T, as qlora_linear_fwd returns it) and L bf16
 * [rows, r] (the adapter B).  Large-batch forwards run exactly this product
 * after dequantizing into their workspace.  Shape rules as qlora_linear_fwd;
 * no workspace; M == 0: no work. */
qn_status lora_linear_bf16(const uint16_t* x, int64_t M, const uint16_t* W, int64_t rows,
                           int64_t cols, const float* V, const uint16_t* L, int r, float alpha,
                           uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
