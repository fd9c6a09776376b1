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
 *     streams that share a workspace race.
 *   - Decode-sized forwards (1 <= M <= 16, r <= 16, cols % 1024 == 0) run as
 *     one kernel whose column slices meet through arrival counters in the
 *     library's static device memory: 64 slots per device, one per call,
 *     taken round robin and left at zero when the call ends.  More than 64
 *     such calls executing at the same time on one device would race.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QN_ABI_VERSION 2

typedef enum {
  QN_OK = 0,
  QN_EINVAL = 1,
  QN_ENONFINITE = 2,
  QN_EALIGN = 3,
  QN_EWORKSPACE = 4,
  QN_EDEVICE = 5
} qn_status;

typedef enum { QN_F32 = 0, QN_BF16 = 1 } qn_dtype;

/* A quantized weight in format v1 (device pointers, host struct). */
typedef struct {
  const uint8_t* packed; /* [32*nb] */
  const uint8_t* qscale; /* [nb]    */
  const float* scale2;   /* [ng]    */
  const float* offset;   /* [1]     */
  int64_t rows;          /* d_out   */
  int64_t cols;          /* d_in    */
} qn_nf4dq;

/* ABI version of the loaded library (QN_ABI_VERSION). */
int qn_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* qn_status_str(qn_status s);

/* The 16 NF4 levels the library uses, as fp32, into host memory. */
void qn_nf4_codebook(float out[16]);

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

/* Dequantize w into out [rows, cols]: fp32 (QN_F32) or bf16 bit patterns
 * (QN_BF16, round to nearest even of the fp32 value). */
qn_status nf4_dequantize(const qn_nf4dq* w, qn_dtype out_dtype, void* out, void* stream);

/* Workspace bytes needed by qlora_linear_fwd (backward == 0) or
 * qlora_linear_bwd (backward != 0) for M rows of activations. */
size_t qlora_linear_workspace(int64_t M, int64_t rows, int64_t cols, int r, int backward);

/* Forward: y [M, rows] bf16 = X Qhat(W)^T + (alpha/r) (X A^T) B^T.
 * cols must be a multiple of 64 and rows a multiple of 8 (so that every row
 * of X, G and W starts 16-byte aligned); 1 <= r <= 64; M >= 0 (M == 0: no
 * work).
 * u_out (nullable) receives u = X A^T, fp32 [M, r], for the backward. */
qn_status qlora_linear_fwd(const qn_nf4dq* w, const uint16_t* x, int64_t M, const uint16_t* A,
                           const uint16_t* B, int r, float alpha, uint16_t* y, float* u_out,
                           void* workspace, size_t workspace_bytes, void* stream);

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
