/*
 * Plain CPU oracle for the QLoRA NF4 hot path.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (the HIP library) never links,
 * imports or calls it, and the two share no source, header, table or
 * constant: the codebook below is typed from the decimal literals printed on
 * the page "QLoRA: NF4 storage, gradients and local integration"
 * (section "Exact CPU teaching quantizer and adapter gradient path"), while
 * the GPU side keeps its own table as raw fp32 bit patterns.
 *
 * Every step is written in the plainest order the pages state it:
 *   - blocks of 64 consecutive elements of the flattened weight, the tail
 *     padded with zeros (teaching quantizer listing; course notebook
 *     "Exercise 1", the 64-value block reshape);
 *   - block scale = max |w| (same listing);
 *   - normalise by the scale (a zero block divides by 1), then take the
 *     nearest codebook level, the first one on ties (np.argmin semantics);
 *   - pack two 4-bit codes per byte, low nibble first (same listing);
 *   - double quantisation of the fp32 block scales: subtract one mean
 *     offset, take the absmax C2 of every 256 consecutive scales, divide by
 *     C2/448 and store OCP FP8 E4M3FN codes ("QLoRA Deep Dive", section
 *     "2. Squeezing More Memory: Double Quantization (DQ)"; 8-bit scales with
 *     one 32-bit constant per 256 scales on the page 2 section "Double
 *     quantization: correct the scale arithmetic").
 *   - dequantize: level * block scale (teaching listing, dequantize_nf4).
 *   - the QLoRA linear and its gradients as plain fp64 loops:
 *       Y  = X Qhat(W)^T + s (X A^T) B^T
 *       dX = G Qhat(W) + s (G B) A
 *       dB = s G^T (X A^T),   dA = s (G B)^T X
 *     (page 2 paragraph after the listing: the formulas for dB, dA, dX).
 *
 * Floating point: built with -O2 -fno-fast-math -ffp-contract=off on x86-64
 * (SSE, FLT_EVAL_METHOD 0), so every float expression rounds once to fp32
 * and nothing is fused unless fmaf() is written.  No SIMD intrinsics, no
 * BLAS.  OpenMP only splits independent blocks / output rows; every sum runs
 * in one fixed sequential order.
 *
 * Readings where the pages are silent (listed with reasons in the design
 * notes of this repository):
 *   R1  8-bit scale code = OCP FP8 E4M3FN, round-to-nearest-even, values
 *       beyond the largest finite 448 saturate to +-448.
 *   R2  one fp32 mean offset per weight tensor.
 *   R3  the mean is a fixed fp64 stride-halving tree: per group of 256 slots,
 *       then over the group partials zero-padded to a power of two.
 *   R5  normalisation is fp32 IEEE division (the page uses fp64).
 *   R12 the dequant scale is fmaf(code_value, s2, mu): one rounding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENONFINITE 2

/* Page 2, "Exact CPU teaching quantizer ...": the NF4 table as printed. */
static const double NF4_PAGE_LITERALS[16] = {
    -1.0, -0.6961928009986877, -0.5250730514526367, -0.39491748809814453,
    -0.28444138169288635, -0.18477343022823334, -0.09105003625154495, 0.0,
    0.07958029955625534, 0.16093020141124725, 0.24611230194568634,
    0.33791524171829224, 0.44070982933044434, 0.5626170039176941,
    0.7229568362236023, 1.0};

static float level(int k) { return (float)NF4_PAGE_LITERALS[k]; }

/* FP4 (course notebook FT-02, "Exercise 3: NF4 vs FP4 at equal memory"): an
 * E2M1 float format whose normalized positive levels, as the notebook
 * prints them from bitsandbytes, are 0, 0.0052, 0.1667, 0.25, 0.3333, 0.5,
 * 0.6667, 1.  Reading: the exact levels are {0, 0.0625, 2, 3, 4, 6, 8, 12}
 * / 12 (each rounds to the printed value at four decimals), stored as fp32;
 * a code is sign (bit 3) and magnitude index (bits 0..2), code c meaning
 * (c & 8 ? -1 : +1) * FP4_MAG[c & 7]. */
static const double FP4_MAG[8] = {0.0,       0.0625 / 12, 2.0 / 12, 3.0 / 12,
                                  4.0 / 12, 6.0 / 12,    8.0 / 12, 1.0};

static float fp4_level(int c) {
  float m = (float)FP4_MAG[c & 7];
  return (c & 8) ? -m : m;
}

void orc_fp4_codebook(float out[16]) {
  for (int c = 0; c < 16; ++c) out[c] = fp4_level(c);
}

/* FP4 code of a normalised value n: the sign of n, and the nearest
 * magnitude of |n| (exact fp64 midpoints of adjacent fp32 magnitudes; a
 * value exactly on a midpoint takes the lower magnitude). */
int orc_fp4_code(float n) {
  float a = fabsf(n);
  int m = 0;
  for (int k = 0; k < 7; ++k) {
    double mid = ((double)(float)FP4_MAG[k] + (double)(float)FP4_MAG[k + 1]) / 2.0;
    if ((double)a > mid) m = k + 1;
  }
  return (signbit(n) ? 8 : 0) | m;
}

void orc_codebook(float out[16]) {
  for (int k = 0; k < 16; ++k) out[k] = level(k);
}

/* Nearest level of a normalised value: scan k upward, keep the first
 * minimum of RN32(|n - L_k|).  Equivalent to np.argmin on the distances. */
int orc_nf4_code(float n) {
  int best = 0;
  float bestd = fabsf(n - level(0));
  for (int k = 1; k < 16; ++k) {
    float d = fabsf(n - level(k));
    if (d < bestd) {
      bestd = d;
      best = k;
    }
  }
  return best;
}

void orc_nf4_codes(const float* n, int64_t count, uint8_t* codes) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) codes[i] = (uint8_t)orc_nf4_code(n[i]);
}

/* ---------------- OCP FP8 E4M3FN (bias 7, 3 mantissa bits, no inf) ------- */

/* Value of a non-negative finite magnitude code 0..126, from the format's
 * definition: exponent field e, mantissa m; e == 0 is subnormal m * 2^-9,
 * otherwise (1 + m/8) * 2^(e-7).  Code 127 is NaN. */
static double e4m3_magnitude(int code7) {
  int e = code7 >> 3, m = code7 & 7;
  if (e == 0) return ldexp((double)m, -9);
  return ldexp((double)(8 + m), e - 10);
}

float orc_e4m3_decode(uint8_t q) {
  int mag = q & 0x7f;
  double v = (mag == 0x7f) ? NAN : e4m3_magnitude(mag);
  return (float)((q & 0x80) ? -v : v);
}

/* Round a finite fp32 to the nearest E4M3FN value, ties to the even code
 * (even mantissa), magnitudes beyond 448 saturate to 448.  Brute force over
 * the 127 finite magnitudes. */
uint8_t orc_e4m3_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  int mag;
  if (a >= 448.0) {
    mag = 126;
  } else {
    int k = 0;
    while (k < 126 && e4m3_magnitude(k + 1) <= a) ++k; /* value(k) <= a */
    if (e4m3_magnitude(k) == a) {
      mag = k;
    } else {
      double lo = a - e4m3_magnitude(k), hi = e4m3_magnitude(k + 1) - a;
      if (lo < hi)
        mag = k;
      else if (hi < lo)
        mag = k + 1;
      else
        mag = (k & 1) ? k + 1 : k;
    }
  }
  return (uint8_t)(sign | mag);
}

/* ---------------- bf16 round-to-nearest-even ------------------------------ */

static float f32_from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t bits_from_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* The two bf16 neighbours of v (toward and away from zero) and a choice of
 * the nearer, ties to the even one. */
uint16_t orc_bf16_rne(float v) {
  uint32_t u = bits_from_f32(v);
  uint32_t lo = u & 0xffff0000u;
  if (lo == u) return (uint16_t)(u >> 16);
  uint32_t hi = lo + 0x10000u;
  double dv = v, dlo = f32_from_bits(lo), dhi = f32_from_bits(hi);
  double elo = fabs(dv - dlo), ehi = fabs(dhi - dv);
  uint32_t r;
  if (elo < ehi)
    r = lo;
  else if (ehi < elo)
    r = hi;
  else
    r = ((lo >> 16) & 1u) ? hi : lo;
  return (uint16_t)(r >> 16);
}

float orc_bf16_value(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* ---------------- fixed-order fp64 tree ----------------------------------- */

/* len is a power of two; v is overwritten. */
static double stride_halving_sum(double* v, int64_t len) {
  for (int64_t h = len / 2; h >= 1; h /= 2)
    for (int64_t j = 0; j < h; ++j) v[j] += v[j + h];
  return v[0];
}

/* Mean of the first-level scales, reading R3. */
float orc_scale_mean(const float* absmax, int64_t nb) {
  int64_t ng = (nb + 255) / 256;
  int64_t len = 1;
  while (len < ng) len *= 2;
  double* part = (double*)calloc((size_t)len, sizeof(double));
  for (int64_t g = 0; g < ng; ++g) {
    double v[256];
    for (int j = 0; j < 256; ++j) {
      int64_t b = g * 256 + j;
      v[j] = (b < nb) ? (double)absmax[b] : 0.0;
    }
    part[g] = stride_halving_sum(v, 256);
  }
  double total = stride_halving_sum(part, len);
  free(part);
  return (float)(total / (double)nb);
}

/* Double quantisation of nb first-level scales (reading R1, R2, R3). */
static void double_quantize(const float* absmax, int64_t nb, uint8_t* qscale,
                            float* scale2, float* offset) {
  float mu = orc_scale_mean(absmax, nb);
  *offset = mu;
  int64_t ng = (nb + 255) / 256;
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < ng; ++g) {
    int64_t b0 = g * 256, b1 = b0 + 256 < nb ? b0 + 256 : nb;
    float c2 = 0.0f;
    for (int64_t b = b0; b < b1; ++b) {
      float d = absmax[b] - mu;
      if (fabsf(d) > c2) c2 = fabsf(d);
    }
    float s2 = c2 / 448.0f;
    scale2[g] = s2;
    for (int64_t b = b0; b < b1; ++b) {
      float d = absmax[b] - mu;
      float x = (s2 > 0.0f) ? d / s2 : 0.0f;
      qscale[b] = orc_e4m3_encode(x);
    }
  }
}

/* Blockwise 4-bit quantisation with the NF4 (codebook 0) or FP4 (codebook
 * 1) codes; the same blocks, scales, packing and double quantisation as
 * orc_quantize below, which is codebook 0. */
int orc_quantize_cb(const float* w, int64_t n, int codebook, int double_quant,
                    uint8_t* packed, float* absmax, uint8_t* qscale, float* scale2,
                    float* offset);

/* Blockwise NF4 quantisation of n fp32 values.
 *   packed [32*nb]  two codes per byte, element 2j low nibble
 *   absmax [nb]     fp32 first-level scales (kept: the DQ-off state)
 *   qscale/scale2/offset: the DQ state, written when double_quant != 0
 * Returns ORC_EINVAL for n < 1 and ORC_ENONFINITE before writing anything
 * when some input is NaN or infinite. */
int orc_quantize(const float* w, int64_t n, int double_quant, uint8_t* packed,
                 float* absmax, uint8_t* qscale, float* scale2,
                 float* offset) {
  return orc_quantize_cb(w, n, 0, double_quant, packed, absmax, qscale, scale2, offset);
}

int orc_quantize_cb(const float* w, int64_t n, int codebook, int double_quant,
                    uint8_t* packed, float* absmax, uint8_t* qscale, float* scale2,
                    float* offset) {
  if (n < 1 || codebook < 0 || codebook > 1) return ORC_EINVAL;
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(w[i])) return ORC_ENONFINITE;
  int64_t nb = (n + 63) / 64;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    float blk[64];
    for (int i = 0; i < 64; ++i) {
      int64_t idx = b * 64 + i;
      blk[i] = (idx < n) ? w[idx] : 0.0f;
    }
    float s = 0.0f;
    for (int i = 0; i < 64; ++i)
      if (fabsf(blk[i]) > s) s = fabsf(blk[i]);
    absmax[b] = s;
    uint8_t code[64];
    for (int i = 0; i < 64; ++i) {
      float nv = (s > 0.0f) ? blk[i] / s : blk[i] / 1.0f;
      code[i] = (uint8_t)(codebook ? orc_fp4_code(nv) : orc_nf4_code(nv));
    }
    for (int j = 0; j < 32; ++j)
      packed[b * 32 + j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
  }
  if (double_quant) double_quantize(absmax, nb, qscale, scale2, offset);
  return ORC_OK;
}

/* Per-block dequant scale s'_b. */
static float block_scale(int64_t b, int double_quant, const float* absmax,
                         const uint8_t* qscale, const float* scale2,
                         const float* offset) {
  if (!double_quant) return absmax[b];
  return fmaf(orc_e4m3_decode(qscale[b]), scale2[b / 256], *offset);
}

/* w'_i = RN32(L[c_i] * s'_b); fp32 and/or bf16 (RNE of w') outputs, n
 * elements (padding is not written).  Either output may be NULL. */
void orc_dequantize_cb(const uint8_t* packed, int64_t n, int codebook, int double_quant,
                       const float* absmax, const uint8_t* qscale, const float* scale2,
                       const float* offset, float* out_f32, uint16_t* out_bf16);

void orc_dequantize(const uint8_t* packed, int64_t n, int double_quant,
                    const float* absmax, const uint8_t* qscale,
                    const float* scale2, const float* offset, float* out_f32,
                    uint16_t* out_bf16) {
  orc_dequantize_cb(packed, n, 0, double_quant, absmax, qscale, scale2, offset, out_f32,
                    out_bf16);
}

/* orc_dequantize with the codes of either codebook (0 NF4, 1 FP4). */
void orc_dequantize_cb(const uint8_t* packed, int64_t n, int codebook, int double_quant,
                       const float* absmax, const uint8_t* qscale, const float* scale2,
                       const float* offset, float* out_f32, uint16_t* out_bf16) {
  int64_t nb = (n + 63) / 64;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    float sp = block_scale(b, double_quant, absmax, qscale, scale2, offset);
    for (int i = 0; i < 64; ++i) {
      int64_t idx = b * 64 + i;
      if (idx >= n) break;
      uint8_t byte = packed[idx / 2];
      int c = (idx % 2 == 0) ? (byte & 15) : (byte >> 4);
      float v = (codebook ? fp4_level(c) : level(c)) * sp;
      if (out_f32) out_f32[idx] = v;
      if (out_bf16) out_bf16[idx] = orc_bf16_rne(v);
    }
  }
}

/* ---------------- QLoRA linear in fp64 ------------------------------------ */

static double bf(const uint16_t* p, int64_t i) {
  return (double)orc_bf16_value(p[i]);
}

/* u = X A^T for the listed rows of X.
 *   X [*, K] bf16, A [r, K] bf16, u [nrows, r] fp64; rows == NULL means
 *   rows 0..nrows-1. */
void orc_lora_down(const uint16_t* X, const uint16_t* A, int64_t K, int r,
                   const int64_t* rows, int64_t nrows, double* u) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t m = rows ? rows[i] : i;
    for (int j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += bf(X, m * K + k) * bf(A, (int64_t)j * K + k);
      u[i * r + j] = acc;
    }
  }
}

/* Forward for the listed rows: Y = X W'^T + s u B^T.
 *   Wd [N, K] fp32 dequantized weights, B [N, r] bf16, Y [nrows, N] fp64,
 *   u [nrows, r] fp64 (output, X A^T). */
void orc_qlora_fwd(const float* Wd, int64_t N, int64_t K, const uint16_t* X,
                   const uint16_t* A, const uint16_t* B, int r, double s,
                   const int64_t* rows, int64_t nrows, double* Y, double* u) {
  orc_lora_down(X, A, K, r, rows, nrows, u);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t m = rows ? rows[i] : i;
    for (int64_t n = 0; n < N; ++n) {
      double base = 0.0;
      for (int64_t k = 0; k < K; ++k) base += bf(X, m * K + k) * (double)Wd[n * K + k];
      double lora = 0.0;
      for (int j = 0; j < r; ++j) lora += u[i * r + j] * bf(B, n * r + j);
      Y[i * N + n] = base + s * lora;
    }
  }
}

/* v = G B for the listed rows: G [*, N] bf16, B [N, r] bf16, v [nrows, r]. */
void orc_lora_up_grad(const uint16_t* G, const uint16_t* B, int64_t N, int r,
                      const int64_t* rows, int64_t nrows, double* v) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t m = rows ? rows[i] : i;
    for (int j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) acc += bf(G, m * N + n) * bf(B, n * r + j);
      v[i * r + j] = acc;
    }
  }
}

/* Input gradient for the listed rows: dX = G W' + s v A.
 *   dX [nrows, K] fp64, v [nrows, r] fp64 (output, G B). */
void orc_qlora_dx(const float* Wd, int64_t N, int64_t K, const uint16_t* G,
                  const uint16_t* A, const uint16_t* B, int r, double s,
                  const int64_t* rows, int64_t nrows, double* dX, double* v) {
  orc_lora_up_grad(G, B, N, r, rows, nrows, v);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t m = rows ? rows[i] : i;
    for (int64_t k = 0; k < K; ++k) {
      double base = 0.0;
      for (int64_t n = 0; n < N; ++n) base += bf(G, m * N + n) * (double)Wd[n * K + k];
      double lora = 0.0;
      for (int j = 0; j < r; ++j) lora += v[i * r + j] * bf(A, (int64_t)j * K + k);
      dX[i * K + k] = base + s * lora;
    }
  }
}

/* Adapter gradients over all M rows:
 *   dB [N, r] = s G^T u,  dA [r, K] = s v^T X,
 * with u = X A^T and v = G B given in fp64 ([M, r] each). */
void orc_adapter_grads(const uint16_t* X, const uint16_t* G, const double* u,
                       const double* v, int64_t M, int64_t N, int64_t K, int r,
                       double s, double* dA, double* dB) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int64_t m = 0; m < M; ++m) acc += bf(G, m * N + n) * u[m * r + j];
      dB[n * r + j] = s * acc;
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; ++k) {
    for (int j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int64_t m = 0; m < M; ++m) acc += v[m * r + j] * bf(X, m * K + k);
      dA[(int64_t)j * K + k] = s * acc;
    }
  }
}

/* Threads the oracle's parallel loops use from now on (n >= 1). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---------------- dropout on the adapter branch ---------------------------- */

/* Course notebook FT-02, the LoraConfig of the QLoRA setup (lora_dropout
 * 0.05): dropout acts on the adapter branch's input only.  Reading: a kept
 * element passes unchanged, a dropped one is zero, and the 1/(1-p) of
 * inverted dropout is folded into the branch's scale s (the caller passes
 * s / (1 - p)).  mask is bit-packed row-major over [M, K]: element e is kept
 * when bit e % 8 of byte e / 8 is set.
 *   X [M, K] bf16 -> Xd [M, K] bf16 (the masked input). */
void orc_dropout_apply(const uint16_t* X, const uint8_t* mask, int64_t M, int64_t K,
                       uint16_t* Xd) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) {
      int64_t e = m * K + k;
      int kept = (mask[e / 8] >> (e % 8)) & 1;
      Xd[e] = kept ? X[e] : (uint16_t)0;
    }
}

/* Input gradient with dropout on the adapter branch, for the listed rows:
 * dX = G W' + s ((G B) A) (.) mask, the mask applied elementwise to the
 * branch's contribution (its input was masked in the forward).
 *   dX [nrows, K] fp64, v [nrows, r] fp64 (output, G B). */
void orc_qlora_dx_dropout(const float* Wd, int64_t N, int64_t K, const uint16_t* G,
                          const uint16_t* A, const uint16_t* B, int r, double s,
                          const uint8_t* mask, const int64_t* rows, int64_t nrows,
                          double* dX, double* v) {
  orc_lora_up_grad(G, B, N, r, rows, nrows, v);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t m = rows ? rows[i] : i;
    for (int64_t k = 0; k < K; ++k) {
      double base = 0.0;
      for (int64_t n = 0; n < N; ++n) base += bf(G, m * N + n) * (double)Wd[n * K + k];
      double lora = 0.0;
      for (int j = 0; j < r; ++j) lora += v[i * r + j] * bf(A, (int64_t)j * K + k);
      int64_t e = m * K + k;
      int kept = (mask[e / 8] >> (e % 8)) & 1;
      dX[i * K + k] = base + (kept ? s * lora : 0.0);
    }
  }
}

/* ---------------- 8-bit AdamW step for the adapters ------------------------ */

/* The adapters' optimizer (course notebook FT-02, the training arguments'
 * optim="paged_adamw_8bit": AdamW whose two moment states are stored in 8
 * bits).  The pages fix no 8-bit state format; reading: each state tensor
 * is stored blockwise, 256 elements per block, as OCP E4M3FN codes of
 * x / s_b with one fp32 block scale s_b = RN32(max|x| / 448) (s_b = 0: all
 * codes 0).  The update follows AdamW with decoupled weight decay, in fp32,
 * one rounding per operation in this order:
 *   m = RN(RN(b1 m_old) + RN(omb1 g)),  v = RN(RN(b2 v_old) + RN(RN(omb2 g) g))
 *   p = RN(p decay),  denom = RN(sqrt(RN(v / c2)) + eps)
 *   p = RN(p - RN(lr RN(RN(m / c1) / denom)))
 * with m_old = RN(e4m3(code) s_b) (likewise v_old), omb1 = 1 - b1 and
 * omb2 = 1 - b2, c1 = 1 - b1^t and c2 = 1 - b2^t (bias corrections of step
 * t >= 1) and decay = 1 - lr wd, all given as fp32; then both states are
 * quantized again with new block scales.
 *   p [n] fp32 (updated), g [n] fp32, mq/vq [n] codes, ms/vs [ceil(n/256)]
 *   fp32 block scales (updated); pb (nullable) receives bf16(p). */
static void state_requant(const float* x, int64_t b0, int64_t b1, uint8_t* q, float* sc,
                          int64_t blk) {
  float amax = 0.0f;
  for (int64_t i = b0; i < b1; ++i)
    if (fabsf(x[i - b0]) > amax) amax = fabsf(x[i - b0]);
  float s = amax / 448.0f;
  sc[blk] = s;
  for (int64_t i = b0; i < b1; ++i) q[i] = s > 0.0f ? orc_e4m3_encode(x[i - b0] / s) : 0;
}

void orc_adamw8_step(float* p, const float* g, int64_t n, uint8_t* mq, float* ms, uint8_t* vq,
                     float* vs, uint16_t* pb, float lr, float b1, float b2, float omb1,
                     float omb2, float eps, float c1, float c2, float decay) {
  int64_t nb = (n + 255) / 256;
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < nb; ++blk) {
    int64_t i0 = blk * 256, i1 = i0 + 256 < n ? i0 + 256 : n;
    float m[256], v[256];
    for (int64_t i = i0; i < i1; ++i) {
      float mo = orc_e4m3_decode(mq[i]) * ms[blk];
      float vo = orc_e4m3_decode(vq[i]) * vs[blk];
      float mi = b1 * mo + omb1 * g[i];
      float vi = b2 * vo + (omb2 * g[i]) * g[i];
      float pi = p[i] * decay;
      float denom = sqrtf(vi / c2) + eps;
      float upd = (mi / c1) / denom;
      pi = pi - lr * upd;
      p[i] = pi;
      if (pb) pb[i] = orc_bf16_rne(pi);
      m[i - i0] = mi;
      v[i - i0] = vi;
    }
    state_requant(m, i0, i1, mq, ms, blk);
    state_requant(v, i0, i1, vq, vs, blk);
  }
}

/* ---------------- merge of the adapter into the weight -------------------- */

/* Page 2, section "Merge changes the operator: test it explicitly": merging
 * the adapter into the dequantized weight gives the operator
 * Qhat(W) + s B A; requantizing it is a further, separate step (done by
 * orc_quantize on the result).  Reading for the rounding: per element
 * d = sum_j B[n][j] A[j][k] in fp64 with j ascending (each product of two
 * bf16 values is exact in fp64), then out = RN32(RN64(w' + RN64(s d))).
 *   Wd [rows, cols] fp32 dequantized weight, A [r, cols] and B [rows, r]
 *   bf16, s = alpha / r as fp32; out [rows, cols] fp32. */
void orc_merge(const float* Wd, int64_t rows, int64_t cols, const uint16_t* A,
               const uint16_t* B, int r, float s, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < rows; ++n) {
    for (int64_t k = 0; k < cols; ++k) {
      double d = 0.0;
      for (int j = 0; j < r; ++j) d += bf(B, n * r + j) * bf(A, (int64_t)j * cols + k);
      double t = (double)s * d;
      double m = (double)Wd[n * cols + k] + t;
      out[n * cols + k] = (float)m;
    }
  }
}

int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
