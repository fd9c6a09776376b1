// Host-side launchers of the HIP kernels (one translation unit each).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qn_device.h"

namespace qn {

// Arrival counters: the first kArrivalWords 32-bit words of every linear
// workspace.  They are zero before a call that counts on them (zeroed once
// when the workspace is allocated, or by an earlier kernel of the same call)
// and every workgroup that finishes a reduction puts its counter back to
// zero, so the words are zero again when the call ends.
constexpr int kArrivalWords = 1024;

// n words at p to clear (by the first workgroup of a launch); n == 0: none.
struct Clear {
  unsigned* p;
  int n;
};

// ws_bad [ng] per-group non-finite flags; *flag = 1 when any weight is NaN
// or infinite, else 0 (written by the last kernel; no clearing needed).
// codebook: kCodeNF4 or kCodeFP4.  absmax_out (nullable): double
// quantization off, the fp32 block scales are written there (qscale,
// scale2, offset unused; ws_offset receives a mean nobody reads).
hipError_t launch_quantize(const float* W, int64_t n, uint8_t* packed, uint8_t* qscale,
                           float* scale2, float* offset, float* ws_absmax, double* ws_part,
                           int64_t part_len, int* ws_bad, int* flag, hipStream_t st,
                           int codebook = kCodeNF4, float* absmax_out = nullptr,
                           float* ws_offset = nullptr);

// out = sum over S slices of part[S][count] (slice order); count == 0: none.
struct SliceSum {
  const float* part;
  int64_t count;
  int S;
  float* out;
};

// n weights -> bf16 or fp32 out; the slice sum ss (independent of the
// weight) runs in spare workgroups of the same launch.
// codebook and absmax (nullable: double quantized scales) as the state has
// them.
hipError_t launch_dequant(const uint8_t* packed, const uint8_t* qscale, const float* scale2,
                          const float* offset, int64_t n, bool bf16, void* out, hipStream_t st,
                          const SliceSum& ss = SliceSum{nullptr, 0, 0, nullptr},
                          int codebook = kCodeNF4, const float* absmax = nullptr,
                          bool nt = false);

// Small backward jobs, run by spare workgroups of another launch or alone:
//   Bt [r, N] = B[N, r]^T and At [K, r] = A[r, K]^T (bf16);
//   su = (s u)^T and sv = (s v)^T, each [2][16 ceil(r/16)][Mp] bf16 (high
//   parts, then remainders; zero for j >= r or m >= M), u and v fp32 [M, r];
//   when Sv > 1, v is first written as the slice sum of vpart [Sv][M][r].
// A null destination skips its job.  One thread per output element.
struct BwdAux {
  const uint16_t* B;
  uint16_t* Bt;
  int64_t N;
  const uint16_t* A;
  uint16_t* At;
  int64_t K;
  const float* u;
  uint16_t* su;
  int64_t Mpu;
  const float* vpart;
  int Sv;
  float* v;
  uint16_t* sv;
  int64_t Mpv;
  int64_t M;
  int r;
  float s;
};
// The jobs are rows, one per thread: a row n of B (Bt[j][n] = B[n][j]), a
// column k of A (At[k][j] = A[j][k]), a column m of su and of sv (all rp
// ranks of it).  A thread reads its row of B, u or v's slices whole (16-byte
// loads when r allows), the threads of a wave read neighbouring elements of
// A's rows, and the transposed writes of neighbouring threads are neighbours.
__host__ __device__ inline int64_t bwd_aux_count(const BwdAux& a) {
  return (a.Bt ? a.N : 0) + (a.At ? a.K : 0) + (a.su ? a.Mpu : 0) + (a.sv ? a.Mpv : 0);
}
// x as bf16 at dst[idx] and its remainder as bf16 at dst[half + idx]
__device__ inline void put_split(uint16_t* dst, int64_t half, int64_t idx, float x) {
  const uint32_t h = pack_bf16x2(x, 0.f) & 0xffffu;
  dst[idx] = (uint16_t)h;
  dst[half + idx] = (uint16_t)(pack_bf16x2(x - bf16_lo(h), 0.f) & 0xffffu);
}
// row job i of the concatenated jobs (Bt, At, su, sv in that order)
__device__ inline void bwd_aux_at(const BwdAux& a, int64_t i) {
  const int r = a.r;
  const int64_t rp = 16 * ((r + 15) / 16);
  const int64_t nb = a.Bt ? a.N : 0;
  if (i < nb) {  // Bt[j][n] = B[n][j]
    const int64_t n = i;
    const uint16_t* row = a.B + n * r;
    if ((r & 7) == 0) {
      for (int j0 = 0; j0 < r; j0 += 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + j0);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          a.Bt[(int64_t)(j0 + q) * a.N + n] = (uint16_t)(v[q >> 1] >> (16 * (q & 1)));
      }
    } else {
      for (int j = 0; j < r; ++j) a.Bt[(int64_t)j * a.N + n] = row[j];
    }
    return;
  }
  i -= nb;
  const int64_t na = a.At ? a.K : 0;
  if (i < na) {  // At[k][j] = A[j][k]
    const int64_t k = i;
    uint16_t* row = a.At + k * r;
    if ((r & 7) == 0) {
      for (int j0 = 0; j0 < r; j0 += 8) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)a.A[(int64_t)(j0 + 2 * q) * a.K + k] |
                 ((uint32_t)a.A[(int64_t)(j0 + 2 * q + 1) * a.K + k] << 16);
        *reinterpret_cast<u32x4*>(row + j0) = u32x4{w[0], w[1], w[2], w[3]};
      }
    } else {
      for (int j = 0; j < r; ++j) row[j] = a.A[(int64_t)j * a.K + k];
    }
    return;
  }
  i -= na;
  // su: (s u)^T split, column m; sv: v = sum of the slices (written), then
  // (s v)^T split; ranks j >= r and columns m >= M are zero
  const int64_t nu = a.su ? a.Mpu : 0;
  const bool is_u = i < nu;
  const int64_t m = is_u ? i : i - nu;
  const int64_t Mp = is_u ? a.Mpu : a.Mpv;
  uint16_t* dst = is_u ? a.su : a.sv;
  const int64_t half = rp * Mp;
  const bool in = m < a.M;
  const bool vec = (r & 3) == 0;
  for (int j0 = 0; j0 < rp; j0 += 4) {
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (in && j0 < r) {
      const int64_t e = m * r + j0;
      if (is_u) {
        if (vec) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(a.u + e);
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = v[q];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = j0 + q < r ? a.u[e + q] : 0.f;
        }
      } else if (a.Sv > 1) {
        // slices added in slice order
        const int64_t cnt = a.M * (int64_t)r;
        if (vec) {
          // eight slices' loads in flight at a time (clamped), added in order
          f32x4 acc = *reinterpret_cast<const f32x4*>(a.vpart + e);
          for (int s0 = 1; s0 < a.Sv; s0 += 8) {
            f32x4 w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
              w[k] = *reinterpret_cast<const f32x4*>(
                  a.vpart + (int64_t)min(s0 + k, a.Sv - 1) * cnt + e);
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (s0 + k < a.Sv) acc += w[k];
          }
          *reinterpret_cast<f32x4*>(a.v + e) = acc;
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = acc[q];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (j0 + q < r) {
              x[q] = slice_sum(a.vpart, cnt, a.Sv, e + q);
              a.v[e + q] = x[q];
            }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = j0 + q < r ? a.v[e + q] : 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) put_split(dst, half, (int64_t)(j0 + q) * Mp + m, a.s * x[q]);
  }
}
hipError_t launch_bwd_aux(const BwdAux& a, hipStream_t st);

// out[k][n] = Qhat(W)[n][k] as bf16 with row length ldt (ldt % 8 == 0,
// ldt >= rows); zero for rows <= n < ldt.  cols % 64 == 0.  The jobs of
// aux run in extra workgroups of the same launch.
hipError_t launch_dequant_t(const uint8_t* packed, const uint8_t* qscale, const float* scale2,
                            const float* offset, int64_t rows, int64_t cols, uint16_t* out,
                            int64_t ldt, const BwdAux& aux, hipStream_t st,
                            int codebook = kCodeNF4, const float* absmax = nullptr);

// C[M, Nc] bf16 = A[M, R] (row stride lda) * Bm[Nc, :R]^T (row stride ldb,
// ldb % 64 == 0, zero in columns R..ldb) + s * V[M, r] * L[Nc, r]^T.
// lda >= R, R % 8 == 0, Nc % 8 == 0; 16-byte aligned pointers.
hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, int64_t R, const uint16_t* Bm,
                          int64_t ldb, int64_t M, int64_t Nc, const float* V, const uint16_t* L,
                          int r, float s, uint16_t* C, hipStream_t st);

// Weight state as the kernels take it.
struct WState;
// Decode-sized forward (M <= 16, cols % 1024 == 0): number of K slices, or
// 0 when the decode kernels do not apply.
int decode_slices(int64_t M, int64_t rows, int64_t cols);

struct WState {
  const uint8_t* packed;
  const uint8_t* qscale;
  const float* scale2;
  const float* offset;
  int64_t rows, cols;
  const float* absmax = nullptr;  // fp32 block scales (double quantization off), or null
  int codebook = kCodeNF4;        // kCodeNF4 or kCodeFP4
};

// out[M, r] (fp32) = sum over S slices of Z[M, P] * T[r, P]^T.  When S > 1
// the slices are written to part[S][M][r] and summed in slice order into
// out; S == 1 writes out directly.
// sum == false leaves the slices in part for the caller to add.  t_rows:
// T is given as its transpose [P, r] (r <= 16 only).  clr: words the first
// workgroup zeroes.  zmask (nullable): Z's elements whose bit is clear read
// as zero (bit-packed over the row-major elements, bit e % 8 of byte e / 8;
// P % 8 == 0).
hipError_t launch_thin_nt(const uint16_t* Z, const uint16_t* T, int64_t M, int64_t P, int r,
                          float* out, float* part, int S, hipStream_t st, bool sum = true,
                          bool t_rows = false, Clear clr = Clear{nullptr, 0},
                          const uint8_t* zmask = nullptr);

// fp32 scalars of one 8-bit AdamW step (the 1 - b, bias corrections and
// decay formed on the host).
struct AdamScalars {
  float lr, b1, b2, omb1, omb2, eps, c1, c2, decay;
};
// One 8-bit AdamW step over n parameters (p, g fp32; moments as E4M3 codes
// with fp32 scales per 256; pb nullable: bf16 copy of the new p).  p, g
// 16-byte aligned, mq, vq 4-byte aligned.
hipError_t launch_adamw8(float* p, const float* g, int64_t n, uint8_t* mq, float* ms, uint8_t* vq,
                         float* vs, uint16_t* pb, const AdamScalars& h, hipStream_t st);

// dX[m][k] (bf16) += s (v A)[m][k] where mask bit (m, k) is set: the
// adapter branch's input gradient under dropout.  v fp32 [M, r], A bf16
// [r, K], K % 8 == 0, 1 <= r <= 64.
hipError_t launch_lora_masked_add(uint16_t* dX, const float* v, const uint16_t* A,
                                  const uint8_t* mask, int64_t M, int64_t K, int r, float s,
                                  hipStream_t st);
int thin_nt_slices(int64_t M, int64_t P);
bool thin_nt_rows_ok(int64_t M, int64_t P, int r);

// p[0..n) = 0 (a kernel, so it may sit in a captured graph).
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);


// One transposed adapter product out = Z^T (s V), reduced over the M rows:
// Z bf16 [M, P] (null: no product), vt = (s V)^T split as BwdAux makes it
// with Mp = thin_tn_rows_padded(M, P, r); transposed == false: out fp32
// [P, r]; true: out fp32 [r, P].  Split over thin_tn_slices(M, P, r) row
// slices with partials part[S][P][r], summed in slice order.  P % 8 == 0.
struct ThinTn {
  const uint16_t* Z;
  const uint16_t* vt;
  int64_t P;
  float* out;
  bool transposed;
  float* part;
  const uint8_t* zmask = nullptr;  // keep bits of Z [M, P] (dropout), or null
};
// Two such products (same M and r) in one launch; the slices are added by
// the last workgroup of each column tile to finish (arrivals: kArrivalWords
// counters, zero at the launch and left at zero), or, past kArrivalWords
// column tiles or with arrivals == null, by a second launch.
hipError_t launch_thin_tn2(const ThinTn& a, const ThinTn& b, int64_t M, int r,
                           unsigned* arrivals, hipStream_t st);
int thin_tn_slices(int64_t M, int64_t P, int r);
int64_t thin_tn_rows_padded(int64_t M, int64_t P, int r);

// Decode forward, u = X A^T included (written to u_out [M, r]); workspace
// part [S, M, rows] and upart [S, M, r] fp32, S = decode_slices(...).
hipError_t launch_decode_fwd(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                             const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                             float* part, float* upart, int S, hipStream_t st);

// One-kernel decode forward (M <= 16, r <= 16, cols % 1024 == 0): tiles of
// 16 rgt rows x 1024 columns; S = cols / 1024 slices, `bands` row bands.
// rgt == 0 when it does not apply.  Workspace: part [S, M, rows rounded up
// to 4] and upart [bands, S, 256] fp32, 16-byte aligned; arrivals: one
// counter per band (bands <= kArrivalWords), zero at the launch and left at
// zero.  Writes Y and u_out.
struct DecodeTiles {
  int rgt, S, bands;
};
DecodeTiles decode_tiles(int64_t M, int64_t rows, int64_t cols, int r);
hipError_t launch_decode_tile(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                              const DecodeTiles& t, unsigned* arrivals, float* part,
                              float* upart, hipStream_t st);

// Whole-row decode forward (M <= 16, r <= 16, cols 2048 or 4096): bands of
// `br` rows (a multiple of 8, at most 64), one workgroup each, every column;
// writes Y and u_out, no workspace.  decode_rows_band gives br, or 0 when the
// kernel does not apply (also when bands would be 32 rows or fewer).
int decode_rows_band(int64_t M, int64_t rows, int64_t cols, int r);
hipError_t launch_decode_rows(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                              int br, hipStream_t st);

// out [rows, cols] fp32 = Qhat(W) + s B A (fp64 rank sum in rank order, one
// fp32 rounding at the end); A [r, cols], B [rows, r] bf16, 1 <= r <= 64.
hipError_t launch_merge(const WState& w, const uint16_t* A, const uint16_t* B, int r, float s,
                        float* out, hipStream_t st, int codebook = kCodeNF4,
                        const float* absmax = nullptr);

// Y[M, N] bf16 = X[M, K] * W'[N, K]^T + s * u[M, r] * B[N, r]^T.
hipError_t launch_qgemm_fwd(const WState& w, const uint16_t* X, int64_t M, const float* u,
                            const uint16_t* B, int r, float s, uint16_t* Y, hipStream_t st);

// dX[M, K] bf16 = G[M, N] * W'[N, K] + s * v[M, r] * A[r, K].
hipError_t launch_qgemm_dx(const WState& w, const uint16_t* G, int64_t M, const float* v,
                           const uint16_t* A, int r, float s, uint16_t* dX, hipStream_t st);

}  // namespace qn
