// Host-side launchers of the HIP kernels (one translation unit each).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qn_device.h"

namespace qn {

// ws_bad [ng] per-group non-finite flags; *flag = 1 when any weight is NaN
// or infinite, else 0 (written by the last kernel; no clearing needed).
hipError_t launch_quantize(const float* W, int64_t n, uint8_t* packed, uint8_t* qscale,
                           float* scale2, float* offset, float* ws_absmax, double* ws_part,
                           int64_t part_len, int* ws_bad, int* flag, hipStream_t st);

// out = sum over S slices of part[S][count] (slice order); count == 0: none.
struct SliceSum {
  const float* part;
  int64_t count;
  int S;
  float* out;
};

// n weights -> bf16 or fp32 out; the slice sum ss (independent of the
// weight) runs in spare workgroups of the same launch.
hipError_t launch_dequant(const uint8_t* packed, const uint8_t* qscale, const float* scale2,
                          const float* offset, int64_t n, bool bf16, void* out, hipStream_t st,
                          const SliceSum& ss = SliceSum{nullptr, 0, 0, nullptr});

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
__host__ __device__ inline int64_t bwd_aux_count(const BwdAux& a) {
  const int64_t rp = 16 * ((a.r + 15) / 16);
  return (a.Bt ? a.N * a.r : 0) + (a.At ? a.K * a.r : 0) + (a.su ? rp * a.Mpu : 0) +
         (a.sv ? rp * a.Mpv : 0);
}
// element i of the concatenated jobs (Bt, At, su, sv in that order)
__device__ inline void bwd_aux_at(const BwdAux& a, int64_t i) {
  const int64_t rp = 16 * ((a.r + 15) / 16);
  const int64_t nb = a.Bt ? a.N * a.r : 0;
  if (i < nb) {
    const int64_t j = i / a.N, n = i % a.N;
    a.Bt[i] = a.B[n * a.r + j];
    return;
  }
  i -= nb;
  const int64_t na = a.At ? a.K * a.r : 0;
  if (i < na) {
    const int64_t k = i / a.r, j = i % a.r;
    a.At[i] = a.A[j * a.K + k];
    return;
  }
  i -= na;
  const int64_t nu = a.su ? rp * a.Mpu : 0;
  uint16_t* dst;
  int64_t count;
  float x = 0.f;
  if (i < nu) {
    const int64_t j = i / a.Mpu, m = i % a.Mpu;
    if (j < a.r && m < a.M) x = a.s * a.u[m * a.r + j];
    dst = a.su;
    count = nu;
  } else {
    i -= nu;
    const int64_t j = i / a.Mpv, m = i % a.Mpv;
    if (j < a.r && m < a.M) {
      const int64_t e = m * a.r + j;
      float val;
      if (a.Sv > 1) {
        val = slice_sum(a.vpart, a.M * a.r, a.Sv, e);
        a.v[e] = val;
      } else {
        val = a.v[e];
      }
      x = a.s * val;
    }
    dst = a.sv;
    count = rp * a.Mpv;
  }
  const uint32_t h = pack_bf16x2(x, 0.f) & 0xffffu;
  dst[i] = (uint16_t)h;
  dst[count + i] = (uint16_t)(pack_bf16x2(x - bf16_lo(h), 0.f) & 0xffffu);
}
hipError_t launch_bwd_aux(const BwdAux& a, hipStream_t st);

// out[k][n] = Qhat(W)[n][k] as bf16 with row length ldt (ldt % 8 == 0,
// ldt >= rows); zero for rows <= n < ldt.  cols % 64 == 0.  The jobs of
// aux run in extra workgroups of the same launch.
hipError_t launch_dequant_t(const uint8_t* packed, const uint8_t* qscale, const float* scale2,
                            const float* offset, int64_t rows, int64_t cols, uint16_t* out,
                            int64_t ldt, const BwdAux& aux, hipStream_t st);

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
};

// out[M, r] (fp32) = sum over S slices of Z[M, P] * T[r, P]^T.  When S > 1
// the slices are written to part[S][M][r] and summed in slice order into
// out; S == 1 writes out directly.
// sum == false leaves the slices in part for the caller to add.  t_rows:
// T is given as its transpose [P, r] (r <= 16 only).
hipError_t launch_thin_nt(const uint16_t* Z, const uint16_t* T, int64_t M, int64_t P, int r,
                          float* out, float* part, int S, hipStream_t st, bool sum = true,
                          bool t_rows = false);
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
};
// Two such products (same M and r) in one launch, their slice sums in a
// second.
hipError_t launch_thin_tn2(const ThinTn& a, const ThinTn& b, int64_t M, int r, hipStream_t st);
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
// to 4] and upart [bands, S, 256] fp32, 16-byte aligned.  Writes Y and u_out.  Calls on one device share
// a table of 64 call slots of arrival counters (taken round robin): more than
// 64 such calls in flight at once on one device would race.
struct DecodeTiles {
  int rgt, S, bands;
};
DecodeTiles decode_tiles(int64_t M, int64_t rows, int64_t cols, int r);
hipError_t launch_decode_tile(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                              const DecodeTiles& t, float* part, float* upart, hipStream_t st);

// Whole-row decode forward (M <= 16, r <= 16, cols 2048 or 4096): bands of
// `br` rows (a multiple of 8, at most 64), one workgroup each, every column;
// writes Y and u_out, no workspace.  decode_rows_band gives br, or 0 when the
// kernel does not apply (also when bands would be 32 rows or fewer).
int decode_rows_band(int64_t M, int64_t rows, int64_t cols, int r);
hipError_t launch_decode_rows(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                              int br, hipStream_t st);

// Y[M, N] bf16 = X[M, K] * W'[N, K]^T + s * u[M, r] * B[N, r]^T.
hipError_t launch_qgemm_fwd(const WState& w, const uint16_t* X, int64_t M, const float* u,
                            const uint16_t* B, int r, float s, uint16_t* Y, hipStream_t st);

// dX[M, K] bf16 = G[M, N] * W'[N, K] + s * v[M, r] * A[r, K].
hipError_t launch_qgemm_dx(const WState& w, const uint16_t* G, int64_t M, const float* v,
                           const uint16_t* A, int r, float s, uint16_t* dX, hipStream_t st);

}  // namespace qn
