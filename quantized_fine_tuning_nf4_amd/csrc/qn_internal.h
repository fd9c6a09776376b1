// Host-side launchers of the HIP kernels (one translation unit each).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Adapter transposes done by spare workgroups of another launch:
// At [K, r] = A[r, K]^T and Bt [r, N] = B[N, r]^T (bf16); a null A or B
// skips that one.
struct AdapterTransposes {
  const uint16_t* A;
  uint16_t* At;
  int64_t K;
  const uint16_t* B;
  uint16_t* Bt;
  int64_t N;
  int r;
};

// out[k][n] = Qhat(W)[n][k] as bf16 with row length ldt (ldt % 8 == 0,
// ldt >= rows); zero for rows <= n < ldt.  cols % 64 == 0.  The transposes
// in tj run in the same launch.
hipError_t launch_dequant_t(const uint8_t* packed, const uint8_t* qscale, const float* scale2,
                            const float* offset, int64_t rows, int64_t cols, uint16_t* out,
                            int64_t ldt, const AdapterTransposes& tj, hipStream_t st);

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
// sum == false leaves the slices in part for the caller to add.
hipError_t launch_thin_nt(const uint16_t* Z, const uint16_t* T, int64_t M, int64_t P, int r,
                          float* out, float* part, int S, hipStream_t st, bool sum = true);
int thin_nt_slices(int64_t M, int64_t P);

// p[0..n) = 0 (a kernel, so it may sit in a captured graph).
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

// Bt[r, N] = B[N, r]^T (bf16).
hipError_t launch_transpose_b(const uint16_t* B, int64_t N, int r, uint16_t* Bt, hipStream_t st);

// One transposed adapter product out = Z^T (s V), reduced over the M rows:
// Z bf16 [M, P] (null: no product), V fp32 [M, r]; transposed == false:
// out fp32 [P, r]; true: out fp32 [r, P].  Split over
// thin_tn_slices(M, P, r) row slices with partials part[S][P][r], summed in
// slice order.  P % 8 == 0.
struct ThinTn {
  const uint16_t* Z;
  const float* V;
  int64_t P;
  float* out;
  bool transposed;
  float* part;
};
// Two such products (same M, r and s) in one launch, their slice sums in a
// second.
hipError_t launch_thin_tn2(const ThinTn& a, const ThinTn& b, int64_t M, int r, float s,
                           hipStream_t st);
int thin_tn_slices(int64_t M, int64_t P, int r);

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

// Y[M, N] bf16 = X[M, K] * W'[N, K]^T + s * u[M, r] * B[N, r]^T.
hipError_t launch_qgemm_fwd(const WState& w, const uint16_t* X, int64_t M, const float* u,
                            const uint16_t* B, int r, float s, uint16_t* Y, hipStream_t st);

// dX[M, K] bf16 = G[M, N] * W'[N, K] + s * v[M, r] * A[r, K].
hipError_t launch_qgemm_dx(const WState& w, const uint16_t* G, int64_t M, const float* v,
                           const uint16_t* A, int r, float s, uint16_t* dX, hipStream_t st);

}  // namespace qn
