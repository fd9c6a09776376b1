// Adapter merge into the dequantized weight (page "QLoRA: NF4 storage,
// gradients and local integration", section "Merge changes the operator:
// test it explicitly"):
//   out[n][k] = RN32(RN64(w'[n][k] + RN64(s d))),  d = sum_j B[n][j] A[j][k]
// with w' = RN32(L[c] s') the dequantized weight (exactly nf4_dequantize's
// fp32 value) and d summed in fp64 in rank order (a product of two bf16
// values is exact in fp64).  Requantizing the merged weight is
// nf4_quantize_dq on `out`.
//
// Thread = one column; a workgroup covers 256 columns of a band of MB rows,
// whose B rows it keeps in LDS as fp64.  The ranks go in chunks of 16: the
// chunk's A[j][k] are held as fp64 in registers and every row of the band
// accumulates its B[n][j] (an LDS broadcast) against them, so each rank's
// product is added in rank order.  Loads of a row's codes and scale
// codes are shared by neighbouring lanes.
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int MB = 16;   // rows per workgroup
constexpr int RC = 16;   // ranks per chunk

template <int CB, bool ABS>
__global__ __launch_bounds__(256) void k_merge(const uint8_t* __restrict__ packed,
                                               const uint8_t* __restrict__ qscale,
                                               const float* __restrict__ scale2,
                                               const float* __restrict__ offset,
                                               const float* __restrict__ absmax, int64_t rows,
                                               int64_t cols, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ B, int r, float s,
                                               float* __restrict__ out) {
  __shared__ float lut[16];
  __shared__ double sb[MB][64];  // the band's B rows as fp64 (read as broadcasts)
  const int tid = threadIdx.x;
  if (tid < 16) {  // levels from immediates
    uint32_t v = level_bits(CB, 0);
#pragma unroll
    for (int k = 1; k < 16; ++k) v = tid == k ? level_bits(CB, k) : v;
    lut[tid] = as_f32(v);
  }
  const int64_t n0 = (int64_t)blockIdx.y * MB;
  for (int e = tid; e < MB * r; e += 256) {
    const int i = e / r, j = e - i * r;  // rows past the end repeat the last one (not stored)
    sb[i][j] = (double)bf16_lo(B[min(n0 + i, rows - 1) * r + j]);
  }
  const int64_t k = (int64_t)blockIdx.x * 256 + tid;
  const int64_t kc = min(k, cols - 1);  // columns past the end compute on the last one
  double acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = 0.0;
  __syncthreads();
  for (int j0 = 0; j0 < r; j0 += RC) {
    const int jn = min(RC, r - j0);
    double a[RC];
#pragma unroll
    for (int j = 0; j < RC; ++j)
      a[j] = (double)bf16_lo(A[(int64_t)min(j0 + j, r - 1) * cols + kc]);
    // rank order within each element; ranks past r are skipped
    if (jn == RC) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < RC; ++j) acc[i] = __builtin_fma(sb[i][j0 + j], a[j], acc[i]);
    } else {
#pragma unroll
      for (int i = 0; i < MB; ++i)
        for (int j = 0; j < jn; ++j) acc[i] = __builtin_fma(sb[i][j0 + j], a[j], acc[i]);
    }
  }
  if (k >= cols) return;
  const float mu = ABS ? 0.f : *offset;
  const double s64 = (double)s;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if (n0 + i >= rows) break;
    const int64_t e = (n0 + i) * cols + k;
    const uint32_t c = (packed[e >> 1] >> (4 * (uint32_t)(e & 1))) & 15u;
    const int64_t b = e / kBlock;
    const float w = lut[c] * (ABS ? absmax[b] : dq_scale(qscale[b], scale2[b / kGroup], mu));
    const double t = s64 * acc[i];
    out[e] = (float)((double)w + t);
  }
}

}  // namespace

hipError_t launch_merge(const WState& w, const uint16_t* A, const uint16_t* B, int r, float s,
                        float* out, hipStream_t st, int codebook, const float* absmax) {
  const dim3 grid((unsigned)((w.cols + 255) / 256), (unsigned)((w.rows + MB - 1) / MB));
#define QN_MERGE(CB, ABS)                                                                  \
  hipLaunchKernelGGL((k_merge<CB, ABS>), grid, dim3(256), 0, st, w.packed, w.qscale, w.scale2, \
                     w.offset, absmax, w.rows, w.cols, A, B, r, s, out)
  if (codebook == kCodeFP4) {
    if (absmax) QN_MERGE(kCodeFP4, true); else QN_MERGE(kCodeFP4, false);
  } else {
    if (absmax) QN_MERGE(kCodeNF4, true); else QN_MERGE(kCodeNF4, false);
  }
#undef QN_MERGE
  return hipGetLastError();
}

}  // namespace qn
