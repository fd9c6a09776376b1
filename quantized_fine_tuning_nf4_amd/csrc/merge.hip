// Adapter merge into the dequantized weight (page "QLoRA: NF4 storage,
// gradients and local integration", section "Merge changes the operator:
// test it explicitly"):
//   out[n][k] = RN32(RN64(w'[n][k] + RN64(s d))),  d = sum_j B[n][j] A[j][k]
// with w' = RN32(L[c] s') the dequantized weight (exactly nf4_dequantize's
// fp32 value) and d summed in fp64 in rank order (a product of two bf16
// values is exact in fp64).  Requantizing the merged weight is
// nf4_quantize_dq on `out`.
//
// Thread = four neighbouring columns of a band of MB rows; a workgroup covers
// 1024 columns of the band, whose B rows it keeps in LDS as fp64.  The ranks
// go in chunks of RC whose A[j][k..k+3] the thread holds as bf16 pairs; every
// global load of the first chunk, the codes and the block scales is issued
// before the first barrier.  Rank by rank, every row of the band takes its
// B[n][j] (one LDS broadcast serves four columns) against the rank's four A
// values, so each element adds its rank products in rank order.  With cols a multiple of 4 a thread's four weights share one block,
// their codes are one 16-bit load and the output one 16-byte store; other
// widths go element by element.
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int MB = 4;    // rows per workgroup
constexpr int RC = 8;    // ranks per chunk of A held in registers
constexpr int CW = 4;    // columns per thread

template <int CB, bool ABS, bool VEC>
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
  const int64_t k0 = ((int64_t)blockIdx.x * 256 + tid) * CW;
  int64_t kc[CW];  // columns past the end compute on the last one
#pragma unroll
  for (int c = 0; c < CW; ++c) kc[c] = min(k0 + c, cols - 1);
  const float mu = ABS ? 0.f : *offset;
  // VEC: every row's code bits and block scale are loaded ahead of the rank
  // products, so their latency overlaps the fp64 work
  uint32_t qv[MB];
  float sv[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    qv[i] = 0u;
    sv[i] = 0.f;
    if (VEC && k0 < cols && n0 + i < rows) {
      const int64_t e0 = (n0 + i) * cols + k0;  // e0 % 4 == 0: one block, two code bytes
      qv[i] = *reinterpret_cast<const uint16_t*>(packed + (e0 >> 1));
      const int64_t b = e0 / kBlock;
      sv[i] = ABS ? absmax[b] : dq_scale(qscale[b], scale2[b / kGroup], mu);
    }
  }
  // the first chunk of A, as bf16 pairs: ranks j0..j0+RC-1 of the thread's
  // four columns (ranks past r repeat the last one and are skipped)
  uint32_t ap[RC][2];
  auto load_a = [&](int j0) {
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      const uint16_t* arow = A + (int64_t)min(j0 + j, r - 1) * cols;
      if (VEC && k0 < cols) {  // k0 % 4 == 0 and cols % 4 == 0: one 8-byte load
        const uint2 v = *reinterpret_cast<const uint2*>(arow + k0);
        ap[j][0] = v.x;
        ap[j][1] = v.y;
      } else {
        ap[j][0] = (uint32_t)arow[kc[0]] | ((uint32_t)arow[kc[1]] << 16);
        ap[j][1] = (uint32_t)arow[kc[2]] | ((uint32_t)arow[kc[3]] << 16);
      }
    }
  };
  load_a(0);
  double acc[MB][CW];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[i][c] = 0.0;
  __syncthreads();
  // one rank at a time over every row of the band, so each element adds its
  // rank products in rank order
  auto rank = [&](int j, int jj) {
    const double a[CW] = {(double)bf16_lo(ap[jj][0]), (double)bf16_hi(ap[jj][0]),
                          (double)bf16_lo(ap[jj][1]), (double)bf16_hi(ap[jj][1])};
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const double b = sb[i][j];
#pragma unroll
      for (int c = 0; c < CW; ++c) acc[i][c] = __builtin_fma(b, a[c], acc[i][c]);
    }
  };
  for (int j0 = 0;;) {
    const int jn = min(RC, r - j0);
    if (jn == RC) {
#pragma unroll
      for (int jj = 0; jj < RC; ++jj) rank(j0 + jj, jj);
    } else {
#pragma unroll
      for (int jj = 0; jj < RC; ++jj)
        if (jj < jn) rank(j0 + jj, jj);
    }
    j0 += RC;
    if (j0 >= r) break;
    load_a(j0);
  }
  if (k0 >= cols) return;
  const double s64 = (double)s;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if (n0 + i >= rows) break;
    const int64_t e0 = (n0 + i) * cols + k0;
    if (VEC) {
      f32x4 o;
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        const float w = lut[(qv[i] >> (4 * c)) & 15u] * sv[i];
        o[c] = (float)((double)w + s64 * acc[i][c]);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(out + e0));
    } else {
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        if (k0 + c >= cols) break;
        const int64_t e = e0 + c;
        const uint32_t code = (packed[e >> 1] >> (4 * (uint32_t)(e & 1))) & 15u;
        const int64_t b = e / kBlock;
        const float w =
            lut[code] * (ABS ? absmax[b] : dq_scale(qscale[b], scale2[b / kGroup], mu));
        out[e] = (float)((double)w + s64 * acc[i][c]);
      }
    }
  }
}

}  // namespace

hipError_t launch_merge(const WState& w, const uint16_t* A, const uint16_t* B, int r, float s,
                        float* out, hipStream_t st, int codebook, const float* absmax) {
  const dim3 grid((unsigned)((w.cols + 256 * CW - 1) / (256 * CW)),
                  (unsigned)((w.rows + MB - 1) / MB));
  const bool vec = w.cols % CW == 0;
#define QN_MERGE(CB, ABS, VEC)                                                              \
  hipLaunchKernelGGL((k_merge<CB, ABS, VEC>), grid, dim3(256), 0, st, w.packed, w.qscale,   \
                     w.scale2, w.offset, absmax, w.rows, w.cols, A, B, r, s, out)
#define QN_MERGE_V(CB, ABS) \
  if (vec) QN_MERGE(CB, ABS, true); else QN_MERGE(CB, ABS, false)
  if (codebook == kCodeFP4) {
    if (absmax) { QN_MERGE_V(kCodeFP4, true); } else { QN_MERGE_V(kCodeFP4, false); }
  } else {
    if (absmax) { QN_MERGE_V(kCodeNF4, true); } else { QN_MERGE_V(kCodeNF4, false); }
  }
#undef QN_MERGE_V
#undef QN_MERGE
  return hipGetLastError();
}

}  // namespace qn
