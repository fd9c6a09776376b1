// Dropout on the adapter branch (course notebook FT-02, the LoraConfig of
// the QLoRA setup: lora_dropout).  The keep mask is an input, bit-packed
// over the row-major elements of x [M, K] (bit e % 8 of byte e / 8 set:
// kept); kept elements pass unchanged and 1/(1-p) is folded into the
// branch's scale by the caller.  Two streaming kernels:
//   - k_dropout_apply writes the branch's input mask (.) x (the backward's
//     dA product reads it);
//   - k_lora_masked_add adds the branch's share of the input gradient,
//     s ((G B) A) (.) mask, to the base product's dX.
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

// Thread = 8 consecutive elements (one mask byte, 16 bytes of x).
__global__ __launch_bounds__(256) void k_dropout_apply(const uint16_t* __restrict__ X,
                                                       const uint8_t* __restrict__ mask,
                                                       int64_t n8, uint16_t* __restrict__ Xd) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n8) return;
  u32x4 v = reinterpret_cast<const u32x4*>(X)[c];
  const uint32_t mb = mask[c];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] &= (((mb >> (2 * q)) & 1u) * 0xffffu) | (((mb >> (2 * q + 1)) & 1u) * 0xffff0000u);
  reinterpret_cast<u32x4*>(Xd)[c] = v;
}

// Thread = 8 consecutive columns k of one row band: A[j][k .. k+7] for the
// ranks of a chunk of 16 stay in registers (bf16 pairs), the rows of the
// band go one after another with their v[m][j] read from LDS as broadcasts.
// Per element: t = sum_j v[m][j] A[j][k] in fp32 in rank order, then
// dX = bf16(dX + s t) where the mask bit is set.
constexpr int LB = 8;   // rows per workgroup
__global__ __launch_bounds__(256) void k_lora_masked_add(uint16_t* __restrict__ dX,
                                                         const float* __restrict__ v,
                                                         const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ mask,
                                                         int64_t M, int64_t K, int r, float s) {
  __shared__ float sv[LB][64];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * LB;
  for (int e = tid; e < LB * r; e += 256) {
    const int i = e / r, j = e - i * r;
    sv[i][j] = v[min(m0 + i, M - 1) * r + j];
  }
  const int64_t k = 8 * ((int64_t)blockIdx.x * 256 + tid);
  const int64_t kc = min(k, K - 8);
  float t[LB][8];
#pragma unroll
  for (int i = 0; i < LB; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) t[i][q] = 0.f;
  __syncthreads();
  for (int j0 = 0; j0 < r; j0 += 16) {
    const int jn = min(16, r - j0);
    u32x4 a[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      a[j] = *reinterpret_cast<const u32x4*>(A + (int64_t)min(j0 + j, r - 1) * K + kc);
#pragma unroll
    for (int i = 0; i < LB; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j < jn) {
          const float vj = sv[i][j0 + j];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            t[i][2 * q] = __builtin_fmaf(vj, bf16_lo(a[j][q]), t[i][2 * q]);
            t[i][2 * q + 1] = __builtin_fmaf(vj, bf16_hi(a[j][q]), t[i][2 * q + 1]);
          }
        }
      }
  }
  if (k >= K) return;
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int64_t m = m0 + i;
    if (m >= M) break;
    const uint32_t mb = mask[(m * K + k) >> 3];
    u32x4* p = reinterpret_cast<u32x4*>(dX + m * K + k);
    const u32x4 d = *p;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float lo = bf16_lo(d[q]), hi = bf16_hi(d[q]);
      if ((mb >> (2 * q)) & 1u) lo += s * t[i][2 * q];
      if ((mb >> (2 * q + 1)) & 1u) hi += s * t[i][2 * q + 1];
      o[q] = pack_bf16x2(lo, hi);
    }
    *p = u32x4{o[0], o[1], o[2], o[3]};
  }
}

}  // namespace

hipError_t launch_dropout_apply(const uint16_t* X, const uint8_t* mask, int64_t M, int64_t K,
                                uint16_t* Xd, hipStream_t st) {
  const int64_t n8 = M * K / 8;
  if (n8 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_dropout_apply, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, X,
                     mask, n8, Xd);
  return hipGetLastError();
}

hipError_t launch_lora_masked_add(uint16_t* dX, const float* v, const uint16_t* A,
                                  const uint8_t* mask, int64_t M, int64_t K, int r, float s,
                                  hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const dim3 grid((unsigned)((K / 8 + 255) / 256), (unsigned)((M + LB - 1) / LB));
  hipLaunchKernelGGL(k_lora_masked_add, grid, dim3(256), 0, st, dX, v, A, mask, M, K, r, s);
  return hipGetLastError();
}

}  // namespace qn
