// Dropout on the adapter branch (course notebook FT-02, the LoraConfig of
// the QLoRA setup: lora_dropout).  The keep mask is an input, bit-packed
// over the row-major elements of x [M, K] (bit e % 8 of byte e / 8 set:
// kept); kept elements pass unchanged and 1/(1-p) is folded into the
// branch's scale by the caller.  The products that read x apply the mask
// where they load it (u in the forward, dA in the backward); this file's
// streaming kernel, k_lora_masked_add, adds the branch's share of the input
// gradient, s ((G B) A) (.) mask, to the base product's dX.
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

// Thread = 4 consecutive columns k (one mask nibble, 8 bytes of dX) of a
// band of LB rows.  With r <= 16 (ONE) the thread's A[j][k .. k+3] are held
// in fp32 registers for the whole band, loaded before the first barrier;
// above 16 ranks they are reloaded in chunks of 16 for every row.  The rows go
// one after another, each row's v[m][j] read from LDS as broadcasts; they
// move in groups of RG, the next group's dX and mask loaded while the current
// one is computed.  At 8192 x 4096, r = 16: 39 us (groups of 8: 46 us at 3
// waves per SIMD; with a branch per rank, which kept every rank's LDS read
// waiting on its own, 55-59 us; one row ahead 66 us; a first design that
// converted A for every row 73 us).  Per
// element: t = sum_j v[m][j] A[j][k] in fp32 in rank order, then
// dX = bf16(dX + s t) where the mask bit is set (dX unchanged elsewhere).
constexpr int LB = 32;  // rows per workgroup
constexpr int RG = 4;   // rows per group (the next group's loads go out before this one's products)
template <bool ONE>
__global__ __launch_bounds__(256) void k_lora_masked_add(uint16_t* __restrict__ dX,
                                                         const float* __restrict__ v,
                                                         const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ mask,
                                                         int64_t M, int64_t K, int r, float s) {
  __shared__ float sv[LB][64];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * LB;
  // ONE: ranks r..15 are zero in both operands, so the products run without a
  // branch per rank; t starts at +0 and a sum of nonzero terms is never -0,
  // so adding +0 leaves every t as the sum over the r ranks alone
  const int rw = ONE ? 16 : r;
  for (int e = tid; e < LB * rw; e += 256) {
    const int i = e / rw, j = e - i * rw;
    sv[i][j] = j < r ? v[min(m0 + i, M - 1) * r + j] : 0.f;
  }
  const int64_t k = 4 * ((int64_t)blockIdx.x * 256 + tid);
  const int64_t kc = min(k, K - 4);  // K % 64 == 0: four columns never straddle a row
  float a[16][4];
  auto load_a = [&](int j0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint2 q = *reinterpret_cast<const uint2*>(A + (int64_t)min(j0 + j, r - 1) * K + kc);
      const bool live = !ONE || j < r;
      a[j][0] = live ? bf16_lo(q.x) : 0.f;
      a[j][1] = live ? bf16_hi(q.x) : 0.f;
      a[j][2] = live ? bf16_lo(q.y) : 0.f;
      a[j][3] = live ? bf16_hi(q.y) : 0.f;
    }
  };
  if (ONE) load_a(0);
  const int nrow = (int)min((int64_t)LB, M - m0);
  // a group's dX and mask nibbles (rows past the band repeat its last row and
  // are not stored; a thread past K loads at the clamped column, never stores)
  uint2 d[RG];
  uint32_t mb[RG];
  auto load_rows = [&](int i0, uint2* dd, uint32_t* mm) {
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int64_t e = (m0 + min(i0 + g, nrow - 1)) * K + kc;
      dd[g] = *reinterpret_cast<const uint2*>(dX + e);
      mm[g] = mask[e >> 3] >> (kc & 4);
    }
  };
  load_rows(0, d, mb);
  __syncthreads();
  for (int i0 = 0; i0 < nrow; i0 += RG) {
    uint2 dn[RG];
    uint32_t mn[RG];
    if (i0 + RG < nrow) load_rows(i0 + RG, dn, mn);  // the next group, ahead of this one
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int i = i0 + g;
      if (i >= nrow) break;
      float t[4] = {0.f, 0.f, 0.f, 0.f};
      if (ONE) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float vj = sv[i][j];
#pragma unroll
          for (int c = 0; c < 4; ++c) t[c] = __builtin_fmaf(vj, a[j][c], t[c]);
        }
      } else {
        for (int j0 = 0; j0 < r; j0 += 16) {
          load_a(j0);
          const int jn = min(16, r - j0);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            if (j < jn) {
              const float vj = sv[i][j0 + j];
#pragma unroll
              for (int c = 0; c < 4; ++c) t[c] = __builtin_fmaf(vj, a[j][c], t[c]);
            }
          }
        }
      }
      if (k < K) {
        const uint2 x = d[g];
        const uint32_t q = mb[g];
        float lo0 = bf16_lo(x.x), hi0 = bf16_hi(x.x), lo1 = bf16_lo(x.y), hi1 = bf16_hi(x.y);
        if (q & 1u) lo0 += s * t[0];
        if (q & 2u) hi0 += s * t[1];
        if (q & 4u) lo1 += s * t[2];
        if (q & 8u) hi1 += s * t[3];
        *reinterpret_cast<uint2*>(dX + (m0 + i) * K + k) =
            uint2{pack_bf16x2(lo0, hi0), pack_bf16x2(lo1, hi1)};
      }
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      d[g] = dn[g];
      mb[g] = mn[g];
    }
  }
}

}  // namespace

hipError_t launch_lora_masked_add(uint16_t* dX, const float* v, const uint16_t* A,
                                  const uint8_t* mask, int64_t M, int64_t K, int r, float s,
                                  hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const dim3 grid((unsigned)((K / 4 + 255) / 256), (unsigned)((M + LB - 1) / LB));
  if (r <= 16)
    hipLaunchKernelGGL(k_lora_masked_add<true>, grid, dim3(256), 0, st, dX, v, A, mask, M, K, r,
                       s);
  else
    hipLaunchKernelGGL(k_lora_masked_add<false>, grid, dim3(256), 0, st, dX, v, A, mask, M, K, r,
                       s);
  return hipGetLastError();
}

}  // namespace qn
