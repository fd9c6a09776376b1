// Rank-r adapter products of the QLoRA linear (page "QLoRA: NF4 storage,
// gradients and local integration", paragraph after the teaching listing):
//   u = X A^T and v = G B          -- "thin NT" products, reduction along a
//                                     row of both operands;
//   dB = s G^T u and dA = s v^T X  -- "thin TN" products, reduction over the
//                                     M rows, split in slices whose partial
//                                     sums are added in slice order.
// All use v_mfma_f32_16x16x32_bf16; fp32 operands (u, v) enter the MFMA as a
// bf16 high part plus a bf16 remainder, so they keep ~16 significant bits.
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 consecutive bf16 of a row at column p (zero past the row end P).
__device__ __forceinline__ u32x4 load8(const uint16_t* row, int64_t p, int64_t P) {
  if (p + 8 <= P) return *reinterpret_cast<const u32x4*>(row + p);
  uint32_t w[4];
  for (int h = 0; h < 4; ++h) {
    uint32_t lo = p + 2 * h < P ? row[p + 2 * h] : 0u;
    uint32_t hi = p + 2 * h + 1 < P ? row[p + 2 * h + 1] : 0u;
    w[h] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace

// out[M, r] = Z[M, P] T[r, P]^T.  Workgroup (mt, s): rows 16mt..16mt+15,
// columns of slice s; its four waves take consecutive quarters of the slice
// and their sums are added in wave order.  MFMA lane l holds row l%16 and
// the eight columns 8(l/16).. of each 32-wide step; the k order inside a step
// is the same for both operands, so the product is the plain dot product.
__global__ __launch_bounds__(kThreads) void k_thin_nt(const uint16_t* __restrict__ Z,
                                                      const uint16_t* __restrict__ T, int64_t M,
                                                      int64_t P, int r, int64_t slice,
                                                      float* __restrict__ out) {
  __shared__ float red[4][4][16][17];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int64_t p_begin = (int64_t)blockIdx.y * slice;
  const int64_t quarter = slice / 4;
  const int64_t pw0 = p_begin + wave * quarter;
  const int64_t pw1 = min(pw0 + quarter, P);
  const int nj = (r + 15) / 16;
  const int64_t m = min(m0 + (lane & 15), M - 1);
  const uint16_t* zrow = Z + m * P;
  f32x4 acc[4] = {};
  // uniform trip count; columns at or past pw1 load as zero (P and the
  // quarter bounds are multiples of 8, so a chunk is all in or all out)
  for (int64_t ps = pw0; ps < pw1; ps += 32) {
    const int64_t p = ps + 8 * (lane >> 4);
    const bf16x8 a = as_bf16x8(p < pw1 ? load8(zrow, p, pw1) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt < nj) {
        const int j = jt * 16 + (lane & 15);
        const u32x4 bv = (j < r && p < pw1) ? load8(T + (int64_t)j * P, p, P) : u32x4{0, 0, 0, 0};
        acc[jt] = mfma16(a, as_bf16x8(bv), acc[jt]);
      }
    }
  }
  // 16x16 result: lane l holds column l%16, rows 4(l/16)+i
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
    if (jt < nj)
      for (int i = 0; i < 4; ++i) red[wave][jt][4 * (lane >> 4) + i][lane & 15] = acc[jt][i];
  __syncthreads();
  for (int e = tid; e < 16 * r; e += kThreads) {
    const int row = e / r, j = e % r;
    const int jt = j / 16, jj = j % 16;
    const float s = ((red[0][jt][row][jj] + red[1][jt][row][jj]) + red[2][jt][row][jj]) +
                    red[3][jt][row][jj];
    if (m0 + row < M) out[((int64_t)blockIdx.y * M + m0 + row) * r + j] = s;
  }
}

// out[i] = sum over s of part[s][i], in slice order.
__global__ void k_sum_slices(const float* __restrict__ part, int64_t count, int S,
                             float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float acc = part[i];
  for (int s = 1; s < S; ++s) acc += part[(int64_t)s * count + i];
  out[i] = acc;
}

int thin_nt_slices(int64_t M, int64_t P) {
  const int64_t mt = (M + 15) / 16;
  int64_t S = 512 / (mt > 0 ? mt : 1);
  const int64_t smax = P / 256 > 0 ? P / 256 : 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  return (int)S;
}

hipError_t launch_thin_nt(const uint16_t* Z, const uint16_t* T, int64_t M, int64_t P, int r,
                          float* out, float* part, int S, hipStream_t st) {
  // slice width: a multiple of 128 so each wave's quarter is whole 32-steps
  int64_t slice = (P + S - 1) / S;
  slice = (slice + 127) / 128 * 128;
  const dim3 grid((unsigned)((M + 15) / 16), (unsigned)S);
  hipLaunchKernelGGL(k_thin_nt, grid, dim3(kThreads), 0, st, Z, T, M, P, r, slice,
                     S > 1 ? part : out);
  if (S > 1) {
    const int64_t count = M * r;
    hipLaunchKernelGGL(k_sum_slices, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                       part, count, S, out);
  }
  return hipGetLastError();
}

__global__ void k_fill_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

__global__ void k_transpose_b(const uint16_t* __restrict__ B, int64_t N, int r,
                              uint16_t* __restrict__ Bt) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * r) return;
  const int64_t n = i / r;
  const int j = (int)(i % r);
  Bt[(int64_t)j * N + n] = B[i];
}

hipError_t launch_transpose_b(const uint16_t* B, int64_t N, int r, uint16_t* Bt, hipStream_t st) {
  const int64_t count = N * r;
  hipLaunchKernelGGL(k_transpose_b, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, B, N,
                     r, Bt);
  return hipGetLastError();
}

// part[s][p][j] = sum over the rows m of slice s of Z[m, p] * (s*V[m, j]).
// Workgroup (pt, s): 64 columns p0..p0+63; wave w owns columns 16w..16w+15.
// Each 32-row step stages Z^T (64 x 32) and (sV)^T split in bf16 high and
// remainder parts (r x 32) in LDS, so that both MFMA operands read eight
// consecutive rows from one LDS row.
__global__ __launch_bounds__(kThreads) void k_thin_tn(const uint16_t* __restrict__ Z,
                                                      const float* __restrict__ V, int64_t M,
                                                      int64_t P, int r, float scale,
                                                      int64_t slice, float* __restrict__ part) {
  constexpr int LD = 40;  // 32 rows + 8 pad (bf16) per LDS row: 80 B
  __shared__ __attribute__((aligned(16))) uint16_t zt[64][LD];
  __shared__ __attribute__((aligned(16))) uint16_t vh[64][LD];
  __shared__ __attribute__((aligned(16))) uint16_t vl[64][LD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t p0 = (int64_t)blockIdx.x * 64;
  const int64_t mb = (int64_t)blockIdx.y * slice;
  const int64_t me = min(mb + slice, M);
  const int nj = (r + 15) / 16;
  f32x4 acc[4] = {};
  for (int64_t m = mb; m < me; m += 32) {
    {  // Z rows m..m+31, columns p0..p0+63 -> zt[p][row]
      const int row = tid >> 3, c = tid & 7;
      const int64_t mm = m + row, pp = p0 + 8 * c;
      u32x4 v = {0, 0, 0, 0};
      if (mm < me && pp < P) v = load8(Z + mm * P, pp, P);
      for (int h = 0; h < 4; ++h) {
        zt[8 * c + 2 * h][row] = (uint16_t)(v[h] & 0xffffu);
        zt[8 * c + 2 * h + 1][row] = (uint16_t)(v[h] >> 16);
      }
    }
    for (int e = tid; e < 32 * 16 * nj; e += kThreads) {  // (sV)^T, zero past r / rows
      const int row = e / (16 * nj), j = e % (16 * nj);
      const int64_t mm = m + row;
      const float x = (mm < me && j < r) ? scale * V[mm * r + j] : 0.f;
      const uint32_t hi = pack_bf16x2(x, 0.f) & 0xffffu;
      const float rem = x - bf16_lo(hi);
      vh[j][row] = (uint16_t)hi;
      vl[j][row] = (uint16_t)(pack_bf16x2(rem, 0.f) & 0xffffu);
    }
    __syncthreads();
    const int kk = 8 * (lane >> 4);
    const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&zt[16 * wave + (lane & 15)][kk]));
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt < nj) {
        const int j = 16 * jt + (lane & 15);
        const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&vh[j][kk]));
        const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&vl[j][kk]));
        acc[jt] = mfma16(a, bh, acc[jt]);
        acc[jt] = mfma16(a, bl, acc[jt]);
      }
    }
    __syncthreads();
  }
  // lane l: column j = 16jt + l%16, rows p = 16w + 4(l/16) + i
  float* dst = part + (int64_t)blockIdx.y * P * r;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    if (jt >= nj) continue;
    const int j = 16 * jt + (lane & 15);
    if (j >= r) continue;
    for (int i = 0; i < 4; ++i) {
      const int64_t p = p0 + 16 * wave + 4 * (lane >> 4) + i;
      if (p < P) dst[p * r + j] = acc[jt][i];
    }
  }
}

// out = sum over slices of part (slice order); transposed: out[j][p].
__global__ void k_sum_slices_tn(const float* __restrict__ part, int64_t P, int r, int S,
                                bool transposed, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t count = P * r;
  if (i >= count) return;
  float acc = part[i];
  for (int s = 1; s < S; ++s) acc += part[(int64_t)s * count + i];
  if (transposed)
    out[(i % r) * P + i / r] = acc;
  else
    out[i] = acc;
}

int thin_tn_slices(int64_t M, int64_t P) {
  const int64_t pt = (P + 63) / 64;
  int64_t S = 512 / (pt > 0 ? pt : 1);
  const int64_t smax = (M + 255) / 256;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  return (int)S;
}

hipError_t launch_thin_tn(const uint16_t* Z, const float* V, int64_t M, int64_t P, int r,
                          float s, float* out, bool transposed, float* part, int S,
                          hipStream_t st) {
  int64_t slice = (M + S - 1) / S;
  slice = (slice + 31) / 32 * 32;
  const dim3 grid((unsigned)((P + 63) / 64), (unsigned)S);
  hipLaunchKernelGGL(k_thin_tn, grid, dim3(kThreads), 0, st, Z, V, M, P, r, s, slice, part);
  const int64_t count = P * r;
  hipLaunchKernelGGL(k_sum_slices_tn, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                     part, P, r, S, transposed, out);
  return hipGetLastError();
}

}  // namespace qn
