// Forward of decode-sized batches (M <= 16 rows):
//   y = X Qhat(W)^T + s u B^T
// (page "QLoRA: NF4 storage, gradients and local integration", paragraph
// after the teaching listing).  Streaming the NF4 weight is the cost, so the
// kernel reads every code byte once and keeps the per-element work small:
//   - a 256-entry LDS table maps one code byte to the bf16 pair
//     (L[low nibble], L[high nibble]), so one table read yields two
//     unscaled levels in MFMA operand form;
//   - v_mfma_f32_16x16x32_bf16 forms x . L[c] over half a block at a time,
//     and the block scale s' multiplies the fp32 partial of each 64-element
//     block (sum_k x_k (L[c_k] s') = s' sum_k x_k L[c_k]: the scale is applied
//     after the products instead of before a bf16 rounding of L[c] s').
// Workgroup (row group g, slice z): weight rows 64g .. 64g+63 (wave w: rows
// 64g + 16w .. +15), blocks z*nbs .. (z+1)*nbs-1 of every row; X's slice is
// staged in LDS once for the four waves.  Partial sums go to part[z][m][n];
// a second kernel adds the slices, the LoRA term and rounds to bf16.
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int T = 256;
constexpr int CB = 16;  // blocks per wave per pass (codes held in registers)

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 4 * (byte B of v) in one instruction (SDWA source byte select)
template <int B>
__device__ __forceinline__ uint32_t byte_x4(uint32_t v) {
  uint32_t r;
  if constexpr (B == 0)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(v));
  else if constexpr (B == 1)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(v));
  else if constexpr (B == 2)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(v));
  else
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(v));
  return r;
}

// bf16 pair of the two codes of byte `byte_x4 / 4`, from the pair table
__device__ __forceinline__ uint32_t pair_at(const uint8_t* tab, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(tab + off);
}
__device__ __forceinline__ u32x4 pairs4(const uint8_t* tab, uint32_t w) {
  return u32x4{pair_at(tab, byte_x4<0>(w)), pair_at(tab, byte_x4<1>(w)),
               pair_at(tab, byte_x4<2>(w)), pair_at(tab, byte_x4<3>(w))};
}

// X slice in LDS: M rows of nbs*64 bf16, row pitch nbs*128 + 16 bytes; the
// MFMA rows past M read zeros from registers.
// Workgroups with blockIdx.x == groups compute u's partial over the slice
// instead: upart[z][m][j] = sum_k X[m][k] A[j][k] (wave w: ranks 16w ..).
__global__ __launch_bounds__(T, 4) void k_decode_partial(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ scale2, const float* __restrict__ offset,
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Aad, int r, int64_t M,
    int64_t N, int64_t K, int nbs, float* __restrict__ part, float* __restrict__ upart) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t s_tab[256];
  __shared__ float s_e4m3[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  {  // pair table: entry b = bf16(L[b & 15]) | bf16(L[b >> 4]) << 16
    const float lo = as_f32(kNF4Bits[tid & 15]), hi = as_f32(kNF4Bits[tid >> 4]);
    s_tab[tid] = pack_bf16x2(lo, hi);
    s_e4m3[tid] = e4m3_to_f32(tid);  // scale code -> value
  }
  const uint8_t* tab = reinterpret_cast<const uint8_t*>(s_tab);
  const int64_t groups = (N + 63) / 64;
  const bool u_wg = blockIdx.x == groups;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int z = blockIdx.y;
  const int64_t kblocks = K / 64;
  const int64_t b0 = (int64_t)z * nbs;  // first block column of the slice
  const int pitch = nbs * 128 + 16;
  const int64_t n = min(n0 + 16 * wave + l16, N - 1);
  const uint8_t* crow = packed + n * (K / 2) + 8 * g4;

  uint2 code[CB];
  u32x4 q4 = {0u, 0u, 0u, 0u};
  float s2 = 0.f;
  auto load_pass = [&](int jb) {
    const int64_t bb = b0 + jb;
#pragma unroll
    for (int j = 0; j < CB; ++j) code[j] = *reinterpret_cast<const uint2*>(crow + (bb + j) * 32);
    q4 = *reinterpret_cast<const u32x4*>(qscale + n * kblocks + bb);
    s2 = scale2[(n * kblocks + bb) / kGroup];
  };
  // ---- stage X[0:M, slice] (nbs == 16: at most 8 16-byte chunks per
  // thread) before the weight loads go out, so that waiting for X does not
  // wait for them
  {
    constexpr int XCH = 16 * 16 * 8 / T;
    const int chunks_per_row = nbs * 8;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + T * i, m = c / chunks_per_row, q = c % chunks_per_row;
      if (m < M)
        *reinterpret_cast<u32x4*>(smem + m * pitch + 16 * q) =
            *reinterpret_cast<const u32x4*>(X + m * K + b0 * 64 + 8 * q);
    }
  }
  __syncthreads();
  if (!u_wg) load_pass(0);

  // A fragment of half h of block j: row l16, k = 64 j + 16 g4 + 8 h; rows
  // past M are zero
  const bool xrow_ok = l16 < M;
  const uint8_t* xrow = smem + min(l16, (int)M - 1) * pitch + 32 * g4;
  auto xfrag = [&](int off) {
    u32x4 v = *reinterpret_cast<const u32x4*>(xrow + off);
    if (!xrow_ok) v = u32x4{0u, 0u, 0u, 0u};
    return as_bf16x8(v);
  };
  if (u_wg) {
    // u partial: B operand = adapter rows j = 16 wave + l16 (zero past r)
    if (16 * wave >= r) return;
    const int j = 16 * wave + l16;
    const uint16_t* arow = Aad + (int64_t)min(j, r - 1) * K + b0 * 64 + 16 * g4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int jb = 0; jb < nbs; ++jb) {
      u32x4 w0 = *reinterpret_cast<const u32x4*>(arow + jb * 64);
      u32x4 w1 = *reinterpret_cast<const u32x4*>(arow + jb * 64 + 8);
      if (j >= r) w0 = w1 = u32x4{0u, 0u, 0u, 0u};
      const bf16x8 a0 = xfrag(jb * 128);
      const bf16x8 a1 = xfrag(jb * 128 + 16);
      acc = mfma16(a0, as_bf16x8(w0), acc);
      acc = mfma16(a1, as_bf16x8(w1), acc);
    }
    if (j < r) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g4 + v;
        if (m < M) upart[((int64_t)z * M + m) * r + j] = acc[v];
      }
    }
    return;
  }

  const float mu = *offset;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int jb = 0; jb < nbs; jb += CB) {
    if (jb > 0) load_pass(jb);
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const uint32_t qb = (q4[j >> 2] >> (8 * (j & 3))) & 0xffu;
      const float sc = __builtin_fmaf(s_e4m3[qb], s2, mu);
      const bf16x8 a0 = xfrag((jb + j) * 128);
      const bf16x8 a1 = xfrag((jb + j) * 128 + 16);
      const bf16x8 w0 = as_bf16x8(pairs4(tab, code[j].x));
      const bf16x8 w1 = as_bf16x8(pairs4(tab, code[j].y));
      f32x4 t = mfma16(a0, w0, f32x4{0.f, 0.f, 0.f, 0.f});
      t = mfma16(a1, w1, t);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(sc, t[v], acc[v]);
      // one block at a time: no hoisting of later blocks' LDS reads
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // lane holds rows m = 4 g4 + v of column n
  if (n0 + 16 * wave + l16 < N) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g4 + v;
      if (m < M) part[((int64_t)z * M + m) * N + n] = acc[v];
    }
  }
}

// Workgroup (bx, m): row m, columns 256 bx .. +255:
//   y[m][n] = bf16(sum_z part[z][m][n] + s * sum_j u[m][j] B[n][j]),
// u[m] = sum_z upart[z][m] (workgroups bx == 0 also write it to u_out).
__global__ __launch_bounds__(T) void k_decode_finish(const float* __restrict__ part,
                                                     const float* __restrict__ upart, int S,
                                                     int64_t M, int64_t N,
                                                     const uint16_t* __restrict__ B, int r,
                                                     float s, uint16_t* __restrict__ Y,
                                                     float* __restrict__ u_out) {
  __shared__ float su[64];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.y;
  if (tid < r) {
    float a = 0.f;
    for (int z = 0; z < S; ++z) a += upart[((int64_t)z * M + m) * r + tid];
    su[tid] = a;
    if (blockIdx.x == 0) u_out[m * r + tid] = a;
  }
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * T + tid;
  if (n >= N) return;
  float acc = 0.f;
  for (int z = 0; z < S; ++z) acc += part[((int64_t)z * M + m) * N + n];
  float lora = 0.f;
  for (int j = 0; j < r; ++j) lora = __builtin_fmaf(su[j], bf16_lo(B[n * r + j]), lora);
  Y[m * N + n] = (uint16_t)(pack_bf16x2(__builtin_fmaf(s, lora, acc), 0.f) & 0xffffu);
}

}  // namespace

int decode_slices(int64_t M, int64_t N, int64_t K) {
  // one slice per 16 blocks (1024 columns) of the weight
  (void)N;
  if (M < 1 || M > 16 || K % 1024 != 0) return 0;
  return (int)(K / 1024);
}

hipError_t launch_decode_fwd(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                             const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                             float* part, float* upart, int S, hipStream_t st) {
  const int64_t N = w.rows, K = w.cols;
  const int nbs = (int)(K / 64 / S);
  const size_t lds = (size_t)M * (nbs * 128 + 16);
  constexpr size_t kMaxLds = 64 * 1024;  // X slice: at most 16 rows of 16 blocks
  static hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(k_decode_partial),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
  if (attr != hipSuccess) return attr;
  if (nbs != 16 || lds > kMaxLds) return hipErrorInvalidValue;
  const int64_t groups = (N + 63) / 64;
  const dim3 grid((unsigned)(groups + 1), (unsigned)S);
  hipLaunchKernelGGL(k_decode_partial, grid, dim3(T), lds, st, w.packed, w.qscale, w.scale2,
                     w.offset, X, A, r, M, N, K, nbs, part, upart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_finish, dim3((unsigned)((N + T - 1) / T), (unsigned)M), dim3(T), 0,
                     st, part,
                     upart, S, M, N, B, r, s, Y, u_out);
  return hipGetLastError();
}

}  // namespace qn
