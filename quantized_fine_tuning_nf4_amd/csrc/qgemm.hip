// Fused NF4-dequant bf16 MFMA GEMMs of the QLoRA linear (gfx950).
//
//   forward  Y  = X Qhat(W)^T + s (X A^T) B^T      (u = X A^T precomputed)
//   backward dX = G Qhat(W)   + s (G B) A          (v = G B precomputed)
// (page "QLoRA: NF4 storage, gradients and local integration", paragraph
// after the teaching listing; s = alpha / r as in the course notebook's
// LoRALinear.)  Qhat(W) is the dequantized weight w' = L[c] * s', rounded to
// bf16 (round to nearest even) as the MFMA operand -- the compute dtype the
// pages recommend -- and never written to memory: each workgroup dequantizes
// the tile it needs into LDS.
//
// Tiling: a workgroup computes a BM x BN output tile with WM x WN waves, each
// wave TM x TN tiles of v_mfma_f32_32x32x16_bf16.  The reduction advances 64
// at a time (in the forward one NF4 block per weight row, so one scale per
// row per step).  LDS holds two stages of the activation tile and of the
// dequantized weight tile, rows padded to 144 B so that 32 lanes reading 16 B
// from 32 consecutive rows hit distinct banks.  Global loads of the next step
// are issued before the MFMAs of the current one.
//
// MFMA operand layout used here: lane l supplies row (or column) l%32 and
// eight reduction elements 8(l/32)+0..7 of a 16-wide step; the same element
// order is used for both operands, so the hardware's internal k order does
// not matter.  Accumulator register v of lane l holds row
// 8(v/4) + 4(l/32) + v%4, column l%32 of the 32x32 tile.
#include <type_traits>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int BK = 64;   // reduction step
constexpr int LDK = 72;  // LDS row length in bf16 (64 + 8 pad)

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

template <int WM, int WN, int TM, int TN>
struct Tile {
  static constexpr int BM = WM * TM * 32;
  static constexpr int BN = WN * TN * 32;
  static constexpr int T = 64 * WM * WN;
  static constexpr int A_CHUNKS = BM * 8 / T;  // 16-byte chunks of the activation tile
  static constexpr size_t LDS =
      (size_t)2 * (BM + BN) * LDK * sizeof(uint16_t) + 16 * sizeof(float);
  static_assert(BM * 8 % T == 0, "activation tile must split evenly");
};

// Activation tile rows m0.., reduction columns c0..c0+63 of a row-major bf16
// matrix with row length ld; rows past `rows` are clamped (their results are
// never stored), columns at or past `cols` load as zero.
template <class Cfg>
__device__ __forceinline__ void load_act(const uint16_t* __restrict__ Xm, int64_t ld,
                                         int64_t rows, int64_t cols, int64_t m0, int64_t c0,
                                         u32x4 (&reg)[Cfg::A_CHUNKS]) {
#pragma unroll
  for (int i = 0; i < Cfg::A_CHUNKS; ++i) {
    const int c = threadIdx.x + i * Cfg::T;
    const int64_t m = min(m0 + (c >> 3), rows - 1);
    const int64_t k = c0 + 8 * (c & 7);
    reg[i] = k < cols ? *reinterpret_cast<const u32x4*>(Xm + m * ld + k) : u32x4{0, 0, 0, 0};
  }
}

template <class Cfg>
__device__ __forceinline__ void store_act(uint16_t* sA, const u32x4 (&reg)[Cfg::A_CHUNKS]) {
#pragma unroll
  for (int i = 0; i < Cfg::A_CHUNKS; ++i) {
    const int c = threadIdx.x + i * Cfg::T;
    *reinterpret_cast<u32x4*>(sA + (c >> 3) * LDK + 8 * (c & 7)) = reg[i];
  }
}

// MFMAs of one 64-deep step from LDS stage (sA, sB).
template <class Cfg, int WM, int WN, int TM, int TN>
__device__ __forceinline__ void mma_step(const uint16_t* sA, const uint16_t* sB,
                                         f32x16 (&acc)[TM][TN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const uint16_t* pa = sA + (wm * TM * 32 + (lane & 31)) * LDK + 8 * (lane >> 5);
  const uint16_t* pb = sB + (wn * TN * 32 + (lane & 31)) * LDK + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    bf16x8 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(pa + i * 32 * LDK + ks * 16));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(pb + j * 32 * LDK + ks * 16));
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

// bf16 high part and bf16 remainder of s * v[m][j..j+7] (zero for j >= r).
__device__ __forceinline__ void lora_rows(const float* __restrict__ V, int64_t m, int r, int j0,
                                          float s, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = j0 + 2 * q;
    const float x0 = j < r ? s * V[m * r + j] : 0.f;
    const float x1 = j + 1 < r ? s * V[m * r + j + 1] : 0.f;
    h[q] = pack_bf16x2(x0, x1);
    l[q] = pack_bf16x2(x0 - bf16_lo(h[q]), x1 - bf16_hi(h[q]));
  }
  hi = as_bf16x8(u32x4{h[0], h[1], h[2], h[3]});
  lo = as_bf16x8(u32x4{l[0], l[1], l[2], l[3]});
}

template <int WM, int WN, int TM, int TN>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[TM][TN], uint16_t* __restrict__ Out,
                                           int64_t rows, int64_t cols, int64_t m0, int64_t n0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wn * TN * 32 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * TM * 32 + i * 32 + acc_row(v, lane);
        if (row < rows && col < cols)
          Out[row * cols + col] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.f) & 0xffffu);
      }
    }
}

// --------------------------------------------------------------------------
// Forward.  Weight tile: BN rows n0.. of W, columns k0..k0+63 = one NF4 block
// per row.  Thread t dequantizes SPT consecutive 16-weight segments of one
// row (8 packed bytes each) and writes them as bf16 to sB[row][...].
// CB: the codebook (NF4 or FP4); ABS: double quantization off (the block
// scales read from absmax instead of decoded from qscale, scale2, offset).
template <int WM, int WN, int TM, int TN, int CB, bool ABS>
__global__ __launch_bounds__(64 * WM * WN) void k_qgemm_fwd(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ scale2, const float* __restrict__ offset,
    const float* __restrict__ absmax, const uint16_t* __restrict__ X, const float* __restrict__ U, const uint16_t* __restrict__ Bl,
    int64_t M, int64_t N, int64_t K, int r, float s, uint16_t* __restrict__ Y, int tiles_n) {
  using Cfg = Tile<WM, WN, TM, TN>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, T = Cfg::T;
  constexpr int SPT = BN * 4 / T;  // 16-weight segments per thread
  static_assert(SPT == 1 || SPT == 2 || SPT == 4, "weight tile split");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sB = sA + 2 * BM * LDK;
  float* lut = reinterpret_cast<float*>(sB + 2 * BN * LDK);
  const int tid = threadIdx.x;
  if (tid < 16) lut[tid] = as_f32(level_bits(CB, tid));

  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
  const float mu = ABS ? 0.f : *offset;
  const int64_t kblocks = K / BK;

  // this thread's weight segments: row wr of the tile, segments ws0..ws0+SPT-1
  const int wr = tid * SPT / 4, ws0 = tid * SPT % 4;
  const int64_t wn_row = min(n0 + wr, N - 1);
  const uint8_t* wp = packed + wn_row * (K / 2) + ws0 * 8;

  u32x4 areg[Cfg::A_CHUNKS];
  uint32_t wreg[2 * SPT];
  float wscale;
  auto load_w = [&](int64_t kb) {
    const uint8_t* p = wp + kb * 32;
    if constexpr (SPT == 4) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(p);
      const u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
      wreg[0] = a[0]; wreg[1] = a[1]; wreg[2] = a[2]; wreg[3] = a[3];
      wreg[4] = b[0]; wreg[5] = b[1]; wreg[6] = b[2]; wreg[7] = b[3];
    } else if constexpr (SPT == 2) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(p);
      wreg[0] = a[0]; wreg[1] = a[1]; wreg[2] = a[2]; wreg[3] = a[3];
    } else {
      const u32x2 a = *reinterpret_cast<const u32x2*>(p);
      wreg[0] = a[0]; wreg[1] = a[1];
    }
    const int64_t b = wn_row * kblocks + kb;
    wscale = ABS ? absmax[b] : dq_scale(qscale[b], scale2[b / kGroup], mu);
  };
  auto store_w = [&](uint16_t* sBs) {
    uint16_t* dst = sBs + wr * LDK + ws0 * 16;
#pragma unroll
    for (int q = 0; q < 2 * SPT; q += 2) {
      uint32_t d[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t p = wreg[q + h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = lut[(p >> (8 * e)) & 15u] * wscale;
          const float hi = lut[(p >> (8 * e + 4)) & 15u] * wscale;
          d[4 * h + e] = pack_bf16x2(lo, hi);
        }
      }
      *reinterpret_cast<u32x4*>(dst + q * 8) = u32x4{d[0], d[1], d[2], d[3]};
      *reinterpret_cast<u32x4*>(dst + q * 8 + 8) = u32x4{d[4], d[5], d[6], d[7]};
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  load_act<Cfg>(X, K, M, K, m0, 0, areg);
  load_w(0);
  __syncthreads();  // LUT
  store_act<Cfg>(sA, areg);
  store_w(sB);
  __syncthreads();
  for (int64_t kb = 0; kb < kblocks; ++kb) {
    const int cur = (int)(kb & 1);
    const bool more = kb + 1 < kblocks;
    if (more) {
      load_act<Cfg>(X, K, M, K, m0, (kb + 1) * BK, areg);
      load_w(kb + 1);
    }
    mma_step<Cfg, WM, WN, TM, TN>(sA + cur * BM * LDK, sB + cur * BN * LDK, acc);
    if (more) {
      store_act<Cfg>(sA + (cur ^ 1) * BM * LDK, areg);
      store_w(sB + (cur ^ 1) * BN * LDK);
    }
    __syncthreads();
  }

  // LoRA term: acc += (s u) B^T, r in steps of 16
  {
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    for (int j0 = 0; j0 < r; j0 += 16) {
      const int jl = j0 + 8 * (lane >> 5);
      bf16x8 bh[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = min(n0 + wn * TN * 32 + j * 32 + (lane & 31), N - 1);
        uint32_t w4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jj = jl + 2 * q;
          const uint32_t lo = jj < r ? Bl[n * r + jj] : 0u;
          const uint32_t hi = jj + 1 < r ? Bl[n * r + jj + 1] : 0u;
          w4[q] = lo | (hi << 16);
        }
        bh[j] = as_bf16x8(u32x4{w4[0], w4[1], w4[2], w4[3]});
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t m = min(m0 + wm * TM * 32 + i * 32 + (lane & 31), M - 1);
        bf16x8 ah, al;
        lora_rows(U, m, r, jl, s, ah, al);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = mfma32(ah, bh[j], acc[i][j]);
          acc[i][j] = mfma32(al, bh[j], acc[i][j]);
        }
      }
    }
  }
  store_tile<WM, WN, TM, TN>(acc, Y, M, N, m0, n0);
}

// --------------------------------------------------------------------------
// Backward input gradient.  Reduction over the N weight rows, 64 at a time;
// the weight tile is rows n0..n0+63, columns k0..k0+BN-1 of W, stored in LDS
// transposed (sB[k][n]).  A thread unit is 8 rows x 8 columns: eight u32 of
// codes (one per row, one scale per row), written as eight 16-byte LDS rows
// of eight n-values.  Rows past N are zero.
template <int WM, int WN, int TM, int TN, int CB, bool ABS>
__global__ __launch_bounds__(64 * WM * WN) void k_qgemm_dx(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ scale2, const float* __restrict__ offset,
    const float* __restrict__ absmax, const uint16_t* __restrict__ G, const float* __restrict__ Vv, const uint16_t* __restrict__ Al,
    int64_t M, int64_t N, int64_t K, int r, float s, uint16_t* __restrict__ dX, int tiles_k) {
  using Cfg = Tile<WM, WN, TM, TN>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, T = Cfg::T;
  constexpr int UPT = (BN + T - 1) / T;  // 8x8 units per thread (BN units in all)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sB = sA + 2 * BM * LDK;
  float* lut = reinterpret_cast<float*>(sB + 2 * BN * LDK);
  const int tid = threadIdx.x;
  if (tid < 16) lut[tid] = as_f32(level_bits(CB, tid));

  const int64_t m0 = (int64_t)(blockIdx.x / tiles_k) * BM;
  const int64_t k0 = (int64_t)(blockIdx.x % tiles_k) * BN;
  const float mu = ABS ? 0.f : *offset;
  const int64_t kblocks = K / BK;
  const int64_t nsteps = (N + BK - 1) / BK;

  u32x4 areg[Cfg::A_CHUNKS];
  uint32_t wreg[UPT][8];
  float wsc[UPT][8];
  auto load_w = [&](int64_t n0) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + u * T;
      const int rg = unit / (BN / 8), kc = unit % (BN / 8);
      const int64_t k = min(k0 + 8 * kc, K - 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t n = n0 + 8 * rg + i;
        const bool ok = unit < BN && n < N;
        const int64_t nc = min(n, N - 1);
        wreg[u][i] = *reinterpret_cast<const uint32_t*>(packed + (nc * K + k) / 2);
        const int64_t b = nc * kblocks + k / BK;
        wsc[u][i] = ok ? (ABS ? absmax[b] : dq_scale(qscale[b], scale2[b / kGroup], mu)) : 0.f;
      }
    }
  };
  auto store_w = [&](uint16_t* sBs) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + u * T;
      if (unit >= BN) continue;
      const int rg = unit / (BN / 8), kc = unit % (BN / 8);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t d[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float a = lut[(wreg[u][2 * h] >> (4 * c)) & 15u] * wsc[u][2 * h];
          const float b = lut[(wreg[u][2 * h + 1] >> (4 * c)) & 15u] * wsc[u][2 * h + 1];
          d[h] = pack_bf16x2(a, b);
        }
        *reinterpret_cast<u32x4*>(sBs + (8 * kc + c) * LDK + 8 * rg) = u32x4{d[0], d[1], d[2], d[3]};
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  load_act<Cfg>(G, N, M, N, m0, 0, areg);
  load_w(0);
  __syncthreads();
  store_act<Cfg>(sA, areg);
  store_w(sB);
  __syncthreads();
  for (int64_t st = 0; st < nsteps; ++st) {
    const int cur = (int)(st & 1);
    const bool more = st + 1 < nsteps;
    if (more) {
      load_act<Cfg>(G, N, M, N, m0, (st + 1) * BK, areg);
      load_w((st + 1) * BK);
    }
    mma_step<Cfg, WM, WN, TM, TN>(sA + cur * BM * LDK, sB + cur * BN * LDK, acc);
    if (more) {
      store_act<Cfg>(sA + (cur ^ 1) * BM * LDK, areg);
      store_w(sB + (cur ^ 1) * BN * LDK);
    }
    __syncthreads();
  }

  // LoRA term: acc += (s v) A, r in steps of 16; A column k gathered
  {
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    for (int j0 = 0; j0 < r; j0 += 16) {
      const int jl = j0 + 8 * (lane >> 5);
      bf16x8 bh[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t k = min(k0 + wn * TN * 32 + j * 32 + (lane & 31), K - 1);
        uint32_t w4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jj = jl + 2 * q;
          const uint32_t lo = jj < r ? Al[(int64_t)jj * K + k] : 0u;
          const uint32_t hi = jj + 1 < r ? Al[(int64_t)(jj + 1) * K + k] : 0u;
          w4[q] = lo | (hi << 16);
        }
        bh[j] = as_bf16x8(u32x4{w4[0], w4[1], w4[2], w4[3]});
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t m = min(m0 + wm * TM * 32 + i * 32 + (lane & 31), M - 1);
        bf16x8 ah, al;
        lora_rows(Vv, m, r, jl, s, ah, al);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = mfma32(ah, bh[j], acc[i][j]);
          acc[i][j] = mfma32(al, bh[j], acc[i][j]);
        }
      }
    }
  }
  store_tile<WM, WN, TM, TN>(acc, dX, M, K, m0, k0);
}

template <class Kern>
hipError_t set_lds(Kern k, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int WM, int WN, int TM, int TN, int CB, bool ABS>
hipError_t run_fwd_f(const WState& w, const uint16_t* X, int64_t M, const float* u,
                     const uint16_t* B, int r, float s, uint16_t* Y, hipStream_t st) {
  using Cfg = Tile<WM, WN, TM, TN>;
  auto kern = k_qgemm_fwd<WM, WN, TM, TN, CB, ABS>;
  static hipError_t attr = set_lds(kern, Cfg::LDS);
  if (attr != hipSuccess) return attr;
  const int64_t tm = (M + Cfg::BM - 1) / Cfg::BM, tn = (w.rows + Cfg::BN - 1) / Cfg::BN;
  hipLaunchKernelGGL(kern, dim3((unsigned)(tm * tn)), dim3(Cfg::T), Cfg::LDS, st, w.packed,
                     w.qscale, w.scale2, w.offset, w.absmax, X, u, B, M, w.rows, w.cols, r, s, Y,
                     (int)tn);
  return hipGetLastError();
}

template <int WM, int WN, int TM, int TN, int CB, bool ABS>
hipError_t run_dx_f(const WState& w, const uint16_t* G, int64_t M, const float* v,
                    const uint16_t* A, int r, float s, uint16_t* dX, hipStream_t st) {
  using Cfg = Tile<WM, WN, TM, TN>;
  auto kern = k_qgemm_dx<WM, WN, TM, TN, CB, ABS>;
  static hipError_t attr = set_lds(kern, Cfg::LDS);
  if (attr != hipSuccess) return attr;
  const int64_t tm = (M + Cfg::BM - 1) / Cfg::BM, tk = (w.cols + Cfg::BN - 1) / Cfg::BN;
  hipLaunchKernelGGL(kern, dim3((unsigned)(tm * tk)), dim3(Cfg::T), Cfg::LDS, st, w.packed,
                     w.qscale, w.scale2, w.offset, w.absmax, G, v, A, M, w.rows, w.cols, r, s, dX,
                     (int)tk);
  return hipGetLastError();
}

// the state's format picks the instance
template <int WM, int WN, int TM, int TN>
hipError_t run_fwd(const WState& w, const uint16_t* X, int64_t M, const float* u,
                   const uint16_t* B, int r, float s, uint16_t* Y, hipStream_t st) {
  if (w.codebook == kCodeFP4)
    return w.absmax ? run_fwd_f<WM, WN, TM, TN, kCodeFP4, true>(w, X, M, u, B, r, s, Y, st)
                    : run_fwd_f<WM, WN, TM, TN, kCodeFP4, false>(w, X, M, u, B, r, s, Y, st);
  return w.absmax ? run_fwd_f<WM, WN, TM, TN, kCodeNF4, true>(w, X, M, u, B, r, s, Y, st)
                  : run_fwd_f<WM, WN, TM, TN, kCodeNF4, false>(w, X, M, u, B, r, s, Y, st);
}

template <int WM, int WN, int TM, int TN>
hipError_t run_dx(const WState& w, const uint16_t* G, int64_t M, const float* v,
                  const uint16_t* A, int r, float s, uint16_t* dX, hipStream_t st) {
  if (w.codebook == kCodeFP4)
    return w.absmax ? run_dx_f<WM, WN, TM, TN, kCodeFP4, true>(w, G, M, v, A, r, s, dX, st)
                    : run_dx_f<WM, WN, TM, TN, kCodeFP4, false>(w, G, M, v, A, r, s, dX, st);
  return w.absmax ? run_dx_f<WM, WN, TM, TN, kCodeNF4, true>(w, G, M, v, A, r, s, dX, st)
                  : run_dx_f<WM, WN, TM, TN, kCodeNF4, false>(w, G, M, v, A, r, s, dX, st);
}

// Tile choice: a 32-row tile for decode-sized batches, else 128x128 (larger
// batches go through the bf16 copy of the weight and the dense GEMM).
int pick(int64_t M) { return M <= 32 ? 0 : 1; }

}  // namespace

hipError_t launch_qgemm_fwd(const WState& w, const uint16_t* X, int64_t M, const float* u,
                            const uint16_t* B, int r, float s, uint16_t* Y, hipStream_t st) {
  if (w.codebook != kCodeNF4 && w.codebook != kCodeFP4) return hipErrorInvalidValue;
  if (pick(M) == 0) return run_fwd<1, 4, 1, 1>(w, X, M, u, B, r, s, Y, st);
  return run_fwd<2, 2, 2, 2>(w, X, M, u, B, r, s, Y, st);
}

hipError_t launch_qgemm_dx(const WState& w, const uint16_t* G, int64_t M, const float* v,
                           const uint16_t* A, int r, float s, uint16_t* dX, hipStream_t st) {
  if (w.codebook != kCodeNF4 && w.codebook != kCodeFP4) return hipErrorInvalidValue;
  if (pick(M) == 0) return run_dx<1, 4, 1, 1>(w, G, M, v, A, r, s, dX, st);
  return run_dx<2, 2, 2, 2>(w, G, M, v, A, r, s, dX, st);
}

}  // namespace qn
