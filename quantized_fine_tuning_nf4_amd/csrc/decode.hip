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
// CBK: the codebook (NF4 or FP4); ABS: double quantization off (the block
// scales read from absmax instead of decoded from qscale, scale2, offset).
template <int CBK, bool ABS>
__global__ __launch_bounds__(T, 4) void k_decode_partial(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ scale2, const float* __restrict__ offset,
    const float* __restrict__ absmax, const uint16_t* __restrict__ X, const uint16_t* __restrict__ Aad, int r, int64_t M,
    int64_t N, int64_t K, int nbs, float* __restrict__ part, float* __restrict__ upart) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t s_tab[256];
  __shared__ float s_e4m3[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  {  // pair table: entry b = bf16(L[b & 15]) | bf16(L[b >> 4]) << 16
    const float lo = as_f32(level_bits(CBK, tid & 15)), hi = as_f32(level_bits(CBK, tid >> 4));
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
  f32x4 a4[ABS ? CB / 4 : 1];  // double quantization off: the pass's block scales
  auto load_pass = [&](int jb) {
    const int64_t bb = b0 + jb;
#pragma unroll
    for (int j = 0; j < CB; ++j) code[j] = *reinterpret_cast<const uint2*>(crow + (bb + j) * 32);
    if constexpr (ABS) {
#pragma unroll
      for (int q = 0; q < CB / 4; ++q)
        a4[q] = *reinterpret_cast<const f32x4*>(absmax + n * kblocks + bb + 4 * q);
    } else {
      q4 = *reinterpret_cast<const u32x4*>(qscale + n * kblocks + bb);
      s2 = scale2[(n * kblocks + bb) / kGroup];
    }
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

  const float mu = ABS ? 0.f : *offset;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int jb = 0; jb < nbs; jb += CB) {
    if (jb > 0) load_pass(jb);
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const uint32_t qb = (q4[j >> 2] >> (8 * (j & 3))) & 0xffu;
      const float sc = ABS ? a4[j >> 2][j & 3] : __builtin_fmaf(s_e4m3[qb], s2, mu);
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

// ---------------------------------------------------------------------------
// One-kernel decode forward over tiles of (band of 16 RGT rows) x (slice of
// 1024 columns), one workgroup of 16 waves each:
//   - wave w owns block pair w % 8 of the slice and the band's row groups of
//     parity w / 8; its X and A fragments are loaded once;
//   - a unit of work is one 16-row group of the wave's block pair: 16 rows x
//     64 bytes of codes, which the wave itself moves into its own LDS ring by
//     one direct-to-LDS load (lane t: row t / 4, 16-byte chunk
//     (t % 4) ^ ((row / 2) % 4), so that the MFMA-layout reads below are
//     free of bank conflicts).  Each wave runs its own pipeline, NST - 1
//     units in flight, with no barrier in the main loop;
//   - lane (l16, g4) reads bytes 16 g4 .. +15 of row l16's block pair; two
//     v_permlane32_swap regroup the dwords so that each MFMA operand holds
//     one block (the per-block scale stays after the MFMA), koff1/koff2 give
//     the code positions each lane group carries;
//   - a code byte becomes its bf16 pair through a 256-entry LDS table in 32
//     copies (entry e of copy c at byte 256 e + 4 c, copy = lane % 32): the
//     32 lanes of a bank cycle never collide; v_perm_b32 forms the address;
//   - the waves' sums meet in LDS; the tile's partial y and its part of
//     u = X A^T go to the workspace through device-coherent stores; the last
//     tile of a band to arrive (an arrival counter per band) adds the slices
//     in slice order with device-coherent loads, adds s u B^T and writes bf16
//     y, so the result does not depend on the order of arrival.  The
//     counters live in the caller's workspace (zero before the call) and
//     are returned to zero by the tile that finishes the band.
constexpr int TT = 1024;
constexpr int NWV = TT / 64;       // waves
constexpr int NPR = 8;             // block pairs per slice
constexpr int KSL = 1024;          // columns per slice
constexpr int RGM = 16;            // row groups per band, at most
constexpr int RPW = RGM / 2;       // row groups per wave, at most
constexpr int NST = 5;             // ring slots per wave (NST - 1 units in flight)
constexpr int UB = 1024;           // bytes per unit: 16 rows x 64 B
constexpr int L_TAB = 0, L_RING = 65536, L_U = L_RING + NWV * NST * UB;
constexpr int L_URED = L_U + 16 * 17 * 4, L_QS = L_URED + NPR * 4 * 64 * 4;
constexpr int L_S2 = L_QS + RGM * 16 * 16, L_FLAG = L_S2 + RGM * 16 * 4;
constexpr int L_TOTAL = L_FLAG + 16;
constexpr int kMaxBands = kArrivalWords;  // one arrival counter per band
static_assert(NPR * RGM * 4 * 64 * 4 <= L_U, "reduction buffer overlaps");
static_assert(L_TOTAL <= 160 * 1024, "LDS");

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rs(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

__device__ __forceinline__ uint32_t tab_pair(const uint8_t* tab, uint32_t w, uint32_t base, int i) {
  // byte address 256 * (byte i of w) + base, base = 4 (lane % 32)
  const uint32_t a = __builtin_amdgcn_perm(w, base, 0x0c0c0000u | ((4u + (uint32_t)i) << 8));
  return *reinterpret_cast<const uint32_t*>(tab + a);
}
__device__ __forceinline__ bf16x8 tab_pairs4(const uint8_t* tab, uint32_t w, uint32_t base) {
  return as_bf16x8(u32x4{tab_pair(tab, w, base, 0), tab_pair(tab, w, base, 1),
                         tab_pair(tab, w, base, 2), tab_pair(tab, w, base, 3)});
}
// Device-coherent 16-byte store / load (cache policy sc1, the device
// scope): the access goes to the level shared by every XCD, never leaving a
// stale or dirty line in one XCD's L2, so no cache-wide write-back or
// invalidate is needed around it.
constexpr int kDeviceScope = 16;  // sc1
__device__ __forceinline__ void st_dev4(rsrc_t rs, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kDeviceScope);
}
__device__ __forceinline__ f32x4 ld_dev4(rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kDeviceScope));
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// CBK: the codebook of the codes (NF4 or FP4); ABS: double quantization off,
// the block scales read from absmax (fp32, into registers with the other
// small loads) instead of decoded from qscale, scale2 and offset.
template <int CBK, bool ABS>
__global__ __launch_bounds__(TT, 1) void k_decode_tile(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ scale2, const float* __restrict__ offset,
    const float* __restrict__ absmax, const uint16_t* __restrict__ X, int64_t M, int64_t N,
    int64_t K,
    const uint16_t* __restrict__ Aad, const uint16_t* __restrict__ Bad, int r, float s, int rgt,
    int S, unsigned* __restrict__ arrivals, float* __restrict__ part, float* __restrict__ upart,
    uint16_t* __restrict__ Y, float* __restrict__ u_out) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[L_TOTAL];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = wave & (NPR - 1), par = wave / NPR;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int band = blockIdx.x / S, z = blockIdx.x % S;
  const int BR = 16 * rgt;
  const int64_t n0 = (int64_t)band * BR;
  const int nrows = (int)min((int64_t)BR, N - n0);
  const int64_t kb = K / 64;
  const int64_t col0 = (int64_t)z * KSL + 128 * pr;  // first column of the wave's pair

  // ---- small loads first (their waits then never wait for the code stream)
  const float lo_level = as_f32(level_bits(CBK, (tid >> 5) & 15));
  const int koff1 = 32 * (g4 & 1) + ((g4 >> 1) ? 16 : 8);
  const int koff2 = 32 * (g4 & 1) + ((g4 >> 1) ? 24 : 0);
  // rows past M / r read the last valid row: finite values in outputs never stored
  const uint16_t* xrow = X + (int64_t)min(l16, (int)M - 1) * K + col0;
  const uint16_t* arow = Aad + (int64_t)min(l16, r - 1) * K + col0;
  bf16x8 xf[2][2], af[2][2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    xf[b][0] = as_bf16x8(*reinterpret_cast<const u32x4*>(xrow + 64 * b + koff1));
    xf[b][1] = as_bf16x8(*reinterpret_cast<const u32x4*>(xrow + 64 * b + koff2));
    af[b][0] = as_bf16x8(*reinterpret_cast<const u32x4*>(arow + 64 * b + koff1));
    af[b][1] = as_bf16x8(*reinterpret_cast<const u32x4*>(arow + 64 * b + koff2));
  }
  // the block scales of the wave's two blocks for row l16 of each of its
  // row groups (double quantization off: two fp32 values per row group;
  // rows past the band read its last row)
  float sca[RPW], scb[RPW];
  if constexpr (ABS) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = min(16 * (par + 2 * i) + l16, nrows - 1);
      const float2 ab = *reinterpret_cast<const float2*>(
          absmax + (n0 + row) * kb + (int64_t)z * (KSL / 64) + 2 * pr);
      sca[i] = ab.x;
      scb[i] = ab.y;
    }
  } else {
    // the band's scales for this slice, straight into LDS (direct-to-LDS
    // loads: nothing waits for them before the code stream is issued): the
    // 16 scale codes of each row (thread t: row t / 4, bytes 4 (t % 4) ..)
    // and each row's second-level scale (rows past the band read its last row)
    const int row = min(tid >> 2, nrows - 1);
    const rsrc_t rq = make_rs(qscale + n0 * kb + (int64_t)z * (KSL / 64),
                              (uint32_t)((int64_t)(nrows - 1) * kb + KSL / 64));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rq, (__attribute__((address_space(3))) void*)(smem + L_QS + 256 * wave), 4,
        (uint32_t)(row * kb + 4 * (tid & 3)), 0, 0, 0);
    if (wave < RGM * 16 / 64) {
      const rsrc_t r2 = make_rs(scale2, (uint32_t)((N * kb + kGroup - 1) / kGroup * 4));
      const int64_t b2 = (n0 + min(tid, nrows - 1)) * kb + (int64_t)z * (KSL / 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r2, (__attribute__((address_space(3))) void*)(smem + L_S2 + 256 * wave), 4,
          (uint32_t)(b2 / kGroup * 4), 0, 0, 0);
    }
  }

  // ---- the wave's code stream: unit i = row group par + 2 i.  The
  // descriptor of a unit starts at its first row and ends at the band's end,
  // so rows past the band (and units past the last) read zeros without
  // touching memory; the lane offset is fixed.
  const int drow = lane >> 2;
  const uint32_t voff = (uint32_t)drow * (uint32_t)(K / 2) + (uint32_t)z * (KSL / 2) +
                        64u * (uint32_t)pr + 16u * (uint32_t)((lane & 3) ^ ((drow >> 1) & 3));
  uint8_t* ring = smem + L_RING + wave * NST * UB;
  auto dma_unit = [&](int i) {
    const int rg = par + 2 * i;
    const int64_t left = max((int64_t)0, (int64_t)nrows - 16 * rg);
    const rsrc_t rs = make_rs(packed + (n0 + min((int64_t)16 * rg, (int64_t)nrows)) * (K / 2),
                              (uint32_t)(left * (K / 2)));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(ring + (i % NST) * UB), 16, voff, 0, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) dma_unit(i);

  // ---- tables (while the loads are in flight): thread tid fills copy
  // tid % 32 of the entries with low nibble tid / 32 % 16 and high nibble
  // hi = tid / 512 (mod 2); hi is a constant in each branch, so the levels
  // are immediates (no loads that would wait behind the code stream)
  static_assert(TT == 1024, "table fill assumes 1024 threads");
  uint32_t* tab32 = reinterpret_cast<uint32_t*>(smem + L_TAB);
  const int hi_par = __builtin_amdgcn_readfirstlane(tid >> 9);  // wave-uniform
  uint32_t* trow = tab32 + ((tid >> 5) & 15) * 64 + (tid & 31);
#pragma unroll
  for (int hi = 0; hi < 16; ++hi)
    if ((hi & 1) == hi_par) trow[hi * 16 * 64] = pack_bf16x2(lo_level, as_f32(level_bits(CBK, hi)));
  // tables and scales ready (everything but the NST - 1 code units in
  // flight has landed); the code stream stays in flight across the barrier
  wait_vm<NST - 1>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const uint8_t* tab = smem + L_TAB;
  const uint32_t tbase = 4u * (lane & 31);
  const int rd = 16 * (4 * l16 + (g4 ^ ((l16 >> 1) & 3)));  // this lane's chunk in a unit
  if constexpr (!ABS) {
    // the block scales, once: s'_b = fma(e4m3(q_b), s2, mu)
    const float mu = *offset;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = 16 * (par + 2 * i) + l16;
      const uint32_t qs = *reinterpret_cast<const uint16_t*>(smem + L_QS + 16 * row + 2 * pr);
      const float s2 = reinterpret_cast<const float*>(smem + L_S2)[row];
      sca[i] = dq_scale(qs & 0xffu, s2, mu);
      scb[i] = dq_scale((qs >> 8) & 0xffu, s2, mu);
    }
  }

  f32x4 acc[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    if (par + 2 * i >= rgt) continue;
    wait_vm<NST - 2>();  // unit i landed; units i + 1 .. i + NST - 2 still fly
    const u32x4 c = *reinterpret_cast<const u32x4*>(ring + (i % NST) * UB + rd);
    // unit i + NST - 1 goes into the slot of unit i - 1, whose read is done
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    dma_unit(i + NST - 1);
    const auto h = __builtin_amdgcn_permlane32_swap(c[1], c[2], false, false);
    const auto l = __builtin_amdgcn_permlane32_swap(c[0], c[3], false, false);
    const float sa = sca[i], sb = scb[i];
    f32x4 t = mfma16(xf[0][0], tab_pairs4(tab, h[0], tbase), f32x4{0.f, 0.f, 0.f, 0.f});
    t = mfma16(xf[0][1], tab_pairs4(tab, l[0], tbase), t);
    f32x4 t2 = mfma16(xf[1][0], tab_pairs4(tab, h[1], tbase), f32x4{0.f, 0.f, 0.f, 0.f});
    t2 = mfma16(xf[1][1], tab_pairs4(tab, l[1], tbase), t2);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[i][v] = __builtin_fmaf(sa, t[v], acc[i][v]);
      acc[i][v] = __builtin_fmaf(sb, t2[v], acc[i][v]);
    }
  }
  f32x4 uacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    uacc = mfma16(xf[b][0], af[b][0], uacc);
    uacc = mfma16(xf[b][1], af[b][1], uacc);
  }
  wait_vm<0>();  // the trailing unit loads land before their LDS is reused

  // ---- the waves' sums: lane (l16, g4) slot v holds row 16 rg + l16, m = 4 g4 + v
  __syncthreads();
  float* s_red = reinterpret_cast<float*>(smem);            // [pair][rg][v][lane]
  float* s_ured = reinterpret_cast<float*>(smem + L_URED);  // [pair][v][lane]
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int rg = par + 2 * i;
    if (rg < rgt)
#pragma unroll
      for (int v = 0; v < 4; ++v) s_red[((pr * RGM + rg) * 4 + v) * 64 + lane] = acc[i][v];
  }
  if (par == 0)
#pragma unroll
    for (int v = 0; v < 4; ++v) s_ured[(pr * 4 + v) * 64 + lane] = uacc[v];
  __syncthreads();
  // partial sums of this tile: thread (m = tid / 64, rows 4 (tid % 64) ..
  // + 3), one 16-byte store; part rows are Np = N rounded up to 4 long
  const int64_t Np = (N + 3) & ~(int64_t)3;
  const rsrc_t rpart = make_rs(part, (uint32_t)((int64_t)S * M * Np * 4));
  const rsrc_t rupart = make_rs(upart, (uint32_t)((int64_t)gridDim.x * 256 * 4));
  const int om = tid >> 6, orow = 4 * (tid & 63);
  if (om < M && orow < nrows) {
    const f32x4* red4 = reinterpret_cast<const f32x4*>(s_red);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NPR; ++p)
      a += red4[(((p * RGM + (orow >> 4)) * 4 + (om & 3)) * 64 + (orow & 15) + 16 * (om >> 2)) / 4];
    st_dev4(rpart, (uint32_t)((((int64_t)z * M + om) * Np + n0 + orow) * 4), a);
  }
  if (tid < 64) {
    // u partial: [m][j] for m = tid / 4, j = 4 (tid % 4) .. + 3
    const int m = tid >> 2, j = 4 * (tid & 3);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NPR; ++p)
      a += *reinterpret_cast<const f32x4*>(s_ured + (p * 4 + (m & 3)) * 64 + j + 16 * (m >> 2));
    st_dev4(rupart, (uint32_t)((((int64_t)band * S + z) * 256 + 16 * m + j) * 4), a);
  }

  // ---- arrival; the last tile of the band finishes it.  Every wave's
  // device-coherent stores have completed (vmcnt(0)) before the barrier, so
  // they precede the arrival; the finishing tile reads them with
  // device-coherent loads after it has seen all S arrivals.
  wait_vm<0>();
  __syncthreads();
  int* s_flag = reinterpret_cast<int*>(smem + L_FLAG);
  if (tid == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(arrivals + band, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag[0] = old == (unsigned)(S - 1);
  }
  __syncthreads();
  if (!s_flag[0]) return;
  // ---- finishing the band: every load goes out before the first is used
  // (the band's B rows into LDS, the u partials, this thread's S partial
  // sums), then the sums run in slice order
  // B of the band, transposed into LDS (the ring is free): s_bt[j][row],
  // row pitch BTP, zero for j >= r; a thread later reads four consecutive
  // rows of one j at once
  constexpr int BTP = RGM * 16 + 8;
  uint16_t* s_bt = reinterpret_cast<uint16_t*>(smem + L_RING);
  for (int e = tid; e < BR * 16; e += TT) {
    const int row = e >> 4, j = e & 15;
    const int64_t n = n0 + min(row, nrows - 1);
    s_bt[j * BTP + row] = j < r ? Bad[n * r + min(j, r - 1)] : (uint16_t)0;
  }
  float* s_u = reinterpret_cast<float*>(smem + L_U);  // [16][17]
  f32x4 ua = {0.f, 0.f, 0.f, 0.f}, ya = {0.f, 0.f, 0.f, 0.f};
  const bool yok = om < M && orow < nrows;
  for (int z0 = 0; z0 < S; z0 += 4) {
    f32x4 uv[4], yv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int zz = z0 + q;
      uv[q] = (zz < S && tid < 64)
                  ? ld_dev4(rupart, (uint32_t)((((int64_t)band * S + zz) * 256 + 4 * tid) * 4))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
      yv[q] = (zz < S && yok)
                  ? ld_dev4(rpart, (uint32_t)((((int64_t)zz * M + om) * Np + n0 + orow) * 4))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (z0 + q < S) {
        ua += uv[q];
        ya += yv[q];
      }
  }
  if (tid < 64) {
    // u[m][j], m = tid / 4, j = 4 (tid % 4) + q, summed in slice order
    const int m = tid >> 2, j0 = 4 * (tid & 3);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s_u[m * 17 + j0 + q] = ua[q];
      if (band == 0 && m < M && j0 + q < r) u_out[m * r + j0 + q] = ua[q];
    }
  }
  if (tid == 0)  // every tile of the band has arrived: ready for the next call
    __hip_atomic_store(arrivals + band, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();  // s_u, s_bt
  if (yok) {
    float lora[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const u32x2 b4 = *reinterpret_cast<const u32x2*>(s_bt + j * BTP + orow);
      const float uj = s_u[om * 17 + j];
      lora[0] = __builtin_fmaf(uj, bf16_lo(b4[0]), lora[0]);
      lora[1] = __builtin_fmaf(uj, bf16_hi(b4[0]), lora[1]);
      lora[2] = __builtin_fmaf(uj, bf16_lo(b4[1]), lora[2]);
      lora[3] = __builtin_fmaf(uj, bf16_hi(b4[1]), lora[3]);
    }
    uint16_t yo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      yo[q] = (uint16_t)(pack_bf16x2(__builtin_fmaf(s, lora[q], ya[q]), 0.f) & 0xffffu);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (orow + q < nrows) Y[om * N + n0 + orow + q] = yo[q];
  }
}

// ---------------------------------------------------------------------------
// Whole-row decode forward (cols = 1024 PW, M <= 16, r <= 16): workgroup b
// owns rows BR b .. BR b + BR - 1 (BR <= 64, at most four 16-row groups) and
// every column, so each output is finished inside one workgroup: no partial
// sums leave it and no workgroup waits for another.  Every workgroup forms
// u = X A^T itself (A is r x cols bf16, read from L2 once the first
// workgroups of an XCD have brought it in).  Eight waves (256 registers per
// lane: the X and A fragments of a wave's columns stay in registers):
//   - wave w owns block pairs w + 8 i (i < PW); a unit is one 16-row group
//     of one of its pairs (16 rows x 64 B of codes), moved into the wave's
//     LDS ring by one direct-to-LDS load in the layout of the sliced kernel
//     above (same lane mapping, table and MFMA form);
//   - order of issue, which is the order of completion: the band's scale
//     codes, second-level scales and B rows (plain loads, written to LDS
//     before the first barrier), X fragments, the first RS code units; the
//     remaining units refill the ring slot of the unit consumed RS steps
//     earlier.  The wait for unit q counts the operations issued after it, a
//     compile-time number.  The A fragments (for u) go out right after the
//     last refill, so that they neither hold the code stream back nor add
//     their latency after the last unit;
//   - after the main loop the waves' sums meet in LDS (sum over waves in wave
//     order), u likewise; thread (m, row) adds s sum_j u[m][j] B[row][j] and
//     stores bf16 y.  Workgroup 0 writes u.
constexpr int RW_RG = 4;           // row groups per band
constexpr int RW_BR = 16 * RW_RG;  // rows per band, at most
// ring: 64 units of 1 KB split among the waves (16 waves: 4 in flight each of
// 8; 5 measured 0.2-1 us slower per call, 3 the same, 2 slower: more requests
// at once delay the first data)
constexpr int RW_RING_KB = 64;
constexpr int RW_TAB = 0, RW_RING = 65536, RW_QS = RW_RING + RW_RING_KB * UB;
constexpr int RW_S2 = RW_QS + RW_BR * 64, RW_B = RW_S2 + 64 * 4, RW_E4 = RW_B + RW_BR * 16 * 2;
constexpr int RW_TOTAL = RW_E4 + 256 * 4;
// double quantization off: the band's fp32 block scales, after the rest
constexpr int RW_AB = RW_TOTAL, RW_TOTAL_ABS = RW_AB + RW_BR * 64 * 4;
static_assert(RW_TOTAL_ABS <= 160 * 1024, "LDS");
static_assert(16 * RW_RG * 4 * 64 * 4 <= RW_RING, "wave sums overlap the ring");

// operations issued after unit q of NU when it is awaited: RS units go out
// first, then NA other loads; unit RS + k is issued after unit k is read
template <int NU, int RS, int NA>
constexpr int rw_after(int q) {
  return q < RS ? (RS - 1 - q) + NA + (q < NU - RS ? q : (NU - RS > 0 ? NU - RS : 0))
                : ((q - 1 < NU - RS - 1 ? q - 1 : NU - RS - 1) - q + RS);
}

// s_waitcnt vmcnt(n) for a count known after unrolling (0 past 39)
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
#define QN_W1(k) \
  case k:        \
    wait_vm<k>(); \
    break;
#define QN_W10(t) QN_W1(t##0) QN_W1(t##1) QN_W1(t##2) QN_W1(t##3) QN_W1(t##4) \
                  QN_W1(t##5) QN_W1(t##6) QN_W1(t##7) QN_W1(t##8) QN_W1(t##9)
    QN_W1(1) QN_W1(2) QN_W1(3) QN_W1(4) QN_W1(5) QN_W1(6) QN_W1(7) QN_W1(8) QN_W1(9)
    QN_W10(1) QN_W10(2) QN_W10(3)
#undef QN_W10
#undef QN_W1
    default:
      wait_vm<0>();
  }
}

// CBK: the codebook of the codes (NF4 or FP4); ABS: double quantization off,
// the block scales read from absmax (fp32) instead of decoded from qscale,
// scale2 and offset.
template <int PW, int NW, int CBK, bool ABS>
__global__ __launch_bounds__(64 * NW, 1) void k_decode_rows(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ scale2, const float* __restrict__ offset,
    const float* __restrict__ absmax, const uint16_t* __restrict__ X, int64_t M, int64_t N,
    const uint16_t* __restrict__ Aad, const uint16_t* __restrict__ Bad, int r, float s, int br,
    uint16_t* __restrict__ Y, float* __restrict__ u_out) {
  constexpr int RW_T = 64 * NW, RW_W = NW;
  constexpr int64_t K = 128 * NW * PW, kb = K / 64;
  constexpr int NU = RW_RG * PW, RS = NU < RW_RING_KB / NW ? NU : RW_RING_KB / NW, NA = 0;
  constexpr int PT = (RW_BR * 16 + RW_T - 1) / RW_T;  // small-load elements per thread
  static_assert(rw_after<NU, RS, NA>(0) <= 39, "wait counts");
  __shared__ __attribute__((aligned(16))) uint8_t smem[ABS ? RW_TOTAL_ABS : RW_TOTAL];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * br;
  const int nrows = (int)min((int64_t)br, N - n0);

  // ---- the band's scale codes (nrows * kb bytes), second-level scales and
  // B rows: PT dwords / PT elements per thread (or, double quantization off,
  // its fp32 block scales: PA per thread)
  constexpr int QW = RW_BR * (int)kb / 4;  // dwords of scale codes, at most
  static_assert(QW <= PT * RW_T && RW_BR * 16 <= PT * RW_T, "PT per thread");
  constexpr int PA = (RW_BR * (int)kb + RW_T - 1) / RW_T;
  const int64_t g0 = n0 * kb / kGroup;
  const int ns2 = (int)(((n0 + nrows) * kb - 1) / kGroup - g0 + 1);
  const int nq = nrows * (int)kb / 4, nb = nrows * r, na = nrows * (int)kb;
  uint32_t qv[PT];
  uint16_t bv[PT];
  float av[ABS ? PA : 1];
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int e = tid + RW_T * k;
    if constexpr (!ABS) qv[k] = e < nq ? reinterpret_cast<const uint32_t*>(qscale + n0 * kb)[e] : 0u;
    bv[k] = e < nb ? Bad[n0 * r + e] : (uint16_t)0;
  }
  if constexpr (ABS) {
#pragma unroll
    for (int k = 0; k < PA; ++k) {
      const int e = tid + RW_T * k;
      av[k] = e < na ? absmax[n0 * kb + e] : 0.f;
    }
  }
  const float s2v = !ABS && tid < ns2 ? scale2[g0 + tid] : 0.f;
  // level of the low nibble tid / 32 % 16 = 2 (wave % 8) + bit 5 of the
  // lane: a wave-uniform index (scalar loads, never queued behind the code
  // stream) and a select
  const int lsel = 2 * (wave & 7);
  const float lo_level = as_f32((lane & 32) ? level_bits(CBK, lsel + 1) : level_bits(CBK, lsel));

  // ---- X fragments of the wave's pairs (rows past M read the last row)
  const int koff1 = 32 * (g4 & 1) + ((g4 >> 1) ? 16 : 8);
  const int koff2 = 32 * (g4 & 1) + ((g4 >> 1) ? 24 : 0);
  const uint16_t* xrow = X + (int64_t)min(l16, (int)M - 1) * K + 128 * wave;
  const uint16_t* arow = Aad + (int64_t)min(l16, r - 1) * K + 128 * wave;
  constexpr int PS = 128 * NW;  // columns between a wave's pairs
  bf16x8 xf[PW][2][2], af[PW][2][2];
#pragma unroll
  for (int i = 0; i < PW; ++i)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      xf[i][b][0] = as_bf16x8(*reinterpret_cast<const u32x4*>(xrow + PS * i + 64 * b + koff1));
      xf[i][b][1] = as_bf16x8(*reinterpret_cast<const u32x4*>(xrow + PS * i + 64 * b + koff2));
    }

  // ---- the code stream: unit q = (row group q / PW, pair q % PW); rows past
  // the band read zeros without touching memory
  const int drow = lane >> 2;
  const uint32_t voff = (uint32_t)drow * (uint32_t)(K / 2) + 64u * (uint32_t)wave +
                        16u * (uint32_t)((lane & 3) ^ ((drow >> 1) & 3));
  uint8_t* ring = smem + RW_RING + wave * RS * UB;
  auto dma_unit = [&](int q) {
    const int rg = q / PW, i = q % PW;
    const int64_t left = max((int64_t)0, (int64_t)nrows - 16 * rg);
    const rsrc_t rs = make_rs(packed + (n0 + min((int64_t)16 * rg, (int64_t)nrows)) * (K / 2),
                              (uint32_t)(left * (K / 2)));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(ring + (q % RS) * UB), 16,
        voff + 64u * NW * (uint32_t)i, 0, 0, 0);
  };
#pragma unroll
  for (int q = 0; q < RS; ++q) dma_unit(q);
  // ---- table (levels as immediates; entry e of copy c at byte 256 e + 4 c),
  // scales and B into LDS
  {
    // thread tid: copy tid % 32, low nibble tid / 32 % 16, the high nibbles
    // hi with hi % HS == tid / 512 (HS = threads / 512; wave-uniform)
    constexpr int HS = RW_T / 512;
    static_assert(HS >= 1 && RW_T % 512 == 0, "table fill");
    const int hsel = __builtin_amdgcn_readfirstlane(tid >> 9);
    uint32_t* trow = reinterpret_cast<uint32_t*>(smem + RW_TAB) + ((tid >> 5) & 15) * 64 + (tid & 31);
#pragma unroll
    for (int hi = 0; hi < 16; ++hi)
      if (HS == 1 || hi % HS == hsel)
        trow[hi * 16 * 64] = pack_bf16x2(lo_level, as_f32(level_bits(CBK, hi)));
  }
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    if constexpr (!ABS) reinterpret_cast<uint32_t*>(smem + RW_QS)[tid + RW_T * k] = qv[k];
    reinterpret_cast<uint16_t*>(smem + RW_B)[tid + RW_T * k] = bv[k];
  }
  if constexpr (ABS) {
#pragma unroll
    for (int k = 0; k < PA; ++k)
      if (tid + RW_T * k < RW_BR * (int)kb) reinterpret_cast<float*>(smem + RW_AB)[tid + RW_T * k] = av[k];
  } else {
    if (tid < 64) reinterpret_cast<float*>(smem + RW_S2)[tid] = s2v;
    // scale code -> value (a table keeps the main loop free of branches)
    if (tid < 256) reinterpret_cast<float*>(smem + RW_E4)[tid] = e4m3_to_f32(tid);
  }
  wait_vm_n(RS + NA);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  const uint8_t* tab = smem + RW_TAB;
  const uint32_t tbase = 4u * (lane & 31);
  const float mu = ABS ? 0.f : *offset;
  const int rd = 16 * (4 * l16 + (g4 ^ ((l16 >> 1) & 3)));
  f32x4 acc[RW_RG];
#pragma unroll
  for (int g = 0; g < RW_RG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < NU; ++q) {
    const int g = q / PW, i = q % PW;
    // unit q has landed (units after the last refill also count the A loads)
    wait_vm_n(rw_after<NU, RS, NA>(q) + (NU > RS && q > NU - RS - 1 ? 4 * PW : 0));
    const u32x4 c = *reinterpret_cast<const u32x4*>(ring + (q % RS) * UB + rd);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (q + RS < NU) dma_unit(q + RS);  // into the slot just read
    if (NU > RS && q == NU - RS - 1) {
      // after the last refill: the A fragments (for u; issued before the
      // refills, their 128 KB per workgroup from L2 held the code stream
      // back; after the last unit, their latency came after it)
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < PW; ++i)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          af[i][b][0] = as_bf16x8(*reinterpret_cast<const u32x4*>(arow + PS * i + 64 * b + koff1));
          af[i][b][1] = as_bf16x8(*reinterpret_cast<const u32x4*>(arow + PS * i + 64 * b + koff2));
        }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
    }
    // block scales of row l16 of group g for the pair's two blocks (rows
    // past the band use its last row: finite, never stored)
    const int row = min(16 * g + l16, nrows - 1);
    const int blk = 2 * (wave + NW * i);
    float sa, sb;
    if constexpr (ABS) {
      const float2 ab = *reinterpret_cast<const float2*>(smem + RW_AB + 4 * (row * kb + blk));
      sa = ab.x;
      sb = ab.y;
    } else {
      const uint32_t qs = *reinterpret_cast<const uint16_t*>(smem + RW_QS + row * kb + blk);
      const float s2 =
          reinterpret_cast<const float*>(smem + RW_S2)[((n0 + row) * kb + blk) / kGroup - g0];
      const float* e4 = reinterpret_cast<const float*>(smem + RW_E4);
      sa = __builtin_fmaf(e4[qs & 0xffu], s2, mu);  // = dq_scale
      sb = __builtin_fmaf(e4[(qs >> 8) & 0xffu], s2, mu);
    }
    const auto h = __builtin_amdgcn_permlane32_swap(c[1], c[2], false, false);
    const auto l = __builtin_amdgcn_permlane32_swap(c[0], c[3], false, false);
    f32x4 t = mfma16(xf[i][0][0], tab_pairs4(tab, h[0], tbase), f32x4{0.f, 0.f, 0.f, 0.f});
    t = mfma16(xf[i][0][1], tab_pairs4(tab, l[0], tbase), t);
    f32x4 t2 = mfma16(xf[i][1][0], tab_pairs4(tab, h[1], tbase), f32x4{0.f, 0.f, 0.f, 0.f});
    t2 = mfma16(xf[i][1][1], tab_pairs4(tab, l[1], tbase), t2);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc[g][v] = __builtin_fmaf(sa, t[v], acc[g][v]);
      acc[g][v] = __builtin_fmaf(sb, t2[v], acc[g][v]);
    }
    // one unit at a time: later units' table reads are not hoisted into this
    // one (their registers would be live across it)
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (NU <= RS) {  // no refills: the A fragments after the last unit
#pragma unroll
    for (int i = 0; i < PW; ++i)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        af[i][b][0] = as_bf16x8(*reinterpret_cast<const u32x4*>(arow + PS * i + 64 * b + koff1));
        af[i][b][1] = as_bf16x8(*reinterpret_cast<const u32x4*>(arow + PS * i + 64 * b + koff2));
      }
  }
  f32x4 uacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < PW; ++i)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      uacc = mfma16(xf[i][b][0], af[i][b][0], uacc);
      uacc = mfma16(xf[i][b][1], af[i][b][1], uacc);
    }

  // ---- the waves' sums: lane (l16, g4) slot v holds row 16 g + l16,
  // m = 4 g4 + v (and u[m][j = l16])
  __syncthreads();  // every wave is done with the table and its ring
  float* s_red = reinterpret_cast<float*>(smem + RW_TAB);   // [wave][g][v][lane]
  float* s_ured = reinterpret_cast<float*>(smem + RW_RING); // [wave][v][lane]
  float* s_u = s_ured + RW_W * 4 * 64;                       // [m][17]
#pragma unroll
  for (int g = 0; g < RW_RG; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) s_red[((wave * RW_RG + g) * 4 + v) * 64 + lane] = acc[g][v];
#pragma unroll
  for (int v = 0; v < 4; ++v) s_ured[(wave * 4 + v) * 64 + lane] = uacc[v];
  __syncthreads();
  if (tid < 256) {
    const int m = tid >> 4, j = tid & 15;
    const int slot = ((m & 3) * 64) + j + 16 * (m >> 2);
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < RW_W; ++w) a += s_ured[w * 4 * 64 + slot];
    s_u[m * 17 + j] = a;
    if (blockIdx.x == 0 && m < M && j < r) u_out[m * r + j] = a;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < (1024 + RW_T - 1) / RW_T; ++k) {
    const int o = tid + RW_T * k, om = o >> 6, orow = o & 63;
    if (om < M && orow < nrows) {
      const int slot = ((orow >> 4) * 4 + (om & 3)) * 64 + (orow & 15) + 16 * (om >> 2);
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < RW_W; ++w) a += s_red[w * RW_RG * 4 * 64 + slot];
      const uint16_t* sb = reinterpret_cast<const uint16_t*>(smem + RW_B) + orow * r;
      float lora = 0.f;
      for (int j = 0; j < r; ++j) lora = __builtin_fmaf(s_u[om * 17 + j], bf16_lo(sb[j]), lora);
      Y[om * N + n0 + orow] = (uint16_t)(pack_bf16x2(__builtin_fmaf(s, lora, a), 0.f) & 0xffffu);
    }
  }
}

}  // namespace

int decode_slices(int64_t M, int64_t N, int64_t K) {
  // one slice per 16 blocks (1024 columns) of the weight
  (void)N;
  if (M < 1 || M > 16 || K % 1024 != 0) return 0;
  return (int)(K / 1024);
}

DecodeTiles decode_tiles(int64_t M, int64_t N, int64_t K, int r) {
  DecodeTiles t{0, 0, 0};
  if (M < 1 || M > 16 || r < 1 || r > 16 || N < 1 || K < KSL || K % KSL != 0) return t;
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return n;
  }();
  if (cus <= 0) return t;
  const int64_t S = K / KSL, groups = (N + 15) / 16;
  const int64_t per_slice = max((int64_t)1, (int64_t)cus / S);
  const int64_t rgt = min((int64_t)RGM, (groups + per_slice - 1) / per_slice);
  const int64_t bands = (N + 16 * rgt - 1) / (16 * rgt);
  if (bands > kMaxBands || bands * S > (int64_t)1 << 30) return t;
  t.rgt = (int)rgt;
  t.S = (int)S;
  t.bands = (int)bands;
  return t;
}

hipError_t launch_decode_tile(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                              const DecodeTiles& t, unsigned* arrivals, float* part,
                              float* upart, hipStream_t st) {
  const int64_t N = w.rows, K = w.cols;
  if (t.rgt < 1 || t.rgt > RGM || t.S != K / KSL || t.bands < 1 || t.bands > kMaxBands ||
      (int64_t)t.bands * 16 * t.rgt < N || M < 1 || M > 16 || r < 1 || r > 16 || !arrivals)
    return hipErrorInvalidValue;
  if (w.codebook != kCodeNF4 && w.codebook != kCodeFP4) return hipErrorInvalidValue;
#define QN_TILE(CBK, ABS)                                                                       \
  hipLaunchKernelGGL((k_decode_tile<CBK, ABS>), dim3((unsigned)(t.bands * t.S)), dim3(TT), 0, st, \
                     w.packed, w.qscale, w.scale2, w.offset, w.absmax, X, M, N, K, A, B, r, s,   \
                     t.rgt, t.S, arrivals, part, upart, Y, u_out)
  if (w.codebook == kCodeFP4) {
    if (w.absmax) QN_TILE(kCodeFP4, true); else QN_TILE(kCodeFP4, false);
  } else {
    if (w.absmax) QN_TILE(kCodeNF4, true); else QN_TILE(kCodeNF4, false);
  }
#undef QN_TILE
  return hipGetLastError();
}

constexpr int kRowsWaves = 16;  // waves per workgroup of k_decode_rows

int decode_rows_band(int64_t M, int64_t N, int64_t K, int r) {
  if (M < 1 || M > 16 || r < 1 || r > 16 || N < 1 || (K != 2048 && K != 4096)) return 0;
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return n;
  }();
  if (cus <= 0) return 0;
  // one band per compute unit, a multiple of 8 rows; below 33 rows a band's
  // share of A (r x cols, read by every workgroup) outweighs its codes, and
  // the sliced kernel serves better
  const int64_t br = 8 * ((N + 8 * (int64_t)cus - 1) / (8 * (int64_t)cus));
  if (br <= 32) return 0;
  return (int)min(br, (int64_t)RW_BR);
}

hipError_t launch_decode_rows(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                              int br, hipStream_t st) {
  const int64_t N = w.rows, K = w.cols;
  if (br < 8 || br > RW_BR || br % 8 != 0 || M < 1 || M > 16 || r < 1 || r > 16 ||
      (K != 2048 && K != 4096))
    return hipErrorInvalidValue;
  if (w.codebook != kCodeNF4 && w.codebook != kCodeFP4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + br - 1) / br));
  constexpr int NW = kRowsWaves;
#define QN_ROWS(KC, CBK, ABS)                                                                    \
  hipLaunchKernelGGL((k_decode_rows<KC / (128 * NW), NW, CBK, ABS>), grid, dim3(64 * NW), 0, st, \
                     w.packed, w.qscale, w.scale2, w.offset, w.absmax, X, M, N, A, B, r, s, br,   \
                     Y, u_out)
#define QN_ROWS_K(CBK, ABS)      \
  if (K == 4096)                \
    QN_ROWS(4096, CBK, ABS);     \
  else                          \
    QN_ROWS(2048, CBK, ABS)
  if (w.codebook == kCodeFP4) {
    if (w.absmax) { QN_ROWS_K(kCodeFP4, true); } else { QN_ROWS_K(kCodeFP4, false); }
  } else {
    if (w.absmax) { QN_ROWS_K(kCodeNF4, true); } else { QN_ROWS_K(kCodeNF4, false); }
  }
#undef QN_ROWS_K
#undef QN_ROWS
  return hipGetLastError();
}

hipError_t launch_decode_fwd(const WState& w, const uint16_t* X, int64_t M, const uint16_t* A,
                             const uint16_t* B, int r, float s, uint16_t* Y, float* u_out,
                             float* part, float* upart, int S, hipStream_t st) {
  if (w.codebook != kCodeNF4 && w.codebook != kCodeFP4) return hipErrorInvalidValue;
  const int64_t N = w.rows, K = w.cols;
  const int nbs = (int)(K / 64 / S);
  const size_t lds = (size_t)M * (nbs * 128 + 16);
  constexpr size_t kMaxLds = 64 * 1024;  // X slice: at most 16 rows of 16 blocks
  static hipError_t attr = [] {
    const void* k[4] = {reinterpret_cast<const void*>(k_decode_partial<kCodeNF4, false>),
                        reinterpret_cast<const void*>(k_decode_partial<kCodeNF4, true>),
                        reinterpret_cast<const void*>(k_decode_partial<kCodeFP4, false>),
                        reinterpret_cast<const void*>(k_decode_partial<kCodeFP4, true>)};
    for (const void* f : k) {
      const hipError_t e =
          hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  if (nbs != 16 || lds > kMaxLds) return hipErrorInvalidValue;
  const int64_t groups = (N + 63) / 64;
  const dim3 grid((unsigned)(groups + 1), (unsigned)S);
#define QN_PART(CBK, ABS)                                                                      \
  hipLaunchKernelGGL((k_decode_partial<CBK, ABS>), grid, dim3(T), lds, st, w.packed, w.qscale, \
                     w.scale2, w.offset, w.absmax, X, A, r, M, N, K, nbs, part, upart)
  if (w.codebook == kCodeFP4) {
    if (w.absmax) QN_PART(kCodeFP4, true); else QN_PART(kCodeFP4, false);
  } else {
    if (w.absmax) QN_PART(kCodeNF4, true); else QN_PART(kCodeNF4, false);
  }
#undef QN_PART
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_finish, dim3((unsigned)((N + T - 1) / T), (unsigned)M), dim3(T), 0,
                     st, part,
                     upart, S, M, N, B, r, s, Y, u_out);
  return hipGetLastError();
}

}  // namespace qn
