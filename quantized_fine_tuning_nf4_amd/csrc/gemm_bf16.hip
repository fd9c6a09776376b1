// bf16 GEMM with the LoRA term fused in the epilogue, for large batches:
//
//   C[M, Nc] (bf16) = A[M, R] Bm[Nc, R]^T + s V[M, r] L[Nc, r]^T
//
// used for the forward (A = x, Bm = Qhat(W) [N, K], V = u, L = B) and for
// dX (A = dY, Bm = Qhat(W)^T [K, N], V = v, L = A^T) of the page "QLoRA: NF4
// storage, gradients and local integration" (paragraph after the teaching
// listing), once the weight has been dequantized to bf16 in a workspace.
//
// Workgroup tile 256 x 256, four waves (2 x 2), each wave 128 x 128 as 8 x 8
// tiles of v_mfma_f32_16x16x32_bf16 (256 accumulators, pinned in AGPRs).  On
// gfx950 this shape keeps a higher shader clock under load than the 32x32x16
// one at the same issue rate.  A step covers 64 reduction elements: both
// operands go from global memory straight into LDS by buffer loads, each
// load instruction filling eight whole 128-byte rows (one cache line per row
// and step), two stages deep.  A step is multiplied in two halves of 32; the
// fragments of the next half are read from LDS while the current half's
// MFMAs run (A in place, B in a second set).  The loads of step s+2 go out
// during the second half of step s into step s's stage, whose last fragments
// were read during its first half; the end of the first half of step s+1
// waits for them.  Chunk c (16 bytes) of LDS row y sits at unit
// c ^ ((y >> 1) & 7), which keeps the sixteen rows of one fragment read on
// distinct banks.  Rows of A past its length R are moved back onto its last
// chunk; Bm is zero there (its rows are padded to a multiple of 64 with
// zeros).
#include <type_traits>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NST = 2, T = 256;
constexpr int ROWB = BK * 2;            // bytes per tile row per stage (one cache line)
constexpr int OPB = 256 * ROWB;         // bytes per operand per stage (32 KB)
constexpr int STB = 2 * OPB;            // bytes per stage (64 KB)
constexpr int OUTP = 128 * 2 + 16;      // epilogue staging row pitch (bytes)
constexpr int OUTW = 128 * OUTP;        // staging bytes per wave
constexpr size_t LDS_MAIN = (size_t)NST * STB > (size_t)4 * OUTW ? (size_t)NST * STB
                                                                  : (size_t)4 * OUTW;
// the LoRA operands of a tile for r == 16, above the stages and the staging
// tiles: V rows m0 .. m0 + 255 (fp32, 64 B each), then L rows c0 .. c0 + 255
// (bf16, 32 B each)
constexpr int LORA_R = 16;
constexpr size_t LDS_V = LDS_MAIN, LDS_L = LDS_V + 256 * LORA_R * 4;
constexpr size_t LDS_BYTES = LDS_L + 256 * LORA_R * 2;
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// the same product with the accumulator pinned in AGPRs (destination tied to
// the addend); the caller keeps dependent reads of c away from it
__device__ __forceinline__ void mfma16_acc(bf16x8 a, bf16x8 b, f32x4& c) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Descriptor over [base, base + bytes) from wave-uniform values (kept in SGPRs).
__device__ __forceinline__ rsrc_t make_rs(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
// lane l's 16 bytes at base + voff + soff land at lds + 16 l
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LORA16: r == 16, the LoRA operands prefetched into LDS; otherwise read in
// the tail from global memory (one tail per instance keeps the registers of
// the other out of the kernel).
template <bool LORA16>
__global__ __launch_bounds__(T, 1) void k_gemm_nt(
    const uint16_t* __restrict__ A, int64_t lda, int64_t R, const uint16_t* __restrict__ Bm,
    int64_t ldb, int steps, int64_t M, int64_t Nc, const float* __restrict__ V,
    const uint16_t* __restrict__ L, int r, float s, uint16_t* __restrict__ C, int tiles_m,
    int tiles_c) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order: the eight XCDs take workgroups round robin; when the tile
  // count allows, XCD x gets a contiguous run of the grouped order below
  // (four tile rows at a time, across the columns), so that the workgroups
  // sharing an L2 share rows of A and of Bm.
  int bid = blockIdx.x;
  const int ntiles = tiles_m * tiles_c;
  if (ntiles % 8 == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  int tm, tc;
  if (tiles_m % 4 == 0) {
    const int grp = bid / (4 * tiles_c), in = bid % (4 * tiles_c);
    tm = 4 * grp + (in & 3);
    tc = in >> 2;
  } else {
    tm = bid / tiles_c;
    tc = bid % tiles_c;
  }
  tm = __builtin_amdgcn_readfirstlane(tm);
  tc = __builtin_amdgcn_readfirstlane(tc);
  const int64_t m0 = (int64_t)tm * BM, c0 = (int64_t)tc * BN;
  const int64_t mrows = min((int64_t)BM, M - m0), ncols = min((int64_t)BN, Nc - c0);

  // ---- loads: a stage holds 64 reduction elements (128-byte rows, one
  // cache line per row and step).  Load instruction i (0..7) of wave w covers
  // rows 64w + 8i + l/8 of an operand; lane l fills unit l%8 of its row with
  // source chunk (l%8) ^ ((row >> 1) & 7), so the 1 KB it writes is
  // contiguous and the sixteen rows a fragment read touches sit on distinct
  // banks.
  const rsrc_t rsA = make_rs(A + m0 * lda, (uint32_t)(mrows * lda * 2));
  const rsrc_t rsB = make_rs(Bm + c0 * ldb, (uint32_t)(ncols * ldb * 2));
  uint32_t aoff[8], boff[8];
  int achunk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = 64 * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ (int)((row >> 1) & 7);
    achunk[i] = chunk;
    aoff[i] = (uint32_t)((min(row, mrows - 1) * lda + 8 * chunk) * 2);
    boff[i] = (uint32_t)((min(row, ncols - 1) * ldb + 8 * chunk) * 2);
  }
  // A's reduction tail: a chunk past R is moved back onto the row's last
  // chunk (its Bm partner is zero)
  auto a_back = [&](int st, int i) {
    const int64_t k = (int64_t)st * BK + 8 * achunk[i];
    return (uint32_t)(2 * (k - min(k, R - 8)));
  };
  // load q (0..15) of step st: q < 8 A rows, else B rows
  auto load_one = [&](int q, int st, int stage) {
    uint8_t* d = smem + stage * STB + (q >= 8 ? OPB : 0) + wave * 8192 + 1024 * (q & 7);
    const uint32_t so = (uint32_t)st * (BK * 2);
    if (q < 8)
      dma16(rsA, aoff[q] - a_back(st, q), so, d);
    else
      dma16(rsB, boff[q - 8], so, d);
  };

  // ---- fragment reads (v_mfma_f32_16x16x32_bf16): tile t of the wave's 128
  // rows, half h of the stage: lane l reads row 16t + l%16 at chunk
  // 4h + l/16 (eight consecutive reduction elements)
  const int l16 = lane & 15, g4 = lane >> 4;
  int roff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) roff[h] = l16 * ROWB + 16 * ((4 * h + g4) ^ ((l16 >> 1) & 7));
  const int abase = wm * 128 * ROWB, bbase = OPB + wn * 128 * ROWB;
  auto frag = [&](int stage, int opbase, int t, int h) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(smem + stage * STB + opbase + t * 16 * ROWB +
                                                     roff[h]));
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};

  // A fragments are replaced in place once their row of MFMAs has issued;
  // B fragments come in two sets (first and second half of a stage)
  bf16x8 fa[8], fb[2][8];

  // ---- the LoRA operands (r == 16) go first, straight into LDS: they land
  // before step 0's loads (loads complete in order), long before the tail
  // reads them; rows past M or Nc read zeros.
  constexpr bool lora16 = LORA16;
  if constexpr (LORA16) {
    const rsrc_t rsV = make_rs(V + m0 * r, (uint32_t)(mrows * LORA_R * 4));
    const rsrc_t rsL = make_rs(L + c0 * r, (uint32_t)(ncols * LORA_R * 2));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dma16(rsV, (uint32_t)(1024 * (4 * wave + k) + 16 * lane), 0,
            smem + LDS_V + 1024 * (4 * wave + k));
#pragma unroll
    for (int k = 0; k < 2; ++k)
      dma16(rsL, (uint32_t)(1024 * (2 * wave + k) + 16 * lane), 0,
            smem + LDS_L + 1024 * (2 * wave + k));
  }

  // ---- prologue: steps 0 and 1 in flight, 0 landed
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int q = 0; q < 16; ++q) load_one(q, min(k, steps - 1), k);
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  barrier_lds();
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    fa[t] = frag(0, abase, t, 0);
    fb[0][t] = frag(0, bbase, t, 0);
  }

  // ---- half h of step st on stage P: 64 MFMAs.  Half 0 reads half 1's
  // fragments from the same stage, then waits for step st+1 (sent during
  // half 1 of step st-1) and meets the other waves: after that barrier no
  // wave reads stage P again.  Half 1 reads the next step's first half from
  // the other stage and sends the sixteen loads of step st+2 into stage P.
  // Half 1 needs no barrier of its own: the next half 0 reads only data that
  // every wave waited for before the barrier above, and writes none.
  auto half = [&](auto p_t, auto h_t, int st) {
    constexpr int P = decltype(p_t)::value, H = decltype(h_t)::value;
    constexpr int RS = H == 0 ? P : (P + 1) % NST;  // stage of the fragments read ahead
    constexpr int RH = H ^ 1;                       // their half
    const int lst = min(st + 2, steps - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mfma16_acc(fb[H][j], fa[i], acc[i][j]);
        if (j == 1) fb[RH][i] = frag(RS, bbase, i, RH);
        if (H == 1 && (j == 3 || j == 6)) load_one(2 * i + (j == 6), lst, P);
      }
      fa[i] = frag(RS, abase, i, RH);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (H == 0) {
      wait_all_loads();
      barrier_lds();
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  int st = 0;
  for (; st + 2 <= steps; st += 2) {
    half(S0{}, S0{}, st);
    half(S0{}, S1{}, st);
    half(S1{}, S0{}, st + 1);
    half(S1{}, S1{}, st + 1);
  }
  if (st < steps) {
    half(S0{}, S0{}, st);
    half(S0{}, S1{}, st);
  }
  // every wave's loads have landed and all reads are done before the stages
  // are reused for the output staging below; the last products' results are
  // complete before any instruction the compiler places here (a register
  // spill, say) reads an accumulator: it cannot see that the asm MFMAs write
  // them
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  wait_all_loads();
  barrier_lds();

  // ---- LoRA term: acc += (s V) L^T, 16 ranks per MFMA reduction of 32: lane
  // group g4 < 2 carries the bf16 high part of s V, g4 >= 2 its remainder,
  // both against the same eight ranks 8(g4 & 1) .. +7 of L.
  const bool vec = (r % 8) == 0;
  const bool lo_part = g4 >= 2;
  if constexpr (LORA16) {
    // from LDS: L row (tile column) wn 128 + 16 j + l16, ranks 8 (g4 & 1) ..;
    // V row (tile row) wm 128 + 16 i + l16, the same ranks
    const int jb = 8 * (g4 & 1);
    bf16x8 lh[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      lh[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(
          smem + LDS_L + (wn * 128 + 16 * j + l16) * (LORA_R * 2) + 2 * jb));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint8_t* vp = smem + LDS_V + (wm * 128 + 16 * i + l16) * (LORA_R * 4) + 4 * jb;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(vp);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(vp + 16);
      const float vr[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = s * vr[2 * q], x1 = s * vr[2 * q + 1];
        const uint32_t h = pack_bf16x2(x0, x1);
        w[q] = lo_part ? pack_bf16x2(x0 - bf16_lo(h), x1 - bf16_hi(h)) : h;
      }
      const bf16x8 av = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
#pragma unroll
      for (int j = 0; j < 8; ++j) mfma16_acc(lh[j], av, acc[i][j]);
    }
  }
  for (int j0 = 0; j0 < (LORA16 ? 0 : r); j0 += 16) {
    const int jl = j0 + 8 * (g4 & 1);
    bf16x8 lh[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t col = min(c0 + wn * 128 + 16 * j + l16, Nc - 1);
      const uint16_t* lp = L + col * r;
      if (vec) {
        lh[j] = jl < r ? as_bf16x8(*reinterpret_cast<const u32x4*>(lp + jl)) : bf16x8{};
      } else {
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = jl + q < r ? lp[min(jl + q, r - 1)] : 0u;
        lh[j] = as_bf16x8(u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                e[6] | (e[7] << 16)});
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = min(m0 + wm * 128 + 16 * i + l16, M - 1);
      const float* vp = V + m * r;
      float vr[8];
      if (vec && jl < r) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(vp + jl);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(vp + jl + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          vr[q] = v0[q];
          vr[4 + q] = v1[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) vr[q] = jl + q < r ? vp[min(jl + q, r - 1)] : 0.f;
      }
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = s * vr[2 * q], x1 = s * vr[2 * q + 1];
        const uint32_t h = pack_bf16x2(x0, x1);
        w[q] = lo_part ? pack_bf16x2(x0 - bf16_lo(h), x1 - bf16_hi(h)) : h;
      }
      const bf16x8 av = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
#pragma unroll
      for (int j = 0; j < 8; ++j) mfma16_acc(lh[j], av, acc[i][j]);
    }
  }

  // ---- store.  Tile (i, j) is held transposed: lane l has row 16i + l%16
  // and columns 16j + 4(l/16) .. +3 in its four registers; they go to the
  // wave's LDS staging tile as 8 bytes, and the tile then leaves as rows of
  // 256 contiguous bytes, four rows per store.  The staging tiles overlap the
  // stages, freed by the barrier above.
  uint8_t* stg = smem + wave * OUTW;
  // the last products' results are complete before they are read
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4& c = acc[i][j];
      *reinterpret_cast<u32x2*>(stg + (16 * i + l16) * OUTP + 2 * (16 * j + 4 * g4)) =
          u32x2{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
    }
  }
  // (a wave's LDS accesses execute in order, so its reads see its writes)
  // Streaming (non-temporal) stores: the output is written once and never
  // read here, while the caches still serve other tiles' re-reads of the A
  // and Bm rows; ordinary stores would displace those lines.
  const int64_t col = c0 + wn * 128 + 8 * (lane & 15);
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int rl = 4 * q + (lane >> 4);
    const int64_t row = m0 + wm * 128 + rl;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rl * OUTP + 16 * (lane & 15));
    if (row < M && col < Nc)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + row * Nc + col));
  }
}

}  // namespace

size_t gemm_nt_lds_bytes() { return LDS_BYTES; }

hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, int64_t R, const uint16_t* Bm,
                          int64_t ldb, int64_t M, int64_t Nc, const float* V, const uint16_t* L,
                          int r, float s, uint16_t* C, hipStream_t st) {
  static hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gemm_nt<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k_gemm_nt<false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_MAIN);
  }();
  if (attr != hipSuccess) return attr;
  if (M <= 0) return hipSuccess;
  if (ldb % BK != 0 || R < 8 || R > ldb) return hipErrorInvalidValue;
  const int64_t tm = (M + BM - 1) / BM, tc = (Nc + BN - 1) / BN;
  const int steps = (int)(ldb / BK);
  if (r == LORA_R)
    hipLaunchKernelGGL(k_gemm_nt<true>, dim3((unsigned)(tm * tc)), dim3(T), LDS_BYTES, st, A, lda,
                       R, Bm, ldb, steps, M, Nc, V, L, r, s, C, (int)tm, (int)tc);
  else
    hipLaunchKernelGGL(k_gemm_nt<false>, dim3((unsigned)(tm * tc)), dim3(T), LDS_MAIN, st, A, lda,
                       R, Bm, ldb, steps, M, Nc, V, L, r, s, C, (int)tm, (int)tc);
  return hipGetLastError();
}

}  // namespace qn
