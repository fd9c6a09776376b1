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
// tiles of v_mfma_f32_16x16x32_bf16 (256 accumulators, pinned in AGPRs); for
// outputs with too few such tiles to fill the chip, the same kernel with
// 128 x 128 tiles (each wave 64 x 64 as 4 x 4 tiles, half the LDS, two
// workgroups per compute unit).  On
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
// distinct banks.  The next half's B fragments are read during the first
// row of a half's MFMAs (its first row uses all eight), its A fragments one
// per row.  Rows of A past its length R are moved back onto its last
// chunk; Bm is zero there (its rows are padded to a multiple of 64 with
// zeros).
#include <type_traits>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int BK = 64, T = 256;
constexpr int ROWB = BK * 2;  // bytes per tile row per stage (one cache line)
constexpr int LORA_R = 16;
// Tile geometry for a wave tile of WTM x WTN MFMA tiles (16 x 16 each): the
// workgroup tile is BM x BN, BM = 32 WTM rows of A, BN = 32 WTN rows of Bm
// (output columns).
template <int WTM, int WTN>
struct Geo {
  static constexpr int WRM = 16 * WTM, WRN = 16 * WTN;  // rows and columns per wave
  static constexpr int BM = 2 * WRM, BN = 2 * WRN;      // workgroup tile
  static constexpr int OPA = BM * ROWB, OPB = BN * ROWB;  // bytes per operand per stage
  static constexpr int STB = OPA + OPB;                 // bytes per stage
  static constexpr int OUTP = WRN * 2 + 16;             // epilogue staging row pitch (bytes)
  static constexpr int OUTW = WRM * OUTP;               // staging bytes per wave
  static constexpr int LPS = WTM + WTN;                 // loads per wave and step
  // LDS stages: a 128 x 128 tile's step is a quarter of a 256 x 256 one's
  // MFMA time, so its loads go out three steps ahead instead of one
  static constexpr int NST = WTM == 8 ? 2 : 4;
  static constexpr size_t LDS_MAIN = (size_t)NST * STB > (size_t)4 * OUTW ? (size_t)NST * STB
                                                                         : (size_t)4 * OUTW;
  // the LoRA operands of a tile for r == 16, above the stages and the
  // staging tiles: V rows m0 .. m0 + BM - 1 (fp32, 64 B each), then L rows
  // c0 .. c0 + BN - 1 (bf16, 32 B each)
  static constexpr size_t LDS_V = LDS_MAIN, LDS_L = LDS_V + BM * LORA_R * 4;
  static constexpr size_t LDS_BYTES = LDS_L + BN * LORA_R * 2;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(NST == 2 || NST == 4, "stages");
  static_assert(WTN <= WTM && WTN >= WTM / 2, "load slots");
  // the loads of a step: WTM instructions of A rows and WTN of Bm rows per
  // wave, each eight whole rows; two load slots per row of the second half's
  // MFMAs, at these columns (with seven columns, off the row's last one: a
  // load issued just before the row's fragment read cost ~45 cycles a step)
  static constexpr int J1 = WTM == 8 ? (WTN == 7 ? 2 : 3) : 1;
  static constexpr int J2 = WTM == 8 ? (WTN == 7 ? 5 : 6) : 3;
};

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
// the other out of the kernel).  ATAIL: the reduction length R is shorter
// than the steps cover (R < ldb), so A's chunks past R are moved back; with
// R == ldb the A loads need no address arithmetic per step (the 64-bit
// clamp in the loop cost 12% of the main loop's cycles at 8192x4096x4096).
template <bool LORA16, int WTM, int WTN, bool ATAIL>
__global__ __launch_bounds__(T, 1) void k_gemm_nt(
    const uint16_t* __restrict__ A, int64_t lda, int64_t R, const uint16_t* __restrict__ Bm,
    int64_t ldb, int steps, int64_t M, int64_t Nc, const float* __restrict__ V,
    const uint16_t* __restrict__ L, int r, float s, uint16_t* __restrict__ C, int tiles_m,
    int tiles_c) {
  using G = Geo<WTM, WTN>;
  constexpr int BM = G::BM, BN = G::BN, WRM = G::WRM, WRN = G::WRN, OPA = G::OPA, STB = G::STB;
  constexpr int OUTP = G::OUTP, OUTW = G::OUTW, NST = G::NST, LPS = G::LPS;
  constexpr size_t LDS_V = G::LDS_V, LDS_L = G::LDS_L;
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
  // cache line per row and step).  Load instruction i (0..WTM-1 for A,
  // 0..WTN-1 for Bm) of wave w covers rows 8 n w + 8i + l/8 of the operand
  // (n its instruction count); lane l fills unit l%8 of its row with
  // source chunk (l%8) ^ ((row >> 1) & 7), so the 1 KB it writes is
  // contiguous and the sixteen rows a fragment read touches sit on distinct
  // banks.
  const rsrc_t rsA = make_rs(A + m0 * lda, (uint32_t)(mrows * lda * 2));
  const rsrc_t rsB = make_rs(Bm + c0 * ldb, (uint32_t)(ncols * ldb * 2));
  uint32_t aoff[WTM], boff[WTN];
  int achunk[WTM];
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
    const int64_t row = 8 * WTM * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ (int)((row >> 1) & 7);
    achunk[i] = chunk;
    aoff[i] = (uint32_t)((min(row, mrows - 1) * lda + 8 * chunk) * 2);
  }
#pragma unroll
  for (int i = 0; i < WTN; ++i) {
    const int64_t row = 8 * WTN * wave + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ (int)((row >> 1) & 7);
    boff[i] = (uint32_t)((min(row, ncols - 1) * ldb + 8 * chunk) * 2);
  }
  // A's reduction tail: a chunk past R is moved back onto the row's last
  // chunk (its Bm partner is zero)
  auto a_back = [&](int st, int i) {
    if constexpr (!ATAIL) return 0u;
    const int64_t k = (int64_t)st * BK + 8 * achunk[i];
    return (uint32_t)(2 * (k - min(k, R - 8)));
  };
  // load q (0 .. LPS - 1) of step st: q < WTM A rows, else Bm rows
  auto load_one = [&](int q, int st, int stage) {
    const uint32_t so = (uint32_t)st * (BK * 2);
    if (q < WTM) {
      dma16(rsA, aoff[q] - a_back(st, q), so,
            smem + stage * STB + wave * (1024 * WTM) + 1024 * q);
    } else {
      dma16(rsB, boff[q - WTM], so,
            smem + stage * STB + OPA + wave * (1024 * WTN) + 1024 * (q - WTM));
    }
  };

  // ---- fragment reads (v_mfma_f32_16x16x32_bf16): tile t of the wave's
  // rows, half h of the stage: lane l reads row 16t + l%16 at chunk
  // 4h + l/16 (eight consecutive reduction elements)
  const int l16 = lane & 15, g4 = lane >> 4;
  int roff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) roff[h] = l16 * ROWB + 16 * ((4 * h + g4) ^ ((l16 >> 1) & 7));
  const int abase = wm * WRM * ROWB, bbase = OPA + wn * WRN * ROWB;
  auto frag = [&](int stage, int opbase, int t, int h) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(smem + stage * STB + opbase + t * 16 * ROWB +
                                                     roff[h]));
  };

  f32x4 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = f32x4{};

  // A fragments are replaced in place once their row of MFMAs has issued;
  // B fragments come in two sets (first and second half of a stage)
  bf16x8 fa[WTM], fb[2][WTN];

  // ---- the LoRA operands (r == 16) go first, straight into LDS: they land
  // before step 0's loads (loads complete in order), long before the tail
  // reads them; rows past M or Nc read zeros.
  constexpr bool lora16 = LORA16;
  if constexpr (LORA16) {
    const rsrc_t rsV = make_rs(V + m0 * r, (uint32_t)(mrows * LORA_R * 4));
    const rsrc_t rsL = make_rs(L + c0 * r, (uint32_t)(ncols * LORA_R * 2));
    // V: BM rows x 64 B = WTM / 2 KB per wave; L: BN rows x 32 B = WTN KB,
    // instruction k from wave k % 4 (rows past Nc read zeros)
    constexpr int KV = WTM / 2, KL = WTN;
#pragma unroll
    for (int k = 0; k < KV; ++k)
      dma16(rsV, (uint32_t)(1024 * (KV * wave + k) + 16 * lane), 0,
            smem + LDS_V + 1024 * (KV * wave + k));
#pragma unroll
    for (int k = 0; k < (KL + 3) / 4; ++k) {
      const int q = 4 * k + wave;
      if (q < KL)
        dma16(rsL, (uint32_t)(1024 * q + 16 * lane), 0, smem + LDS_L + 1024 * q);
    }
  }

  // ---- prologue: steps 0 .. NST-1 in flight, 0 landed (all but the later
  // steps' LPS loads each)
#pragma unroll
  for (int k = 0; k < NST; ++k)
#pragma unroll
    for (int q = 0; q < LPS; ++q) load_one(q, min(k, steps - 1), k);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS * (NST - 1)) : "memory");
  barrier_lds();
#pragma unroll
  for (int t = 0; t < WTM; ++t) fa[t] = frag(0, abase, t, 0);
#pragma unroll
  for (int t = 0; t < WTN; ++t) fb[0][t] = frag(0, bbase, t, 0);

  // ---- half h of step st on stage P = st % NST: WTM x WTN MFMAs.  Half 0
  // reads half 1's fragments from the same stage, then waits for step st+1
  // (sent during half 1 of step st+1-NST; the later steps' loads stay in
  // flight) and meets the other waves: after that barrier no wave reads
  // stage P again.  Half 1 reads the next step's first half from the next
  // stage and sends the LPS loads of step st+NST into stage P.  Half 1
  // needs no barrier of its own: the next half 0 reads only data that every
  // wave waited for before the barrier above, and writes none.
  auto half = [&](auto p_t, auto h_t, int st) {
    constexpr int P = decltype(p_t)::value, H = decltype(h_t)::value;
    constexpr int RS = H == 0 ? P : (P + 1) % NST;  // stage of the fragments read ahead
    constexpr int RH = H ^ 1;                       // their half
    const int lst = min(st + NST, steps - 1);
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
        mfma16_acc(fb[H][j], fa[i], acc[i][j]);
        // the next half's B fragments are all read during the first row of
        // MFMAs: its first row needs every one of them
        if (i == 0) fb[RH][j] = frag(RS, bbase, j, RH);
        if (H == 1 && (j == G::J1 || j == G::J2) && 2 * i + (j == G::J2) < LPS)
          load_one(2 * i + (j == G::J2), lst, P);
      }
      fa[i] = frag(RS, abase, i, RH);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (H == 0) {
      if constexpr (NST == 2)
        wait_all_loads();
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS * (NST - 2)) : "memory");
      barrier_lds();
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  auto step = [&](auto p_t, int st) {
    half(p_t, S0{}, st);
    half(p_t, S1{}, st);
  };
  // Wherever control flow joins after MFMAs (the loop's exit, the end of a
  // conditional step) the compiler may copy an accumulator to another AGPR
  // for the join; 32 wait states first let the last products complete (it
  // cannot know that the asm MFMAs write late: at the 256 x 224 tile's loop
  // exit it copied the last accumulator 4 cycles after its MFMA issued).
  // The exit test sits at the end of the body, so the back edge skips them.
  auto drain = [&]() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); };
  int st = 0;
  if (steps >= NST) {
    for (;;) {
      step(S0{}, st);
      step(S1{}, st + 1);
      if constexpr (NST == 4) {
        step(S2{}, st + 2);
        step(S3{}, st + 3);
      }
      st += NST;
      if (st + NST > steps) {
        drain();
        break;
      }
    }
  }
  // the last steps % NST steps, on stages 0, 1, 2 in turn
  if (st < steps) {
    step(S0{}, st++);
    drain();
  }
  if constexpr (NST == 4) {
    if (st < steps) {
      step(S1{}, st++);
      drain();
    }
    if (st < steps) {
      step(S2{}, st++);
      drain();
    }
  }
  // The compiler cannot see that the asm MFMAs write the accumulators some
  // cycles after they issue, so nothing it places may read one before the
  // last products are complete: 32 wait states, then an empty asm that
  // "rewrites" every accumulator, which no read of it can move above (a
  // register copy is not ordered by a memory clobber alone; without the ties
  // the compiler hoisted the output conversion's AGPR reads above the wait
  // states and read partial sums).
  auto settle = [&]() {
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j) asm volatile("" : "+a"(acc[i][j]));
  };
  // every wave's loads have landed and all reads are done before the stages
  // are reused for the output staging below
  settle();
  wait_all_loads();
  barrier_lds();

  // ---- LoRA term: acc += (s V) L^T, 16 ranks per MFMA reduction of 32: lane
  // group g4 < 2 carries the bf16 high part of s V, g4 >= 2 its remainder,
  // both against the same eight ranks 8(g4 & 1) .. +7 of L.
  const bool vec = (r % 8) == 0;
  const bool lo_part = g4 >= 2;
  if constexpr (LORA16) {
    // from LDS: L row (tile column) wn WRN + 16 j + l16, ranks 8 (g4 & 1) ..;
    // V row (tile row) wm WRM + 16 i + l16, the same ranks
    const int jb = 8 * (g4 & 1);
    bf16x8 lh[WTN];
#pragma unroll
    for (int j = 0; j < WTN; ++j)
      lh[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(
          smem + LDS_L + (wn * WRN + 16 * j + l16) * (LORA_R * 2) + 2 * jb));
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const uint8_t* vp = smem + LDS_V + (wm * WRM + 16 * i + l16) * (LORA_R * 4) + 4 * jb;
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
      for (int j = 0; j < WTN; ++j) mfma16_acc(lh[j], av, acc[i][j]);
    }
  }
  for (int j0 = 0; j0 < (LORA16 ? 0 : r); j0 += 16) {
    const int jl = j0 + 8 * (g4 & 1);
    bf16x8 lh[WTN];
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int64_t col = min(c0 + wn * WRN + 16 * j + l16, Nc - 1);
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
    for (int i = 0; i < WTM; ++i) {
      const int64_t m = min(m0 + wm * WRM + 16 * i + l16, M - 1);
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
      for (int j = 0; j < WTN; ++j) mfma16_acc(lh[j], av, acc[i][j]);
    }
    drain();  // (a loop: its exit is a join)
  }

  // ---- store.  Tile (i, j) is held transposed: lane l has row 16i + l%16
  // and columns 16j + 4(l/16) .. +3 in its four registers; they go to the
  // wave's LDS staging tile as 8 bytes, and the tile then leaves as rows of
  // 2 WRN contiguous bytes (2 WTN lanes of 16 bytes per row).  The staging
  // tiles overlap the stages, freed by the barrier above.
  uint8_t* stg = smem + wave * OUTW;
  // the last products' results are complete before they are read
  settle();
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const f32x4& c = acc[i][j];
      *reinterpret_cast<u32x2*>(stg + (16 * i + l16) * OUTP + 2 * (16 * j + 4 * g4)) =
          u32x2{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
    }
  }
  // (a wave's LDS accesses execute in order, so its reads see its writes)
  // Streaming (non-temporal) stores: the output is written once and never
  // read here, while the caches still serve other tiles' re-reads of the A
  // and Bm rows; ordinary stores would displace those lines.
  // lanes per row, rows per store (with 14 lanes per row, lanes 56..63 idle)
  constexpr int LR = 2 * WTN, RPS = 64 / LR;
  static_assert(WRM % RPS == 0, "store rows");
  const int lc = lane % LR;
  const bool lane_on = lane < RPS * LR;
  const int64_t col = c0 + wn * WRN + 8 * lc;
#pragma unroll
  for (int q = 0; q < WRM / RPS; ++q) {
    const int rl = RPS * q + min(lane / LR, RPS - 1);
    const int64_t row = m0 + wm * WRM + rl;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rl * OUTP + 16 * lc);
    if (lane_on && row < M && col < Nc)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + row * Nc + col));
  }
}

}  // namespace

size_t gemm_nt_lds_bytes() { return Geo<8, 8>::LDS_BYTES; }

namespace {
template <int WTM, int WTN>
hipError_t launch_wt(const uint16_t* A, int64_t lda, int64_t R, const uint16_t* Bm, int64_t ldb,
                     int64_t M, int64_t Nc, const float* V, const uint16_t* L, int r, float s,
                     uint16_t* C, hipStream_t st) {
  using G = Geo<WTM, WTN>;
  static hipError_t attr = [] {
    const void* k16[2] = {reinterpret_cast<const void*>(k_gemm_nt<true, WTM, WTN, false>),
                          reinterpret_cast<const void*>(k_gemm_nt<true, WTM, WTN, true>)};
    const void* kr[2] = {reinterpret_cast<const void*>(k_gemm_nt<false, WTM, WTN, false>),
                         reinterpret_cast<const void*>(k_gemm_nt<false, WTM, WTN, true>)};
    for (int t = 0; t < 2; ++t) {
      hipError_t e = hipFuncSetAttribute(k16[t], hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)G::LDS_BYTES);
      if (e == hipSuccess)
        e = hipFuncSetAttribute(kr[t], hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)G::LDS_MAIN);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  const int64_t tm = (M + G::BM - 1) / G::BM, tc = (Nc + G::BN - 1) / G::BN;
  const int steps = (int)(ldb / BK);
  const dim3 grid((unsigned)(tm * tc)), block(T);
#define QN_GEMM(L16, TAIL)                                                                     \
  hipLaunchKernelGGL((k_gemm_nt<L16, WTM, WTN, TAIL>), grid, block,                           \
                     L16 ? G::LDS_BYTES : G::LDS_MAIN, st, A, lda, R, Bm, ldb, steps, M, Nc, V, \
                     L, r, s, C, (int)tm, (int)tc)
  const bool tail = R != ldb;
  if (r == LORA_R) {
    if (tail) QN_GEMM(true, true); else QN_GEMM(true, false);
  } else {
    if (tail) QN_GEMM(false, true); else QN_GEMM(false, false);
  }
#undef QN_GEMM
  return hipGetLastError();
}

int compute_units() {
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return n > 0 ? n : 256;
  }();
  return cus;
}
}  // namespace

bool gemm_nt_small_tiles(int64_t M, int64_t Nc) {
  return ((M + 255) / 256) * ((Nc + 255) / 256) < 240;
}

hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, int64_t R, const uint16_t* Bm,
                          int64_t ldb, int64_t M, int64_t Nc, const float* V, const uint16_t* L,
                          int r, float s, uint16_t* C, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (ldb % BK != 0 || R < 8 || R > ldb) return hipErrorInvalidValue;
  // 256 x 256 tiles once there are about as many as compute units; fewer
  // would leave most of the chip idle, so 128 x 128 tiles then
  if (gemm_nt_small_tiles(M, Nc))
    return launch_wt<4, 4>(A, lda, R, Bm, ldb, M, Nc, V, L, r, s, C, st);
  // 256 x 224 tiles where they take fewer tile-widths of rounds: with 14336
  // output columns at M = 4096, 896 tiles of 256 fill 3.5 rounds of the
  // chip and the last round runs half empty, while 1024 tiles of 224 fill
  // exactly 4 (4 x 224 < 4 x 256 column-widths of time)
  const int64_t cu = compute_units(), tm = (M + 255) / 256;
  const int64_t r256 = (tm * ((Nc + 255) / 256) + cu - 1) / cu;
  const int64_t r224 = (tm * ((Nc + 223) / 224) + cu - 1) / cu;
  if (r224 * 224 < r256 * 256)
    return launch_wt<8, 7>(A, lda, R, Bm, ldb, M, Nc, V, L, r, s, C, st);
  return launch_wt<8, 8>(A, lda, R, Bm, ldb, M, Nc, V, L, r, s, C, st);
}

}  // namespace qn
