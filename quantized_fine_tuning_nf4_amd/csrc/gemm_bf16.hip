// bf16 GEMM with the LoRA term fused in the epilogue, for large batches:
//
//   C[M, Nc] (bf16) = A[M, R] Bm[Nc, R]^T + s V[M, r] L[Nc, r]^T
//
// used for the forward (A = x, Bm = Qhat(W) [N, K], V = u, L = B) and for
// dX (A = dY, Bm = Qhat(W)^T [K, N], V = v, L = A^T) of the page "QLoRA: NF4
// storage, gradients and local integration" (paragraph after the teaching
// listing), once the weight has been dequantized to bf16 in a workspace.
//
// Workgroup tile 256 x 256, four waves (2 x 2), each wave 128 x 128 as 4 x 4
// tiles of v_mfma_f32_32x32x16_bf16 (256 accumulators).  A step covers 32
// reduction elements; both operands are brought from global memory straight
// into LDS by buffer loads (no registers), four stages deep: the loads of
// step s+3 are issued at the start of step s, and the barrier ending step s
// guarantees step s+2, so the fragments of step s+1 are read during step s.
// LDS rows are 64 bytes (four 16-byte chunks); chunk c of row y sits at unit
// c ^ ((y >> 2) & 3), which keeps 16 consecutive rows read at one chunk on
// distinct banks.  Reduction order inside a step: lane group g = lane/32 and
// substep ks take elements 16 ks + 8 g + 0..7 (chunk 2 ks + g) of both
// operands.  Rows of A past its length R are clamped onto its last chunk;
// Bm is zero there (its rows are padded to a multiple of 32 with zeros).
#include <type_traits>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int BM = 256, BN = 256, BK = 32, NST = 4, T = 256;
constexpr int ROWB = BK * 2;            // bytes per tile row per stage
constexpr int OPB = 256 * ROWB;         // bytes per operand per stage (16 KB)
constexpr int STB = 2 * OPB;            // bytes per stage
constexpr int OUTP = 128 * 2 + 16;      // epilogue staging row pitch (bytes)
constexpr int OUTW = 128 * OUTP;        // staging bytes per wave
constexpr size_t LDS_BYTES = (size_t)NST * STB > (size_t)4 * OUTW ? (size_t)NST * STB
                                                                   : (size_t)4 * OUTW;

typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
// all but the newest step's eight loads have landed
__device__ __forceinline__ void wait_all_but_one_step() {
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}
__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__global__ __launch_bounds__(T, 1) void k_gemm_nt(
    const uint16_t* __restrict__ A, int64_t lda, int64_t R, const uint16_t* __restrict__ Bm,
    int64_t ldb, int steps, int64_t M, int64_t Nc, const float* __restrict__ V,
    const uint16_t* __restrict__ L, int r, float s, uint16_t* __restrict__ C, int tiles_m,
    int tiles_c) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
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

  // ---- loads: instruction i of wave w covers tile rows 64w + 16i + l/4,
  // stored unit l%4, source chunk (l%4) ^ ((row >> 2) & 3).
  const rsrc_t rsA = make_rs(A + m0 * lda, (uint32_t)(mrows * lda * 2));
  const rsrc_t rsB = make_rs(Bm + c0 * ldb, (uint32_t)(ncols * ldb * 2));
  const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = 64 * wave + 16 * i + (lane >> 2);
    aoff[i] = (uint32_t)((min(row, mrows - 1) * lda + 8 * chunk) * 2);
    boff[i] = (uint32_t)((min(row, ncols - 1) * ldb + 8 * chunk) * 2);
  }
  // A's reduction tail: columns past R are clamped onto the row's last chunk
  auto a_back = [&](int st) {
    const int64_t k = (int64_t)st * BK + 8 * chunk;
    return (uint32_t)(2 * (k - min(k, R - 8)));
  };
  // load q (0..7) of step st into its stage: q < 4 A rows, else B rows
  auto load_one = [&](int q, int st, int stage, uint32_t back) {
    uint8_t* d = smem + stage * STB + (q >= 4 ? OPB : 0) + wave * 4096 + 1024 * (q & 3);
    const uint32_t so = (uint32_t)st * (BK * 2);
    if (q < 4)
      dma16(rsA, aoff[q] - back, so, d);
    else
      dma16(rsB, boff[q - 4], so, d);
  };
  auto load_step = [&](int st, int stage) {
    const uint32_t back = a_back(st);
#pragma unroll
    for (int q = 0; q < 8; ++q) load_one(q, st, stage, back);
  };

  // ---- fragment reads: row 32t + l32 of a 32-row tile, chunk 2 ks + g
  int roff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) roff[ks] = l32 * ROWB + 16 * ((2 * ks + g) ^ ((l32 >> 2) & 3));
  const int abase = wm * 128 * ROWB, bbase = OPB + wn * 128 * ROWB;
  auto frag = [&](int stage, int opbase, int t, int ks) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(smem + stage * STB + opbase + t * 32 * ROWB +
                                                     roff[ks]));
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // fragment sets: X holds substep 0, Y substep 1
  bf16x8 xa[4], xb[4], ya[4], yb[4];

  // ---- prologue: steps 0, 1, 2 in flight; 0 and 1 landed
#pragma unroll
  for (int k = 0; k < 3; ++k) load_step(min(k, steps - 1), k);
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  barrier_lds();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    xa[t] = frag(0, abase, t, 0);
    xb[t] = frag(0, bbase, t, 0);
  }

  // ---- one step on stage P: 32 MFMAs in two substeps; during substep 0 the
  // Y set is read (substep 1 of this step), during substep 1 the X set (substep
  // 0 of the next step, whose data the previous barrier guaranteed).
  auto body = [&](auto p_t, int st) {
    constexpr int P = decltype(p_t)::value, PN = (P + 1) % NST, PL = (P + 3) % NST;
    // the loads of step st+3 are spread over the step, one per four MFMAs,
    // so that the wave never waits on a full address queue
    const int lst = min(st + 3, steps - 1);
    const uint32_t lback = a_back(lst);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int i = c >> 1, j0 = 2 * (c & 1);
        bf16x8* ca = ks == 0 ? xa : ya;
        bf16x8* cb = ks == 0 ? xb : yb;
        acc[i][j0] = mfma32(cb[j0], ca[i], acc[i][j0]);
        acc[i][j0 + 1] = mfma32(cb[j0 + 1], ca[i], acc[i][j0 + 1]);
        // one read per MFMA pair into the other set
        const int t = c >> 1;
        if ((c & 1) == 0) load_one(4 * ks + (c >> 1), lst, PL, lback);
        if (ks == 0) {
          if (c & 1) yb[t] = frag(P, bbase, t, 1);
          else ya[t] = frag(P, abase, t, 1);
        } else {
          if (c & 1) xb[t] = frag(PN, bbase, t, 0);
          else xa[t] = frag(PN, abase, t, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_all_but_one_step();
    barrier_lds();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  int st = 0;
  for (; st + 4 <= steps; st += 4) {
    body(S0{}, st);
    body(S1{}, st + 1);
    body(S2{}, st + 2);
    body(S3{}, st + 3);
  }
  if (st < steps) body(S0{}, st);
  if (st + 1 < steps) body(S1{}, st + 1);
  if (st + 2 < steps) body(S2{}, st + 2);
  // every wave's loads have landed and all reads are done before the stages
  // are reused for the output staging below
  wait_all_loads();
  barrier_lds();

  // ---- LoRA term: acc += (s V) L^T, 16 ranks at a time; s V enters as a
  // bf16 high part and a bf16 remainder.
  const bool vec = (r % 8) == 0;
  for (int j0 = 0; j0 < r; j0 += 16) {
    const int jl = j0 + 8 * g;
    bf16x8 lh[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = min(c0 + wn * 128 + 32 * j + l32, Nc - 1);
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
    float vr[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = min(m0 + wm * 128 + 32 * i + l32, M - 1);
      const float* vp = V + m * r;
      if (vec && jl < r) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(vp + jl);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(vp + jl + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          vr[i][q] = v0[q];
          vr[i][4 + q] = v1[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) vr[i][q] = jl + q < r ? vp[min(jl + q, r - 1)] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = s * vr[i][2 * q], x1 = s * vr[i][2 * q + 1];
        h[q] = pack_bf16x2(x0, x1);
        lo[q] = pack_bf16x2(x0 - bf16_lo(h[q]), x1 - bf16_hi(h[q]));
      }
      const bf16x8 ah = as_bf16x8(u32x4{h[0], h[1], h[2], h[3]});
      const bf16x8 al = as_bf16x8(u32x4{lo[0], lo[1], lo[2], lo[3]});
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma32(lh[j], ah, acc[i][j]);
        acc[i][j] = mfma32(lh[j], al, acc[i][j]);
      }
    }
  }

  // ---- store.  Tile (i, j) is held transposed: lane l has row 32i + l%32 and
  // columns 32j + 8q + 4(l/32) + e in register 4q + e.  Swapping lanes 32..63
  // of one register with lanes 0..31 of another gives each lane eight
  // consecutive columns 32j + 16p + 8(l/32) .. +7 of pair p, which go to the
  // wave's LDS staging tile; the
  // tile then leaves as rows of 256 contiguous bytes, four rows per store.
  // The staging tiles overlap the stages, freed by the barrier above.
  uint8_t* stg = smem + wave * OUTW;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const f32x16& c = acc[i][j];
        const int q0 = 2 * pr, q1 = 2 * pr + 1;
        const auto s0 = __builtin_amdgcn_permlane32_swap(pack_bf16x2(c[4 * q0], c[4 * q0 + 1]),
                                                         pack_bf16x2(c[4 * q1], c[4 * q1 + 1]),
                                                         false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(pack_bf16x2(c[4 * q0 + 2], c[4 * q0 + 3]),
                                                         pack_bf16x2(c[4 * q1 + 2], c[4 * q1 + 3]),
                                                         false, false);
        const int col = 32 * j + 16 * pr + 8 * g;
        *reinterpret_cast<u32x4*>(stg + (32 * i + l32) * OUTP + 2 * col) =
            u32x4{s0[0], s1[0], s0[1], s1[1]};
      }
    }
  }
  // (a wave's LDS accesses execute in order, so its reads see its writes)
  const int64_t col = c0 + wn * 128 + 8 * (lane & 15);
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int rl = 4 * q + (lane >> 4);
    const int64_t row = m0 + wm * 128 + rl;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rl * OUTP + 16 * (lane & 15));
    if (row < M && col < Nc) *reinterpret_cast<u32x4*>(C + row * Nc + col) = v;
  }
}

}  // namespace

size_t gemm_nt_lds_bytes() { return LDS_BYTES; }

hipError_t launch_gemm_nt(const uint16_t* A, int64_t lda, int64_t R, const uint16_t* Bm,
                          int64_t ldb, int64_t M, int64_t Nc, const float* V, const uint16_t* L,
                          int r, float s, uint16_t* C, hipStream_t st) {
  static hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(k_gemm_nt),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
  if (attr != hipSuccess) return attr;
  if (M <= 0) return hipSuccess;
  const int64_t tm = (M + BM - 1) / BM, tc = (Nc + BN - 1) / BN;
  const int steps = (int)(ldb / BK);
  hipLaunchKernelGGL(k_gemm_nt, dim3((unsigned)(tm * tc)), dim3(T), LDS_BYTES, st, A, lda, R, Bm,
                     ldb, steps, M, Nc, V, L, r, s, C, (int)tm, (int)tc);
  return hipGetLastError();
}

}  // namespace qn
