// Fused NF4-dequant bf16 MFMA GEMMs, 256 x 256 output tiles (large batches).
//
//   forward  Y  = X Qhat(W)^T + s u B^T,   u = X A^T
//   dX       dX = G Qhat(W)   + s v A,     v = G B
// (page "QLoRA: NF4 storage, gradients and local integration", paragraph
// after the teaching listing.)  Qhat(W) enters the MFMAs as bf16 (round to
// nearest even of w' = L[c] * s') and is never written to memory.
//
// Four waves, one per SIMD; wave w owns output columns 64w..64w+63 for all
// 256 rows: 8 x 2 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators).
// A step consumes 64 reduction elements.
//
// Data movement without prefetch registers: global_load_lds (lane l's bytes
// land at base + size * l) brings
//   - the activation tile of step s+1 (256 rows x 64 bf16 in 16-byte chunks,
//     chunk c of row r stored at unit c ^ f(r), f(r) = ((r >> 1) & 7) ^
//     ((r & 1) << 2), so that 8 or 16 consecutive rows read at one logical
//     chunk hit distinct banks) into the other of two shared stages, and
//   - the weight codes of step s+2 of this wave's 64 weight rows (32 bytes
//     each), their E4M3 scale bytes and fp32 second-level scales into the
//     other of two wave-private stages,
// all issued at the start of step s and drained before the barrier ending it.
// During step s a lane dequantizes the codes of step s+1 between the MFMAs:
//   forward: lane (row 32j + l%32, half l/32) turns 32 codes of each of its
//            two rows into the next step's B registers;
//   dX:      lane l turns row l's 64 codes into row l of a wave-private bf16
//            tile [n][k], read back as B fragments (eight consecutive n of one
//            column) with ds_read_b64_tr_b16, which gives lane i of each
//            16-lane group element i%4 of the chunks addressed by lanes
//            4q + i/4, q = 0..3.
// Reduction order inside a step, both operands: lane group g = lane/32 and
// substep ks take elements 32g + 8ks + 0..7 (activation chunk 4g + ks).
// The step loop is unrolled by two so that stage indices and the forward's
// current/next B registers alternate by name.
#include <type_traits>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int BM = 256, BN = 256, T = 256;
constexpr int STAGE_B = BM * 64 * 2;  // bytes per activation stage (32 KB)
constexpr int WLD = 72;               // private weight tile row (64 + 8 pad), dX
constexpr int WSTAGE_B = 64 * WLD * 2;

// LDS map (bytes)
constexpr int OFF_A = 0;                           // 2 activation stages
constexpr int OFF_C = OFF_A + 2 * STAGE_B;         // codes [wave][stage][64][32 B]
constexpr int OFF_Q = OFF_C + 4 * 2 * 64 * 32;     // scale bytes [wave][stage][64] (u32)
constexpr int OFF_S2 = OFF_Q + 4 * 2 * 64 * 4;     // scale2 [wave][stage][64]
constexpr int OFF_W = OFF_S2 + 4 * 2 * 64 * 4;     // dX: [wave][stage][64][WLD] bf16
constexpr size_t LDS_FWD = OFF_W;
constexpr size_t LDS_DX = OFF_W + (size_t)4 * 2 * WSTAGE_B;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes); the kernels keep every
// access inside it, the range check is a second guard.
// Arguments are wave-uniform; readfirstlane keeps the descriptor in SGPRs
// (a descriptor in VGPRs would need a loop over lanes at every use).
__device__ __forceinline__ rsrc_t make_rs(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
// Buffer loads straight to LDS: lane l's SIZE bytes from base + voff + soff
// land at lds + SIZE * l (SIZE 1 lands zero-extended in a dword, at 4 l).
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(rsrc_t rs, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma1(rsrc_t rs, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 1, voff, soff, 0, 0);
}

__device__ __forceinline__ int swz_f(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }

// (byte B of v) & m in one instruction (SDWA source byte select).
template <int B>
__device__ __forceinline__ uint32_t byte_and(uint32_t v, uint32_t m) {
  uint32_t r;
  if constexpr (B == 0)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD"
        : "=v"(r) : "v"(v), "v"(m));
  else if constexpr (B == 1)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
        : "=v"(r) : "v"(v), "v"(m));
  else if constexpr (B == 2)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
        : "=v"(r) : "v"(v), "v"(m));
  else
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
        : "=v"(r) : "v"(v), "v"(m));
  return r;
}

// Eight codes of one u32 (element e in nibble e) times the scale -> bf16x8.
// The byte offset of code c in the 16-float table is 4c: the low nibble of
// byte b sits at bits 2..5 of byte b of (p << 2), the high one at bits 2..5
// of byte b of (p >> 2).
template <int B>
__device__ __forceinline__ float lut_at(const uint8_t* lut, uint32_t v, uint32_t m) {
  return *reinterpret_cast<const float*>(lut + byte_and<B>(v, m));
}
__device__ __forceinline__ u32x4 deq8(uint32_t p, float sc, const uint8_t* lut, uint32_t m) {
  const uint32_t p4 = p << 2, p2 = p >> 2;
  return u32x4{pack_bf16x2(lut_at<0>(lut, p4, m) * sc, lut_at<0>(lut, p2, m) * sc),
               pack_bf16x2(lut_at<1>(lut, p4, m) * sc, lut_at<1>(lut, p2, m) * sc),
               pack_bf16x2(lut_at<2>(lut, p4, m) * sc, lut_at<2>(lut, p2, m) * sc),
               pack_bf16x2(lut_at<3>(lut, p4, m) * sc, lut_at<3>(lut, p2, m) * sc)};
}

template <bool DX>
__global__ __launch_bounds__(256, 1) void k_qgemm_big(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ scale2, const float* __restrict__ offset,
    const uint16_t* __restrict__ Act, const float* __restrict__ Vr,
    const uint16_t* __restrict__ Lr, int64_t M, int64_t N, int64_t K, int r, float s,
    uint16_t* __restrict__ Out, int tiles_c) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float s_lut[16];  // static LDS: a fixed address folds into ds_read
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint8_t* lut = reinterpret_cast<const uint8_t*>(s_lut);
  if (tid < 16) s_lut[tid] = as_f32(kNF4Bits[tid]);
  const uint32_t nib_mask = 0x3cu;

  const int tile_m = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / tiles_c));
  const int tile_c = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % tiles_c));
  const int64_t m0 = (int64_t)tile_m * BM;
  const int64_t c0 = (int64_t)tile_c * BN;
  const int64_t R = DX ? N : K;   // reduction length (row length of Act)
  const int64_t Cn = DX ? K : N;  // output columns
  const int steps = (int)((R + 63) / 64);
  const int64_t kblocks = K / 64;
  const float mu = *offset;

  // ---- activation DMA: instruction i of wave w covers tile rows 64w+8i..+7;
  // lane l -> row +l/8, stored unit l%8, so source chunk (l%8) ^ f(row).
  // Rows past M are clamped onto row M-1 (their outputs are not stored).
  const int64_t mrows = min((int64_t)BM, M - m0);
  const rsrc_t rsA = make_rs(Act + m0 * R, (uint32_t)(mrows * R * 2));
  uint32_t aoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * wave + 8 * i + (lane >> 3);
    const int64_t rc = min((int64_t)row, mrows - 1);
    const int c = (lane & 7) ^ swz_f(row);
    aoff[i] = (uint32_t)((rc * R + 8 * c) * 2);
  }
  // dX reduction tail: columns past the row end are clamped onto the row's
  // last chunk; they meet weight rows past N, which dequantize to zeros.
  auto dma_act = [&](int st, int stage) {
    uint8_t* dst = smem + OFF_A + stage * STAGE_B + wave * 8192;
    const uint32_t so = (uint32_t)st * 128u;
    if (!DX || (int64_t)st * 64 + 64 <= R) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dma16(rsA, aoff[i], so, dst + 1024 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 64 * wave + 8 * i + (lane >> 3);
        const int64_t k = (int64_t)st * 64 + 8 * ((lane & 7) ^ swz_f(row));
        const int64_t shift = min(k, R - 8) - k;
        dma16(rsA, (uint32_t)((int64_t)aoff[i] + 2 * shift), so, dst + 1024 * i);
      }
    }
  };

  // ---- weight DMA (this wave's 64 rows): codes as 2 x 1 KB, scale byte, scale2
  //   forward: row j = c0 + 64w + j, block column = step
  //   dX:      row j = 64*step + j, block column kbw
  const rsrc_t rsP = make_rs(packed, (uint32_t)(N * K / 2));
  const rsrc_t rsQ = make_rs(qscale, (uint32_t)(N * kblocks));
  const rsrc_t rsS = make_rs(scale2, (uint32_t)((N * kblocks + 255) / 256 * 4));
  const int64_t kbw = min((c0 + 64 * wave) / 64, kblocks - 1);
  uint32_t coff[2], qoff;
  if (!DX) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t n = min(c0 + 64 * wave + 32 * h + (lane >> 1), N - 1);
      coff[h] = (uint32_t)(n * (K / 2) + 16 * (lane & 1));
    }
    qoff = (uint32_t)(min(c0 + 64 * wave + lane, N - 1) * kblocks);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      coff[h] = (uint32_t)((32 * h + (lane >> 1)) * (K / 2) + kbw * 32 + 16 * (lane & 1));
    qoff = (uint32_t)(lane * kblocks + kbw);
  }
  auto dma_w = [&](int st, int stage) {
    uint8_t* cd = smem + OFF_C + (wave * 2 + stage) * 2048;
    uint8_t* qd = smem + OFF_Q + (wave * 2 + stage) * 256;
    uint8_t* sd = smem + OFF_S2 + (wave * 2 + stage) * 256;
    if (!DX) {
      dma16(rsP, coff[0], (uint32_t)st * 32u, cd);
      dma16(rsP, coff[1], (uint32_t)st * 32u, cd + 1024);
      dma1(rsQ, qoff, (uint32_t)st, qd);
      dma4(rsS, ((qoff + (uint32_t)st) >> 8) * 4, 0, sd);
    } else if ((int64_t)st * 64 + 64 <= N) {
      const uint32_t rb = (uint32_t)st * 64u;
      dma16(rsP, coff[0], rb * (uint32_t)(K / 2), cd);
      dma16(rsP, coff[1], rb * (uint32_t)(K / 2), cd + 1024);
      const uint32_t qb = rb * (uint32_t)kblocks;
      dma1(rsQ, qoff, qb, qd);
      dma4(rsS, ((qb + qoff) >> 8) * 4, 0, sd);
    } else {  // last, partial block of rows: clamp to row N-1
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t n = min((int64_t)st * 64 + 32 * h + (lane >> 1), N - 1);
        dma16(rsP, (uint32_t)(n * (K / 2) + kbw * 32 + 16 * (lane & 1)), 0, cd + 1024 * h);
      }
      const int64_t n = min((int64_t)st * 64 + lane, N - 1);
      const uint32_t qb = (uint32_t)(n * kblocks + kbw);
      dma1(rsQ, qb, 0, qd);
      dma4(rsS, (qb >> 8) * 4, 0, sd);
    }
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = f32x16{};

  // A fragment offsets (bytes) of substep ks: row 32i + l32, chunk 4g + ks
  int aoff_rd[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    aoff_rd[ks] = l32 * 128 + 16 * ((4 * g + ks) ^ swz_f(l32));
  auto read_a = [&](int stage, int ks, int i) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(smem + OFF_A + stage * STAGE_B +
                                                     aoff_rd[ks] + 4096 * i));
  };
  // dX: B fragments of substep ks from the private tile (transposed read)
  const int tr_off = [&] {
    const int i16 = lane & 15, grp = lane >> 4;
    return ((32 * g + (i16 >> 2)) * WLD + 16 * (grp & 1) + 4 * (i16 & 3)) * 2;
  }();
  auto read_b_tr = [&](int stage, int ks, bf16x8 (&b)[2]) {
    const uint8_t* w_st = smem + OFF_W + (wave * 2 + stage) * WSTAGE_B + tr_off + ks * 8 * WLD * 2;
    typedef short v4s __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(w_st + 64 * j));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(w_st + 64 * j + 4 * WLD * 2));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      b[j] = as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
    }
  };

  // forward B registers [parity][column subtile][ks]
  u32x4 bf[2][2][4];
  // Codes of the step being dequantized, as eight u32 words of eight codes:
  //   forward: word 4j + ks = codes 32g + 8ks .. +7 of row 32j + l%32;
  //   dX:      word w = codes 8w .. 8w+7 of row l.
  // Element chunk e (0..31) is byte e%4 of word e/4 (two codes).
  u32x4 wc[2];
  uint32_t q_raw[2];
  float s2_raw[2], wsc[2];
  auto fetch_codes = [&](int stage) {
    const uint8_t* cd = smem + OFF_C + (wave * 2 + stage) * 2048;
    const uint32_t* qd = reinterpret_cast<const uint32_t*>(smem + OFF_Q + (wave * 2 + stage) * 256);
    const float* sd = reinterpret_cast<const float*>(smem + OFF_S2 + (wave * 2 + stage) * 256);
    if (!DX) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 32 * j + l32;
        wc[j] = *reinterpret_cast<const u32x4*>(cd + row * 32 + 16 * g);
        q_raw[j] = qd[row];
        s2_raw[j] = sd[row];
      }
    } else {
      wc[0] = *reinterpret_cast<const u32x4*>(cd + lane * 32);
      wc[1] = *reinterpret_cast<const u32x4*>(cd + lane * 32 + 16);
      q_raw[0] = qd[lane];
      s2_raw[0] = sd[lane];
    }
  };
  auto make_scales = [&](int st) {
    if (!DX) {
      wsc[0] = dq_scale(q_raw[0] & 0xffu, s2_raw[0], mu);
      wsc[1] = dq_scale(q_raw[1] & 0xffu, s2_raw[1], mu);
    } else {
      const float sc = dq_scale(q_raw[0] & 0xffu, s2_raw[0], mu);
      wsc[0] = (int64_t)st * 64 + lane < N ? sc : 0.f;
    }
  };

  // ---- prologue: step 0's activations and weights, dequantized directly
  dma_act(0, 0);
  dma_w(0, 0);
  dma_w(min(1, steps - 1), 1);
  wait_dma();
  lds_barrier();
  fetch_codes(0);
  make_scales(0);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const u32x4 v = deq8(wc[w >> 2][w & 3], wsc[DX ? 0 : (w >> 2)], lut, nib_mask);
    if (!DX) {
      bf[0][w >> 2][w & 3] = v;
    } else {
      *reinterpret_cast<u32x4*>(smem + OFF_W + (wave * 2) * WSTAGE_B + lane * WLD * 2 + 16 * w) = v;
    }
  }
  lds_barrier();

  // ---- one step of parity P (stage P holds step st), as 32 chunks of two
  // MFMAs.  Chunk c = 8 ks + i multiplies row tile i of substep ks, reloads
  // that tile's A fragment for substep ks+1, issues the table reads of
  // element chunk c - 1 of the next step's weights and converts element chunk
  // c - 4 (read three chunks earlier).  sched_barrier keeps this order.
  constexpr int LUT_AT = 1, MUL_AT = 4;
  auto body = [&](auto par_t, int st) {
    constexpr int P = decltype(par_t)::value, Q = P ^ 1;
    const int nst = min(st + 1, steps - 1);
    bf16x8 a[8], b[2], b_nx[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = read_a(P, 0, i);
    if (DX) read_b_tr(P, 0, b);
    // the last step dequantizes a clamped repeat that nothing reads, so the
    // pipeline has no branch
    fetch_codes(Q);
    dma_act(nst, Q);
    dma_w(min(st + 2, steps - 1), P);
    uint32_t p4w[8], p2w[8], dq[4];
    float fl[4][2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 32 + MUL_AT; ++c) {
      if (c < 32) {
        const int ks = c >> 3, i = c & 7;
        bf16x8 b0, b1;
        if (!DX) {
          b0 = as_bf16x8(bf[P][0][ks]);
          b1 = as_bf16x8(bf[P][1][ks]);
        } else {
          b0 = b[0];
          b1 = b[1];
        }
        acc[i][0] = mfma32(b0, a[i], acc[i][0]);
        acc[i][1] = mfma32(b1, a[i], acc[i][1]);
        if (ks < 3) a[i] = read_a(P, ks + 1, i);
        if (DX && ks < 3 && i == 0) read_b_tr(P, ks + 1, b_nx);
        if (DX && ks < 3 && i == 7) {
          b[0] = b_nx[0];
          b[1] = b_nx[1];
        }
      }
      if (c == 0) make_scales(nst);
      const int el = c - LUT_AT;  // table reads of element chunk el
      if (el >= 0 && el < 32) {
        const int w = el >> 2, bb = el & 3;
        if (bb == 0) {
          const uint32_t word = wc[w >> 2][w & 3];
          p4w[w] = word << 2;
          p2w[w] = word >> 2;
        }
        float* f = fl[el & 3];
        switch (bb) {
          case 0: f[0] = lut_at<0>(lut, p4w[w], nib_mask); f[1] = lut_at<0>(lut, p2w[w], nib_mask); break;
          case 1: f[0] = lut_at<1>(lut, p4w[w], nib_mask); f[1] = lut_at<1>(lut, p2w[w], nib_mask); break;
          case 2: f[0] = lut_at<2>(lut, p4w[w], nib_mask); f[1] = lut_at<2>(lut, p2w[w], nib_mask); break;
          default: f[0] = lut_at<3>(lut, p4w[w], nib_mask); f[1] = lut_at<3>(lut, p2w[w], nib_mask); break;
        }
      }
      const int em = c - MUL_AT;  // conversion of element chunk em
      if (em >= 0 && em < 32) {
        const int w = em >> 2, bb = em & 3;
        const float sc = wsc[DX ? 0 : (w >> 2)];
        uint32_t v = pack_bf16x2(fl[em & 3][0] * sc, fl[em & 3][1] * sc);
        // keep the conversion here (not sunk next to the next step's MFMAs)
        asm volatile("" : "+v"(v));
        if (!DX) {
          bf[Q][w >> 2][w & 3][bb] = v;
        } else {
          dq[bb] = v;
          if (bb == 3)
            *reinterpret_cast<u32x4*>(smem + OFF_W + (wave * 2 + Q) * WSTAGE_B + lane * WLD * 2 +
                                      16 * w) = u32x4{dq[0], dq[1], dq[2], dq[3]};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_dma();
    lds_barrier();
  };
  using Z = std::integral_constant<int, 0>;
  using O = std::integral_constant<int, 1>;
  for (int st = 0; st < steps; st += 2) {
    body(Z{}, st);
    if (st + 1 < steps) body(O{}, st + 1);
  }

  // ---- LoRA term on the accumulators: acc += (s V) L^T in 16-wide steps.
  // Loads use clamped indices and a select, so that they issue together.
  for (int j0 = 0; j0 < r; j0 += 16) {
    const int jl = j0 + 8 * g;
    bf16x8 bh[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = min(c0 + 64 * wave + 32 * j + l32, Cn - 1);
      uint32_t e[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int jj = min(jl + q, r - 1);
        const uint32_t v = DX ? Lr[(int64_t)jj * K + col]  // A [r, K], column col
                              : Lr[col * r + jj];          // B [N, r], row col
        e[q] = jl + q < r ? v : 0u;
      }
      bh[j] = as_bf16x8(u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                              e[6] | (e[7] << 16)});
    }
    float vr[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = min(m0 + 32 * i + l32, M - 1);
#pragma unroll
      for (int q = 0; q < 8; ++q) vr[i][q] = Vr[m * r + min(jl + q, r - 1)];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = jl + 2 * q < r ? s * vr[i][2 * q] : 0.f;
        const float x1 = jl + 2 * q + 1 < r ? s * vr[i][2 * q + 1] : 0.f;
        h[q] = pack_bf16x2(x0, x1);
        l[q] = pack_bf16x2(x0 - bf16_lo(h[q]), x1 - bf16_hi(h[q]));
      }
      const bf16x8 ah = as_bf16x8(u32x4{h[0], h[1], h[2], h[3]});
      const bf16x8 al = as_bf16x8(u32x4{l[0], l[1], l[2], l[3]});
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = mfma32(bh[j], ah, acc[i][j]);
        acc[i][j] = mfma32(bh[j], al, acc[i][j]);
      }
    }
  }
  // ---- store.  Tile (i, j) is held transposed: lane l has output row
  // 32i + l%32 and columns 32j + 8q + 4(l/32) + e in register 4q + e.  A swap
  // of lanes 32..63 of one register with lanes 0..31 of another gives lane l
  // eight consecutive columns 32j + 16p + 8(l/32) .. +7 of pair p (q = 2p, 2p+1).
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + 32 * i + l32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
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
        const int64_t col = c0 + 64 * wave + 32 * j + 16 * pr + 8 * g;
        if (row < M && col < Cn)
          *reinterpret_cast<u32x4*>(Out + row * Cn + col) = u32x4{s0[0], s1[0], s0[1], s1[1]};
      }
    }
  }
}

template <bool DX>
hipError_t run_big(const WState& w, const uint16_t* Act, int64_t M, const float* V,
                   const uint16_t* L, int r, float s, uint16_t* Out, hipStream_t st) {
  auto kern = k_qgemm_big<DX>;
  const size_t lds = DX ? LDS_DX : LDS_FWD;
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const int64_t cols = DX ? w.cols : w.rows;
  const int64_t tm = (M + BM - 1) / BM, tc = (cols + BN - 1) / BN;
  hipLaunchKernelGGL(kern, dim3((unsigned)(tm * tc)), dim3(T), lds, st, w.packed, w.qscale,
                     w.scale2, w.offset, Act, V, L, M, w.rows, w.cols, r, s, Out, (int)tc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qgemm_big(bool dx, const WState& w, const uint16_t* Act, int64_t M,
                            const float* V, const uint16_t* L, int r, float s, uint16_t* Out,
                            hipStream_t st) {
  return dx ? run_big<true>(w, Act, M, V, L, r, s, Out, st)
            : run_big<false>(w, Act, M, V, L, r, s, Out, st);
}

}  // namespace qn
