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
// Data movement (no prefetch registers): global_load_lds (direct to LDS,
// lane l's 16 bytes land at base + 16 l) brings
//   - the activation tile of step s+1 (256 rows x 64, 16-byte chunks
//     XOR-swizzled by row so eight consecutive rows hit distinct banks) into
//     the other of two shared stages, and
//   - the weight codes of step s+2 of this wave's 64 weight rows (32 bytes
//     each) with their raw E4M3 scale byte and fp32 second-level scale into
//     the other of two wave-private code stages,
// all issued at the start of step s and drained before the barrier that ends
// it.  During step s a lane dequantizes the codes of step s+1 between the
// MFMAs:
//   forward: lane (row 32j + l%32, half l/32) turns 32 codes of each of its
//            two rows into the next step's B registers;
//   dX:      lane l turns row l's 64 codes into row l of a wave-private bf16
//            tile [n][k], read back as B fragments (eight consecutive n of one
//            column) with ds_read_b64_tr_b16, which gives lane i of each
//            16-lane group element i%4 of the chunks addressed by lanes
//            4q + i/4, q = 0..3.
// Reduction order inside a step, both operands: lane group g = lane/32 and
// substep ks take elements 32g + 8ks + 0..7 (activation chunk 4g + ks).
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

constexpr int BM = 256, BN = 256, T = 256;
constexpr int STAGE = BM * 64;  // bf16 per activation stage (32 KB)
constexpr int WLD = 72;         // private weight tile row (64 + 8 pad), dX
constexpr int WSTAGE = 64 * WLD;

// LDS map (bytes)
constexpr int OFF_A = 0;                         // 2 x 32 KB activation stages
constexpr int OFF_C = OFF_A + 2 * STAGE * 2;     // codes [wave][stage][64 rows][32 B]
constexpr int OFF_Q = OFF_C + 4 * 2 * 64 * 32;   // scale bytes [wave][stage][64] (u32 each)
constexpr int OFF_S2 = OFF_Q + 4 * 2 * 64 * 4;   // scale2 [wave][stage][64]
constexpr int OFF_LUT = OFF_S2 + 4 * 2 * 64 * 4; // 16 floats
constexpr int OFF_W = OFF_LUT + 64;              // dX: private tiles [wave][stage][64][WLD]
constexpr size_t LDS_FWD = OFF_W;
constexpr size_t LDS_DX = OFF_W + (size_t)4 * 2 * WSTAGE * 2;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_dma() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}
__device__ __forceinline__ void dma1(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 1, 0, 0);
}

// Eight codes of one u32 (element e in nibble e) times the scale -> bf16x8.
__device__ __forceinline__ u32x4 deq8(uint32_t p, float sc, const float* lut) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = lut[(p >> (4 * e)) & 15u] * sc;
  return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
}

// bf16 high part and bf16 remainder of s * V[m][j..j+7] (zero for j >= r).
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

__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

template <bool DX>
__global__ __launch_bounds__(256, 1) void k_qgemm_big(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ qscale,
    const float* __restrict__ scale2, const float* __restrict__ offset,
    const uint16_t* __restrict__ Act, const float* __restrict__ Vr,
    const uint16_t* __restrict__ Lr, int64_t M, int64_t N, int64_t K, int r, float s,
    uint16_t* __restrict__ Out, int tiles_c) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* lut = reinterpret_cast<float*>(smem + OFF_LUT);
  if (tid < 16) lut[tid] = as_f32(kNF4Bits[tid]);

  const int64_t m0 = (int64_t)(blockIdx.x / tiles_c) * BM;
  const int64_t c0 = (int64_t)(blockIdx.x % tiles_c) * BN;
  const int64_t R = DX ? N : K;   // reduction length (row length of Act)
  const int64_t Cn = DX ? K : N;  // output columns
  const int steps = (int)((R + 63) / 64);
  const int64_t kblocks = K / 64;
  const float mu = *offset;

  auto sA = [&](int st) { return reinterpret_cast<uint16_t*>(smem + OFF_A) + st * STAGE; };
  auto cst = [&](int st) { return smem + OFF_C + (wave * 2 + st) * 2048; };
  auto qst = [&](int st) { return reinterpret_cast<uint32_t*>(smem + OFF_Q + (wave * 2 + st) * 256); };
  auto s2st = [&](int st) { return reinterpret_cast<float*>(smem + OFF_S2 + (wave * 2 + st) * 256); };
  auto wtile = [&](int st) {
    return reinterpret_cast<uint16_t*>(smem + OFF_W) + (wave * 2 + st) * WSTAGE;
  };

  // ---- activation DMA: instruction i of wave w covers tile rows 64w+8i..+7;
  // lane l -> row +l/8, stored unit l%8, source chunk (l%8) ^ (row%8).
  const uint16_t* abase = Act + m0 * R;
  uint32_t aoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * wave + 8 * i + (lane >> 3);
    const int64_t rc = min((int64_t)row, M - 1 - m0);
    const int c = (lane & 7) ^ ((lane >> 3) & 7);
    aoff[i] = (uint32_t)(rc * R + 8 * c);
  }
  auto dma_act = [&](int st, int stage) {
    int shift = 0;
    if (DX) {  // reduction tail: clamp onto the row's last chunk (meets zero weights)
      const int c = (lane & 7) ^ ((lane >> 3) & 7);
      const int64_t k = (int64_t)st * 64 + 8 * c;
      shift = (int)(min(k, R - 8) - k);
    }
    const uint16_t* b = abase + (int64_t)st * 64 + shift;
    uint8_t* dst = reinterpret_cast<uint8_t*>(sA(stage)) + 64 * wave * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(b + aoff[i], dst + 1024 * i);
  };

  // ---- weight DMA (this wave's 64 rows): codes as 2 x 1 KB, scale byte, scale2
  //   forward: row j = c0 + 64w + j, block column = step
  //   dX:      row j = 64*step + j, block column kbw
  const int64_t kbw = min((c0 + 64 * wave) / 64, kblocks - 1);
  int64_t frow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) frow[h] = min(c0 + 64 * wave + 32 * h + (lane >> 1), N - 1);
  const int64_t frow_q = min(c0 + 64 * wave + lane, N - 1);
  auto dma_w = [&](int st, int stage) {
    uint8_t* cd = cst(stage);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t n = DX ? min((int64_t)st * 64 + 32 * h + (lane >> 1), N - 1) : frow[h];
      const int64_t kb = DX ? kbw : st;
      dma16(packed + n * (K / 2) + kb * 32 + 16 * (lane & 1), cd + 1024 * h);
    }
    const int64_t n = DX ? min((int64_t)st * 64 + lane, N - 1) : frow_q;
    const int64_t b = n * kblocks + (DX ? kbw : st);
    dma1(qscale + b, reinterpret_cast<uint8_t*>(qst(stage)));
    dma4(scale2 + (b >> 8), reinterpret_cast<uint8_t*>(s2st(stage)));
  };
  auto row_scale = [&](int stage, int row, bool valid) {
    const float sc = dq_scale(qst(stage)[row] & 0xffu, s2st(stage)[row], mu);
    return valid ? sc : 0.f;
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = f32x16{};

  auto read_a = [&](int stage, int ks, int i) {
    const int off = l32 * 64 + 8 * ((4 * g + ks) ^ (l32 & 7)) + 2048 * i;
    return as_bf16x8(*reinterpret_cast<const u32x4*>(sA(stage) + off));
  };
  // dX: B fragments of substep ks from the private tile (transposed read)
  auto read_b_tr = [&](int stage, int ks, bf16x8 (&b)[2]) {
    const uint16_t* w_st = wtile(stage);
    const int i16 = lane & 15, grp = lane >> 4;
    const int q = i16 >> 2, s4 = i16 & 3;
    const int nb = 32 * g + 8 * ks + q;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 32 * j + 16 * (grp & 1) + 4 * s4;
      typedef short v4s __attribute__((ext_vector_type(4)));
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(w_st + nb * WLD + col));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(w_st + (nb + 4) * WLD + col));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      b[j] = as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
    }
  };

  // forward B registers: [column subtile][ks], current and next step
  u32x4 bcur[2][4], bnext[2][4];
  // codes of the step being dequantized
  u32x4 wc[2];
  float wsc[2];
  auto fetch_codes = [&](int stage, int st) {
    const uint8_t* cd = cst(stage);
    if (!DX) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 32 * j + l32;
        wc[j] = *reinterpret_cast<const u32x4*>(cd + row * 32 + 16 * g);
        wsc[j] = row_scale(stage, row, true);
      }
    } else {
      wc[0] = *reinterpret_cast<const u32x4*>(cd + lane * 32);
      wc[1] = *reinterpret_cast<const u32x4*>(cd + lane * 32 + 16);
      wsc[0] = row_scale(stage, lane, (int64_t)st * 64 + lane < N);
    }
  };
  auto dequant_ks = [&](int ks, int wstage) {
    if (!DX) {
      bnext[0][ks] = deq8(wc[0][ks], wsc[0], lut);
      bnext[1][ks] = deq8(wc[1][ks], wsc[1], lut);
    } else {
      uint16_t* dst = wtile(wstage) + lane * WLD;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int d = 2 * ks + h;
        *reinterpret_cast<u32x4*>(dst + 8 * d) = deq8(wc[d >> 2][d & 3], wsc[0], lut);
      }
    }
  };

  // ---- prologue
  dma_act(0, 0);
  dma_w(0, 0);
  dma_w(min(1, steps - 1), 1);
  wait_dma();
  lds_barrier();
  fetch_codes(0, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) dequant_ks(ks, 0);
  if (!DX) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bcur[0][ks] = bnext[0][ks];
      bcur[1][ks] = bnext[1][ks];
    }
  }
  lds_barrier();

  for (int st = 0; st < steps; ++st) {
    const int cur = st & 1, nxt = cur ^ 1;
    const bool more = st + 1 < steps;
    // prefetch: activation step st+1, codes of step st+2 (clamped at the end)
    dma_act(min(st + 1, steps - 1), nxt);
    dma_w(min(st + 2, steps - 1), cur);
    if (more) fetch_codes(nxt, st + 1);
    bf16x8 a[8], b[2], b_nx[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = read_a(cur, 0, i);
    if (!DX) {
      b[0] = as_bf16x8(bcur[0][0]);
      b[1] = as_bf16x8(bcur[1][0]);
    } else {
      read_b_tr(cur, 0, b);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) {
        if (!DX) {
          b_nx[0] = as_bf16x8(bcur[0][ks + 1]);
          b_nx[1] = as_bf16x8(bcur[1][ks + 1]);
        } else {
          read_b_tr(cur, ks + 1, b_nx);
        }
      }
      // each A register is reloaded for the next substep right after its
      // two MFMAs have consumed it
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i][0] = mfma32(a[i], b[0], acc[i][0]);
        acc[i][1] = mfma32(a[i], b[1], acc[i][1]);
        if (ks < 3) a[i] = read_a(cur, ks + 1, i);
      }
      if (more) dequant_ks(ks, nxt);
      if (ks < 3) {
        b[0] = b_nx[0];
        b[1] = b_nx[1];
      }
    }
    if (!DX && more) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bcur[0][ks] = bnext[0][ks];
        bcur[1][ks] = bnext[1][ks];
      }
    }
    wait_dma();
    lds_barrier();
  }

  // ---- LoRA term on the accumulators: acc += (s V) L^T in 16-wide steps
  for (int j0 = 0; j0 < r; j0 += 16) {
    const int jl = j0 + 8 * g;
    bf16x8 bh[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = min(c0 + 64 * wave + 32 * j + l32, Cn - 1);
      uint32_t w4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jj = jl + 2 * q;
        uint32_t lo, hi;
        if (!DX) {  // B [N, r]
          lo = jj < r ? Lr[col * r + jj] : 0u;
          hi = jj + 1 < r ? Lr[col * r + jj + 1] : 0u;
        } else {    // A [r, K], column col
          lo = jj < r ? Lr[(int64_t)jj * K + col] : 0u;
          hi = jj + 1 < r ? Lr[(int64_t)(jj + 1) * K + col] : 0u;
        }
        w4[q] = lo | (hi << 16);
      }
      bh[j] = as_bf16x8(u32x4{w4[0], w4[1], w4[2], w4[3]});
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = min(m0 + 32 * i + l32, M - 1);
      bf16x8 ah, al;
      lora_rows(Vr, m, r, jl, s, ah, al);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = mfma32(ah, bh[j], acc[i][j]);
        acc[i][j] = mfma32(al, bh[j], acc[i][j]);
      }
    }
  }
  // ---- store: lane holds column lane%32 of each 32x32 tile
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = c0 + 64 * wave + 32 * j + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + 32 * i + acc_row(v, lane);
        if (row < M && col < Cn)
          Out[row * Cn + col] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.f) & 0xffffu);
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
