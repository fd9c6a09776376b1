// NF4 block-64 quantisation with double quantisation, and dequantisation,
// for gfx950.
//
// What is computed (pages: "QLoRA: NF4 storage, gradients and local
// integration", section "Exact CPU teaching quantizer and adapter gradient
// path"; "QLoRA Deep Dive: 4-bit NormalFloat & Double Quantization
// Internals", section "2. Squeezing More Memory: Double Quantization (DQ)"):
//   blocks of 64 consecutive weights (flattened row-major, tail zero-padded),
//   s_b = max|w|, n = RN32(w / s_b) (a zero block divides by 1),
//   code = nearest NF4 level, ties to the lower code, two codes per byte with
//   the even element in the low nibble;
//   mu = mean of all s_b (fixed fp64 stride-halving tree), d_b = s_b - mu,
//   per 256 scales C2 = max|d_b|, s2 = C2 / 448, q_b = E4M3FN(d_b / s2).
//   dequant: s'_b = fmaf(e4m3(q_b), s2, mu), w' = L[c] * s'_b.
//
// Exact code search without a division.  code(w) = #{k : RN32(w/s) > t_k}
// where t_k is the largest fp32 not above the k-th midpoint of adjacent
// levels (a value that lands exactly on a midpoint is not above it, so ties
// go to the lower code).  RN32(x) > t_k holds exactly when x exceeds the
// midpoint mu_k = t_k + h_k between t_k and the next fp32 up (h_k is half
// that gap, a power of two): a quotient of two fp32 numbers is never exactly
// such a midpoint, so there is no tie to break.  x > mu_k is w > mu_k * s,
// decided in fp32 as fma(-t_k, s, w) > h_k * s: h_k * s is exact, and
// wherever w is near t_k s the difference w - t_k s is a multiple of
// ulp(t_k) ulp(s) no larger than a few ulp(w), so it fits in 24 bits and the
// fma returns it exactly; elsewhere rounding keeps its order against the
// representable h_k * s.  Both need every product clear of the subnormal
// range, which holds for s >= 2^-90; a wave holding a smaller block scale
// takes the same comparison in fp64 (mu_k has 25 significant bits and s 24,
// so mu_k * s is exact there).  Which t_k to test is found from an
// approximate quotient q = w * rcp(s) and a table of 65 buckets of width
// 1/32 on [-1, 1]: every bucket holds at most one t_k and every t_k lies at
// least 1.6e-3 from a bucket edge, far beyond the error of q, so the bucket
// is right even when q and the true quotient straddle an edge.  The table
// holds, per bucket, t_k (4.0 when the bucket holds no threshold: then
// h_k = 0) and the bits of h_k with the bucket's lower code c0 in their four
// low bits (a power of two has no mantissa bits), in 16 copies (bucket j,
// copy c at entry 16 j + c; lane l reads copy l % 16) so that the 16 lanes a
// 64-bit LDS read serves per cycle never collide.
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {


__device__ __forceinline__ float f32_next_up(float t) {
  uint32_t b = as_u32(t);
  return as_f32(t > 0.f ? b + 1u : b - 1u);
}
__device__ __forceinline__ float f32_next_down(float t) {
  uint32_t b = as_u32(t);
  return as_f32(t > 0.f ? b - 1u : b + 1u);
}

// Entry j covers quotients in [(j-32)/32, (j-31)/32): t (4.0: the bucket
// holds no threshold) in the low word, h's bits with c0, the code of the
// bucket's lower part, in their four low bits in the high word.
// NF4: the sixteen levels over [-1, 1].  FP4: the eight magnitudes over
// [0, 1] (entries j >= 32; the sign is taken apart).
template <int CB>
__device__ uint64_t code_lut_entry(int j) {
  const double lo = (double)(j - 32) * 0.03125, hi = (double)(j - 31) * 0.03125;
  uint32_t c0 = 0;
  float tb = 4.0f, h = 0.0f;
  constexpr int NT = CB == kCodeFP4 ? 7 : 15;  // thresholds between adjacent levels
  for (int k = 0; k < NT; ++k) {
    // exact midpoint of two adjacent levels, then its round-down to fp32
    double m = ((double)as_f32(level_bits(CB, k)) + (double)as_f32(level_bits(CB, k + 1))) * 0.5;
    float t = (float)m;
    if ((double)t > m) t = f32_next_down(t);
    if ((double)t < lo) {
      ++c0;
    } else if ((double)t < hi) {
      tb = t;
      h = (float)(((double)f32_next_up(t) - (double)t) * 0.5);  // exact: a power of two
    }
  }
  return (uint64_t)as_u32(tb) | (uint64_t)(as_u32(h) | c0) << 32;
}

// Max of v over each row of 16 lanes (DPP: xor 1, xor 2, half-row mirror,
// row mirror; every source lane exists, and 0 is the identity of the
// unsigned max, so each step can be one max with a DPP operand).
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));
  return v;
}

// The code of w in bucket entry e against block scale s: c0 + [w > mu s].
// fp32 form (every block scale of the wave >= 2^-90), rs32 ~ 32 / s:
__device__ __forceinline__ uint32_t bucket_code32(float w, float rs32, float s, const uint64_t* lc,
                                                  int lo) {
  int idx = (int)__builtin_fmaf(w, rs32, 32.0f);
  idx = min(max(idx, lo), 64);
  const uint64_t e = lc[16 * idx];
  const uint32_t hw = (uint32_t)(e >> 32);
  const float r = __builtin_fmaf(-as_f32((uint32_t)e), s, w);
  return (hw & 15u) + (r > as_f32(hw & ~15u) * s ? 1u : 0u);
}
// fp64 form (any positive s, subnormal included: 32 / s overflows fp32 for
// those); mu = t + h is exact in fp64.
__device__ __forceinline__ uint32_t bucket_code64(float w, double rs32, double s64,
                                                  const uint64_t* lc, int lo) {
  int idx = (int)__builtin_fma((double)w, rs32, 32.0);
  idx = min(max(idx, lo), 64);
  const uint64_t e = lc[16 * idx];
  const uint32_t hw = (uint32_t)(e >> 32);
  const double mu = (double)as_f32((uint32_t)e) + (double)as_f32(hw & ~15u);
  return (hw & 15u) + ((double)w > mu * s64 ? 1u : 0u);
}

// NF4: the bucket of w over [-1, 1].  FP4: the sign of w, and the magnitude
// code of |w| from the magnitudes' buckets (entries 32..64).
template <int CB, bool F32>
__device__ __forceinline__ uint32_t code_of(float w, float rs32, float s, double rs64, double s64,
                                            const uint64_t* lc) {
  const float a = CB == kCodeFP4 ? __builtin_fabsf(w) : w;
  const int lo = CB == kCodeFP4 ? 32 : 0;
  const uint32_t m = F32 ? bucket_code32(a, rs32, s, lc, lo) : bucket_code64(a, rs64, s64, lc, lo);
  if constexpr (CB == kCodeFP4)
    return (as_u32(w) >> 28 & 8u) | m;
  else
    return m;
}

template <int CB, bool F32>
__device__ __forceinline__ uint32_t codes4(const float4& v, float s, const uint64_t* lc) {
  float rs32 = 0.f, sf = 1.f;
  double rs64 = 0.0, s64 = 1.0;
  if (F32) {
    sf = s > 0.f ? s : 1.0f;  // a zero block divides by 1
    rs32 = __builtin_amdgcn_rcpf(sf * 0.03125f);
  } else {
    s64 = s > 0.f ? (double)s : 1.0;
    rs64 = 32.0 * __builtin_amdgcn_rcp(s64);
  }
  const uint32_t c0 = code_of<CB, F32>(v.x, rs32, sf, rs64, s64, lc);
  const uint32_t c1 = code_of<CB, F32>(v.y, rs32, sf, rs64, s64, lc);
  const uint32_t c2 = code_of<CB, F32>(v.z, rs32, sf, rs64, s64, lc);
  const uint32_t c3 = code_of<CB, F32>(v.w, rs32, sf, rs64, s64, lc);
  return c0 | (c1 << 4) | (c2 << 8) | (c3 << 12);
}

// Pass 1.  One workgroup per group of 256 blocks (16384 weights); wave w
// owns blocks 64w..64w+63 of the group, and at step j its 64 lanes read
// 1 KB: four blocks, 16 lanes x float4 per block.  The body is instantiated
// for whole groups (every load unconditional, QD in flight at a time) and
// for the tail group (element-wise bounds); the kernel branches once, around
// the whole body, so no loaded value meets a branch join (which would make
// the compiler wait for every load there).  In whole groups the codes gather
// in LDS and leave as 16-byte pieces, and the 256 block scales leave in one
// coalesced store at the end (2-byte and 4-lane stores per step cost more
// than the code search).
// loads in flight per thread in the block pass: all sixteen at once put the
// whole 64 MB in the memory queues together and delay the first data; three
// measured best (21.7-22.0 us at 4096x4096 against 22.6-23.5 for sixteen,
// 22.5-23.2 for four, 22.6 for two)
constexpr int QD = 3;
template <bool FULL, int CB>
__device__ __forceinline__ void quant_group(const float* __restrict__ W, int64_t n, int64_t nb,
                                            uint8_t* __restrict__ packed,
                                            float* __restrict__ absmax, double* tree,
                                            const uint64_t* lut, int* s_bad, uint16_t* codes) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t g = blockIdx.x;
  const int64_t e_wave = (g * kGroup + wave * 64) * kBlock;
  float4 v[16];
  auto load_j = [&](int j) {
    const int64_t e = e_wave + j * 256 + lane * 4;
    if (FULL) {
      // streamed once: a non-temporal load keeps the weights from displacing
      // useful lines in L2 and the MALL (15.7 against 18.4 us at 4096x4096)
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(W + e));
      v[j] = make_float4(t.x, t.y, t.z, t.w);
    } else {
      v[j].x = e + 0 < n ? W[e + 0] : 0.f;
      v[j].y = e + 1 < n ? W[e + 1] : 0.f;
      v[j].z = e + 2 < n ? W[e + 2] : 0.f;
      v[j].w = e + 3 < n ? W[e + 3] : 0.f;
    }
  };
#pragma unroll
  for (int j = 0; j < QD; ++j) load_j(j);
  // code table ready (LDS-only barrier: the loads above stay in flight)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const uint64_t* lc = lut + (lane & 15);
  uint32_t any_bad = 0;
  float bs[16];  // the block scale of step j (row lane & 15 == 0 stores them)
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j + QD < 16) load_j(j + QD);  // QD loads stay in flight
    __builtin_amdgcn_sched_barrier(0);  // (not hoisted: that would issue all sixteen at once)
    const uint32_t a0 = as_u32(v[j].x) & 0x7fffffffu, a1 = as_u32(v[j].y) & 0x7fffffffu;
    const uint32_t a2 = as_u32(v[j].z) & 0x7fffffffu, a3 = as_u32(v[j].w) & 0x7fffffffu;
    // |w| bit patterns order like the values; NaN/Inf sort above all finite
    const uint32_t m = row16_max(max(max(a0, a1), max(a2, a3)));
    any_bad |= m >= 0x7f800000u ? 1u : 0u;
    const float s = as_f32(m);
    bs[j] = s;
    const int slot = wave * 64 + 4 * j + (lane >> 4);
    const int64_t b = g * kGroup + slot;
    // a zero block counts as scale 1 (so does NaN: a block with a non-finite
    // weight only sets the flag, its codes need only stay in range)
    const uint16_t c16 = (uint16_t)(__all(!(s > 0.f) || s >= 0x1p-90f)
                                        ? codes4<CB, true>(v[j], s, lc)
                                        : codes4<CB, false>(v[j], s, lc));
    if (FULL) {
      codes[(wave * 16 + j) * 64 + lane] = c16;
    } else if (b < nb) {
      const int64_t e = e_wave + j * 256 + lane * 4;
      *reinterpret_cast<uint16_t*>(packed + e / 2) = c16;
    }
  }
  if (any_bad) *s_bad = 1;
  if ((lane & 15) == 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int slot = wave * 64 + 4 * j + (lane >> 4);
      const int64_t b = g * kGroup + slot;
      if (!FULL && b < nb) absmax[b] = bs[j];
      tree[slot] = (FULL || b < nb) ? (double)bs[j] : 0.0;
    }
  }
  if (FULL) {
    // the wave's 16 x 128 contiguous code bytes leave as 16-byte pieces (its
    // own LDS writes above are visible to its reads: a wave's LDS accesses
    // execute in order)
    const uint8_t* cw = reinterpret_cast<const uint8_t*>(codes + wave * 16 * 64);
    uint8_t* dst = packed + e_wave / 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = lane + 64 * h;  // 16-byte piece: iteration c / 8, offset 16 (c % 8)
      *reinterpret_cast<u32x4*>(dst + (c >> 3) * 128 + 16 * (c & 7)) =
          *reinterpret_cast<const u32x4*>(cw + 16 * c);
    }
  }
}

template <int CB>
__global__ __launch_bounds__(256) void k_quant_blocks(
    const float* __restrict__ W, int64_t n, int64_t nb, uint8_t* __restrict__ packed,
    float* __restrict__ absmax, double* __restrict__ part, int* __restrict__ bad) {
  __shared__ uint64_t lut[65 * 16];
  __shared__ double tree[kGroup];
  __shared__ __attribute__((aligned(16))) uint16_t codes[4 * 16 * 64];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid < 65) {
    const uint64_t e = code_lut_entry<CB>(tid);
#pragma unroll
    for (int c = 0; c < 16; ++c) lut[16 * tid + c] = e;
  }
  if (tid == 0) s_bad = 0;
  const int64_t g = blockIdx.x;
  const bool full = (g + 1) * (int64_t)(kGroup * kBlock) <= n;
  if (full)
    quant_group<true, CB>(W, n, nb, packed, absmax, tree, lut, &s_bad, codes);
  else
    quant_group<false, CB>(W, n, nb, packed, absmax, tree, lut, &s_bad, codes);
  // (LDS-only barriers from here: the code stores stay in flight)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // a whole group's 256 block scales leave in one coalesced store
  if (full) absmax[g * kGroup + tid] = (float)tree[tid];
  // fixed-order fp64 partial sum of this group's 256 scale slots
  for (int h = kGroup / 2; h >= 1; h >>= 1) {
    if (tid < h) tree[tid] += tree[tid + h];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (tid == 0) {
    part[g] = tree[0];
    bad[g] = s_bad;  // every group writes its flag: no clearing pass needed
  }
}

// Pass 2.  mu = RN32(S / nb), S = stride-halving tree over the group partials
// zero-padded to len (a power of two).  One workgroup; the leading levels of
// a long tree run in global memory, the last 2048 in LDS.
__global__ __launch_bounds__(1024) void k_quant_mean(double* __restrict__ part, int64_t ng,
                                                     int64_t len, int64_t nb,
                                                     float* __restrict__ offset,
                                                     const int* __restrict__ bad,
                                                     int* __restrict__ flag) {
  __shared__ double t[2048];
  __shared__ int s_any;
  const int tid = threadIdx.x;
  if (tid == 0) s_any = 0;
  __syncthreads();
  {  // any group with a non-finite weight
    int any = 0;
    for (int64_t j = tid; j < ng; j += 1024) any |= bad[j];
    if (any) s_any = 1;
  }
  int64_t h = len / 2;
  for (; h >= 2048; h /= 2) {
    for (int64_t j = tid; j < h; j += 1024) {
      const double a = j < ng ? part[j] : 0.0;
      const double b = j + h < ng ? part[j + h] : 0.0;
      part[j] = a + b;
    }
    __threadfence();
    __syncthreads();
  }
  const int64_t active = (len >= 2048) ? 2048 : len;  // == 2h unless len == 1
  const int64_t valid = ng < active ? ng : active;
  for (int64_t i = tid; i < active; i += 1024) t[i] = i < valid ? part[i] : 0.0;
  __syncthreads();
  for (h = active / 2; h >= 1; h /= 2) {
    for (int64_t j = tid; j < h; j += 1024) t[j] += t[j + h];
    __syncthreads();
  }
  if (tid == 0) {
    *offset = (float)(t[0] / (double)nb);
    *flag = s_any;
  }
}

// Pass 3.  One workgroup per group: d_b, C2, s2 and the E4M3 codes.  With
// FUSED, passes 2 and 3 share the launch: every workgroup first forms the
// same mu itself (the stride-halving tree over the group partials zero-padded
// to len: levels of 256 entries and more inside each thread, then LDS, then
// lane shuffles, with the same additions in the same order as
// pass 2; up to 2048 groups, NQ partials per thread: 4 up to 1024 groups, 8
// above), and workgroup 0 writes offset and the non-finite flag.  (Loading 8
// per thread at 1024 groups, half of them the last partial again, cost 0.5 us
// per call.)
template <bool FUSED, int NQ>
__global__ __launch_bounds__(256) void k_quant_dq(const float* __restrict__ absmax, int64_t nb,
                                                  float* __restrict__ offset,
                                                  uint8_t* __restrict__ qscale,
                                                  float* __restrict__ scale2,
                                                  const double* __restrict__ part, int64_t ng,
                                                  int64_t len, const int* __restrict__ bad,
                                                  int* __restrict__ flag) {
  __shared__ float red[4];
  __shared__ double t[128];
  __shared__ int s_any;
  const int tid = threadIdx.x;
  // this thread's block scale, loaded before the mean's tree (whose barriers
  // would otherwise keep the load behind it)
  const int64_t b = (int64_t)blockIdx.x * kGroup + tid;
  const float sb = b < nb ? absmax[b] : 0.f;
  // workgroup 0 also reads the groups' non-finite flags up front (ng <= 256 NQ
  // when FUSED: at most NQ per thread)
  // (every load below is unconditional, at an index clamped into range, and
  // the values past the end are dropped afterwards: a load under its own
  // condition gets its own branch and a wait of its own, which put eight
  // round trips in series)
  int any_bad = 0;
  if (FUSED && blockIdx.x == 0) {
    int fl[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) fl[q] = bad[min((int64_t)tid + 256 * q, ng - 1)];
#pragma unroll
    for (int q = 0; q < NQ; ++q) any_bad |= fl[q];
  }
  float mu;
  if constexpr (FUSED) {
    // thread tid holds entries tid + 256 q of the LDS stage (zero past it);
    // levels h >= 256 pair entries of one thread, h = 128 and 64 go through
    // LDS, h <= 32 through lane shuffles: t[j] + t[j + h] at every level,
    // as in pass 2
    // len <= 256 NQ here: one partial per stage entry
    const int64_t active = len;
    double v[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) v[q] = part[min((int64_t)tid + 256 * q, ng - 1)];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t j = tid + 256 * q;
      if (!(256 * q < active && j < ng)) v[q] = 0.0;
    }
    int64_t h = active / 2;
    for (; h >= 256; h /= 2) {
      const int64_t qh = h / 256;
#pragma unroll
      for (int q = 0; q < NQ / 2; ++q)
        if (q < qh) v[q] += v[q + qh];
    }
    double x = v[0];
    for (; h >= 64; h /= 2) {
      if (tid >= h && tid < 2 * h) t[tid - h] = x;
      __syncthreads();
      if (tid < h) x += t[tid];
      __syncthreads();
    }
    for (; h >= 1; h /= 2) {
      const double y = __shfl_down(x, (unsigned)h);
      if (tid < h) x += y;
    }
    if (tid == 0) t[0] = x;
    __syncthreads();
    mu = (float)(t[0] / (double)nb);
    if (blockIdx.x == 0) {  // workgroup 0: offset and the non-finite flag
      if (tid == 0) s_any = 0;
      __syncthreads();
      if (any_bad) s_any = 1;
      __syncthreads();
      if (tid == 0) {
        *offset = mu;
        *flag = s_any;
      }
    }
  } else {
    mu = *offset;
  }
  const float d = (b < nb) ? sb - mu : 0.f;
  float a = __builtin_fabsf(d);
  for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if ((tid & 63) == 0) red[tid >> 6] = a;
  __syncthreads();
  const float c2 = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s2 = c2 / kE4M3Max;
  const float x = (s2 > 0.f) ? d / s2 : 0.f;
  if (b < nb) qscale[b] = (uint8_t)f32_to_e4m3(x);
  if (tid == 0) scale2[blockIdx.x] = s2;
}

hipError_t launch_quantize(const float* W, int64_t n, uint8_t* packed, uint8_t* qscale,
                           float* scale2, float* offset, float* ws_absmax, double* ws_part,
                           int64_t part_len, int* ws_bad, int* flag, hipStream_t st, int codebook,
                           float* absmax_out, float* ws_offset) {
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kGroup - 1) / kGroup;
  float* am = absmax_out ? absmax_out : ws_absmax;
  if (codebook == kCodeFP4)
    hipLaunchKernelGGL(k_quant_blocks<kCodeFP4>, dim3((unsigned)ng), dim3(256), 0, st, W, n, nb,
                       packed, am, ws_part, ws_bad);
  else
    hipLaunchKernelGGL(k_quant_blocks<kCodeNF4>, dim3((unsigned)ng), dim3(256), 0, st, W, n, nb,
                       packed, am, ws_part, ws_bad);
  if (absmax_out) {
    // double quantization off: the block scales are the state; one small
    // launch reduces the groups' non-finite flags (the mean it also forms
    // goes to the workspace)
    hipLaunchKernelGGL(k_quant_mean, dim3(1), dim3(1024), 0, st, ws_part, ng, part_len, nb,
                       ws_offset, ws_bad, flag);
    return hipGetLastError();
  }
  if (part_len <= 1024) {
    // the mean inside the scale pass: one launch fewer
    hipLaunchKernelGGL((k_quant_dq<true, 4>), dim3((unsigned)ng), dim3(256), 0, st, ws_absmax, nb,
                       offset, qscale, scale2, ws_part, ng, part_len, ws_bad, flag);
  } else if (part_len <= 2048) {
    hipLaunchKernelGGL((k_quant_dq<true, 8>), dim3((unsigned)ng), dim3(256), 0, st, ws_absmax, nb,
                       offset, qscale, scale2, ws_part, ng, part_len, ws_bad, flag);
  } else {
    hipLaunchKernelGGL(k_quant_mean, dim3(1), dim3(1024), 0, st, ws_part, ng, part_len, nb,
                       offset, ws_bad, flag);
    hipLaunchKernelGGL((k_quant_dq<false, 1>), dim3((unsigned)ng), dim3(256), 0, st, ws_absmax, nb,
                       offset, qscale, scale2, ws_part, ng, part_len, ws_bad, flag);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantisation.  Thread-chunk c covers CH consecutive weights (CH = 8 for
// bf16 output: one u32 of codes in, 16 B out; CH = 4 for fp32: one u16 in,
// 16 B out).  A workgroup's 256 threads take 256 consecutive chunks, so
// loads and stores are contiguous; each thread does UNROLL chunks, all of
// whose loads (codes, scale code, second-level scale) go out before the first
// is used.  Whole workgroups (every chunk in range) take unconditional
// loads; only the last workgroup checks bounds, and the kernel branches once
// around the whole body, so no loaded value meets a branch join.
template <bool BF16, bool FULL, bool ABS, bool NT>
__device__ __forceinline__ void dequant_chunks(const uint8_t* __restrict__ packed,
                                               const uint8_t* __restrict__ qscale,
                                               const float* __restrict__ scale2,
                                               const float* __restrict__ offset,
                                               const float* __restrict__ absmax, int64_t n,
                                               void* __restrict__ out, const float* lut) {
  constexpr int CH = BF16 ? 8 : 4;
  constexpr int UNROLL = 4;
  const int64_t nchunk = (n + CH - 1) / CH;
  const int64_t c_first = (int64_t)blockIdx.x * 256 * UNROLL + threadIdx.x;
  uint32_t p[UNROLL], qb[UNROLL];
  float s2[UNROLL];
#pragma unroll
  for (int i = 0; i < UNROLL; ++i) {
    const int64_t c = FULL ? c_first + i * 256 : min(c_first + i * 256, nchunk - 1);
    if (BF16)
      p[i] = *reinterpret_cast<const uint32_t*>(packed + c * 4);
    else
      p[i] = *reinterpret_cast<const uint16_t*>(packed + c * 2);
    const int64_t b = c * CH / kBlock;
    if (ABS) {
      s2[i] = absmax[b];  // double quantization off: the block scale itself
    } else {
      qb[i] = qscale[b];
      s2[i] = scale2[b / kGroup];
    }
  }
  const float mu = ABS ? 0.f : *offset;
  __builtin_amdgcn_sched_barrier(0);  // every load issues before the first use
  // the level table is ready (LDS-only barrier: the loads stay in flight)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < UNROLL; ++i) {
    const int64_t c = c_first + i * 256;
    if (!FULL && c >= nchunk) continue;
    const float sc = ABS ? s2[i] : dq_scale(qb[i], s2[i], mu);
    float w[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) w[k] = lut[(p[i] >> (4 * k)) & 15u] * sc;
    const int64_t e = c * CH;
    if (BF16) {
      uint16_t* o = reinterpret_cast<uint16_t*>(out) + e;
      if (FULL || e + CH <= n) {
        u32x4 q = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
                   pack_bf16x2(w[6], w[7])};
        if (NT)
          __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(o));
        else
          *reinterpret_cast<u32x4*>(o) = q;
      } else {
        for (int k = 0; k < CH && e + k < n; ++k)
          o[k] = (uint16_t)(pack_bf16x2(w[k], 0.f) & 0xffffu);
      }
    } else {
      float* o = reinterpret_cast<float*>(out) + e;
      if (FULL || e + CH <= n) {
        const f32x4 q = {w[0], w[1], w[2], w[3]};
        if (NT)
          __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(o));
        else
          *reinterpret_cast<f32x4*>(o) = q;
      } else {
        for (int k = 0; k < CH && e + k < n; ++k) o[k] = w[k];
      }
    }
  }
}

// NT: non-temporal stores, for a copy that is written once and not read
// back soon (the caller's nf4_dequantize: 8.3 against 11.4 us at 4096x4096
// bf16, 13.0 against 17.3 fp32); the linear calls' own bf16 copy of W',
// which the GEMM reads next, keeps ordinary stores so that it stays in the
// memory-side cache.
template <bool BF16, int CB, bool ABS, bool NT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ packed,
                                                 const uint8_t* __restrict__ qscale,
                                                 const float* __restrict__ scale2,
                                                 const float* __restrict__ offset,
                                                 const float* __restrict__ absmax, int64_t n,
                                                 void* __restrict__ out, SliceSum ss,
                                                 unsigned dq_blocks) {
  constexpr int CH = BF16 ? 8 : 4;
  constexpr int UNROLL = 4;
  if (blockIdx.x >= dq_blocks) {
    // workgroups past the weight: a slice sum from the preceding launch
    const int64_t i = (int64_t)(blockIdx.x - dq_blocks) * blockDim.x + threadIdx.x;
    if (i < ss.count) ss.out[i] = slice_sum(ss.part, ss.count, ss.S, i);
    return;
  }
  __shared__ float lut[16];
  if (threadIdx.x < 16) {  // from immediates: no load that the first weight loads would queue behind
    uint32_t v = level_bits(CB, 0);
#pragma unroll
    for (int k = 1; k < 16; ++k) v = threadIdx.x == k ? level_bits(CB, k) : v;
    lut[threadIdx.x] = as_f32(v);
  }
  const int64_t last_elem = ((int64_t)blockIdx.x + 1) * 256 * UNROLL * CH;  // one past
  if (last_elem <= n)
    dequant_chunks<BF16, true, ABS, NT>(packed, qscale, scale2, offset, absmax, n, out, lut);
  else
    dequant_chunks<BF16, false, ABS, NT>(packed, qscale, scale2, offset, absmax, n, out, lut);
}

template <bool BF16, int CB, bool ABS>
void launch_dq(dim3 grid, hipStream_t st, const uint8_t* packed, const ScaleSrc& sc,
                      int64_t n, void* out, const SliceSum& ss, unsigned dq_blocks, bool nt) {
  if (nt)
    hipLaunchKernelGGL((k_dequant<BF16, CB, ABS, true>), grid, dim3(256), 0, st, packed,
                       sc.qscale, sc.scale2, sc.offset, sc.absmax, n, out, ss, dq_blocks);
  else
    hipLaunchKernelGGL((k_dequant<BF16, CB, ABS, false>), grid, dim3(256), 0, st, packed,
                       sc.qscale, sc.scale2, sc.offset, sc.absmax, n, out, ss, dq_blocks);
}

hipError_t launch_dequant(const uint8_t* packed, const uint8_t* qscale, const float* scale2,
                          const float* offset, int64_t n, bool bf16, void* out, hipStream_t st,
                          const SliceSum& ss, int codebook, const float* absmax, bool nt) {
  const int CH = bf16 ? 8 : 4;
  const int64_t nchunk = (n + CH - 1) / CH;
  const int64_t per_wg = 256 * 4;
  const unsigned grid = (unsigned)((nchunk + per_wg - 1) / per_wg);
  const unsigned extra = ss.count > 0 ? (unsigned)((ss.count + 255) / 256) : 0u;
  const dim3 g(grid + extra);
  const ScaleSrc sc{qscale, scale2, offset, absmax};
  const bool fp4 = codebook == kCodeFP4, abs = absmax != nullptr;
  if (bf16) {
    if (fp4)
      abs ? launch_dq<true, kCodeFP4, true>(g, st, packed, sc, n, out, ss, grid, nt)
          : launch_dq<true, kCodeFP4, false>(g, st, packed, sc, n, out, ss, grid, nt);
    else
      abs ? launch_dq<true, kCodeNF4, true>(g, st, packed, sc, n, out, ss, grid, nt)
          : launch_dq<true, kCodeNF4, false>(g, st, packed, sc, n, out, ss, grid, nt);
  } else {
    if (fp4)
      abs ? launch_dq<false, kCodeFP4, true>(g, st, packed, sc, n, out, ss, grid, nt)
          : launch_dq<false, kCodeFP4, false>(g, st, packed, sc, n, out, ss, grid, nt);
    else
      abs ? launch_dq<false, kCodeNF4, true>(g, st, packed, sc, n, out, ss, grid, nt)
          : launch_dq<false, kCodeNF4, false>(g, st, packed, sc, n, out, ss, grid, nt);
  }
  return hipGetLastError();
}


// Transposed dequantization for the dX product: out[k][n] (bf16, row length
// ldt >= rows, ldt % 8 == 0) = Qhat(W)[n][k], zero for rows <= n < ldt.
// One-dimensional grid: the first `aux_wgs` workgroups run the small jobs of
// the same backward (one row job per thread), so they share the machine
// with the dequantization instead of trailing it; then one workgroup per
// tile of 128 rows x 128 columns (two blocks; cols % 64 == 0, columns past
// cols are not stored): wave q takes half q & 1 (32 columns) of block q >> 1,
// lane l rows n0 + 2l and n0 + 2l + 1, whose two values per column go to the
// LDS tile [k][n] as one word; the tile leaves as 256-byte row pieces.
constexpr int DQT_N = 128, DQT_K = 128, DQT_PITCH = DQT_N * 2 + 16;
template <int CB, bool ABS>
__global__ __launch_bounds__(256) void k_dequant_t(const uint8_t* __restrict__ packed,
                                                   const uint8_t* __restrict__ qscale,
                                                   const float* __restrict__ scale2,
                                                   const float* __restrict__ offset,
                                                   const float* __restrict__ absmax, int64_t rows,
                                                   int64_t cols, uint16_t* __restrict__ out,
                                                   int64_t ldt, BwdAux aux, int aux_wgs,
                                                   int gx) {
  __shared__ float lut[16];
  __shared__ __attribute__((aligned(16))) uint8_t tile[DQT_K * DQT_PITCH];
  const int t = threadIdx.x;
  if ((int)blockIdx.x < aux_wgs) {  // one row job per thread
    const int64_t i = (int64_t)blockIdx.x * 256 + t;
    if (i < bwd_aux_count(aux)) bwd_aux_at(aux, i);
    return;
  }
  if (t < 16) {  // from immediates: no load ahead of the code loads
    uint32_t v = level_bits(CB, 0);
#pragma unroll
    for (int k = 1; k < 16; ++k) v = t == k ? level_bits(CB, k) : v;
    lut[t] = as_f32(v);
  }
  const int d = (int)blockIdx.x - aux_wgs;
  const int64_t kq = d / gx;
  const int64_t n0 = (int64_t)(d - kq * gx) * DQT_N;
  const int q = t >> 6, l = t & 63;
  const int64_t kblocks = cols / kBlock;
  // a block past the last one (cols % 128 != 0) repeats the last block; its
  // columns are not stored
  const int64_t kb = min(kq * 2 + (q >> 1), kblocks - 1);
  const int kh = q & 1;
  const int64_t na = n0 + 2 * l, nb = na + 1;
  const int64_t ra = min(na, rows - 1), rb = min(nb, rows - 1);
  // unconditional, clamped loads (no wait at a branch join)
  const u32x4 a = *reinterpret_cast<const u32x4*>(packed + ra * (cols / 2) + kb * 32 + 16 * kh);
  const u32x4 b = *reinterpret_cast<const u32x4*>(packed + rb * (cols / 2) + kb * 32 + 16 * kh);
  const int64_t ba = ra * kblocks + kb, bb = rb * kblocks + kb;
  float sa, sb;
  if (ABS) {  // double quantization off: the block scales themselves
    sa = na < rows ? absmax[ba] : 0.f;
    sb = nb < rows ? absmax[bb] : 0.f;
  } else {
    const uint32_t qa = qscale[ba], qb = qscale[bb];
    const float s2a = scale2[ba / kGroup], s2b = scale2[bb / kGroup], mu = *offset;
    sa = na < rows ? dq_scale(qa, s2a, mu) : 0.f;
    sb = nb < rows ? dq_scale(qb, s2b, mu) : 0.f;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // lut ready
  uint8_t* trow = tile + (int64_t)(64 * (q >> 1) + 32 * kh) * DQT_PITCH + 4 * l;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const uint32_t ca = (a[e >> 3] >> (4 * (e & 7))) & 15u;
    const uint32_t cb = (b[e >> 3] >> (4 * (e & 7))) & 15u;
    uint32_t v = pack_bf16x2(lut[ca] * sa, lut[cb] * sb);
    if (na >= rows) v &= 0xffff0000u;  // +0 past the last row
    if (nb >= rows) v &= 0x0000ffffu;
    *reinterpret_cast<uint32_t*>(trow + e * DQT_PITCH) = v;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // 128 rows of 256 bytes: pass h, thread t -> row 16h + t/16, chunk t%16
  const int c = t & 15;
  const int64_t col = n0 + 8 * c;
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int k = 16 * h + (t >> 4);
    const u32x4 v = *reinterpret_cast<const u32x4*>(tile + k * DQT_PITCH + 16 * c);
    const int64_t kk = kq * DQT_K + k;
    if (col < ldt && kk < cols) *reinterpret_cast<u32x4*>(out + kk * ldt + col) = v;
  }
}

hipError_t launch_dequant_t(const uint8_t* packed, const uint8_t* qscale, const float* scale2,
                            const float* offset, int64_t rows, int64_t cols, uint16_t* out,
                            int64_t ldt, const BwdAux& aux, hipStream_t st, int codebook,
                            const float* absmax) {
  const int64_t gx = (ldt + DQT_N - 1) / DQT_N, gk = (cols + DQT_K - 1) / DQT_K;
  const int64_t aux_wgs = (bwd_aux_count(aux) + 255) / 256;
  const dim3 g((unsigned)(aux_wgs + gx * gk));
#define QN_DQT(CB, ABS)                                                                         \
  hipLaunchKernelGGL((k_dequant_t<CB, ABS>), g, dim3(256), 0, st, packed, qscale, scale2, offset, \
                     absmax, rows, cols, out, ldt, aux, (int)aux_wgs, (int)gx)
  if (codebook == kCodeFP4) {
    if (absmax) QN_DQT(kCodeFP4, true); else QN_DQT(kCodeFP4, false);
  } else {
    if (absmax) QN_DQT(kCodeNF4, true); else QN_DQT(kCodeNF4, false);
  }
#undef QN_DQT
  return hipGetLastError();
}

}  // namespace qn
