// Device helpers shared by the HIP kernels of the QLoRA NF4 library (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qn {

// NF4 levels, codes 0..15, as IEEE binary32 bit patterns.  These are the
// sixteen values of the NF4 table on the page "QLoRA: NF4 storage, gradients
// and local integration" (section "Exact CPU teaching quantizer and adapter
// gradient path"); every one of them is exactly an fp32 number.
constexpr uint32_t kNF4Bits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b30u, 0xbeca32a0u, 0xbe91a24du, 0xbe3d353fu,
    0xbdba7871u, 0x00000000u, 0x3da2faffu, 0x3e24cae3u,
    0x3e7c04ddu, 0x3ead033au, 0x3ee1a4b8u, 0x3f1007abu, 0x3f3913b3u, 0x3f800000u};

// FP4 code values, codes 0..15 (code c: sign bit 3, magnitude index c & 7),
// as binary32 bit patterns: the E2M1 levels {0, 0.0625, 2, 3, 4, 6, 8, 12}
// / 12 (course notebook FT-02, "Exercise 3: NF4 vs FP4 at equal memory",
// prints them to four decimals: 0, 0.0052, 0.1667, 0.25, 0.3333, 0.5,
// 0.6667, 1), each rounded to fp32.
constexpr uint32_t kFP4Bits[16] = {
    0x00000000u, 0x3baaaaabu, 0x3e2aaaabu, 0x3e800000u, 0x3eaaaaabu, 0x3f000000u,
    0x3f2aaaabu, 0x3f800000u, 0x80000000u, 0xbbaaaaabu, 0xbe2aaaabu, 0xbe800000u,
    0xbeaaaaabu, 0xbf000000u, 0xbf2aaaabu, 0xbf800000u};

// Codebooks of the 4-bit codes.
constexpr int kCodeNF4 = 0, kCodeFP4 = 1;

// Level k of codebook cb, as a bit pattern (cb and k known at compile time
// give an immediate).
__host__ __device__ constexpr uint32_t level_bits(int cb, int k) {
  return cb == kCodeFP4 ? kFP4Bits[k] : kNF4Bits[k];
}

constexpr int kBlock = 64;        // first-level block (weights per absmax scale)
constexpr int kGroup = 256;       // second-level block (scales per fp32 scale2)
constexpr float kE4M3Max = 448.f; // largest finite OCP FP8 E4M3FN value

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 h = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return as_f32(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return as_f32(p & 0xffff0000u); }

// sum over s < S of part[s * count + i], added in slice order (loads issued
// eight at a time)
__device__ __forceinline__ float slice_sum(const float* __restrict__ part, int64_t count, int S,
                                           int64_t i) {
  float acc = part[i];
  for (int s0 = 1; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = s0 + k < S ? part[(int64_t)(s0 + k) * count + i] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < S) acc += v[k];
  }
  return acc;
}

// OCP FP8 E4M3FN byte -> fp32 (exact).  Exponent bias 7, three mantissa
// bits, subnormals m * 2^-9; the NaN pattern is never produced here.
__device__ __forceinline__ float e4m3_to_f32(uint32_t q) {
  uint32_t e = (q >> 3) & 15u, m = q & 7u;
  float v = e ? as_f32(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return as_f32(as_u32(v) | ((q & 0x80u) << 24));
}

// fp32 -> OCP FP8 E4M3FN byte, round to nearest even; magnitudes past the
// largest finite value saturate to 448.  Input must be finite.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t sign = (as_u32(x) >> 24) & 0x80u;
  float a = __builtin_fabsf(x);
  uint32_t mag;
  if (a < 0x1p-6f) {
    // subnormal range: quantum 2^-9, result 0..8 (8 = smallest normal)
    mag = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    uint32_t b = as_u32(a);
    // keep 3 mantissa bits, round half to even on the 20 dropped bits
    uint32_t r = b + 0x7ffffu + ((b >> 20) & 1u);
    mag = (r >> 20) - (120u << 3);
  }
  if (mag > 126u) mag = 126u;
  return sign | mag;
}

// Dequant scale s'_b = fmaf(e4m3(q_b), s2_g, mu): one rounding.
__device__ __forceinline__ float dq_scale(uint32_t q, float s2, float mu) {
  return __builtin_fmaf(e4m3_to_f32(q), s2, mu);
}

// Where a state's block scales come from: the double-quantized codes
// (absmax == null) or fp32 block scales as they are (double quantization
// off).
struct ScaleSrc {
  const uint8_t* qscale;
  const float* scale2;
  const float* offset;
  const float* absmax;
};

}  // namespace qn
