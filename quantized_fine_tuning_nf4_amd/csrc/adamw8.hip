// 8-bit AdamW step for the adapters (course notebook FT-02, the training
// arguments' optim="paged_adamw_8bit": the two Adam moments kept in 8 bits).
// State format (a reading; the pages fix none): each moment tensor in blocks
// of 256 elements, OCP E4M3FN codes of x / s_b with one fp32 scale per block,
// s_b = RN32(max|x| / 448) (0: every code 0).  The update, in fp32 with one
// rounding per operation in this order (no contraction):
//   m = b1 m_old + omb1 g,  v = b2 v_old + (omb2 g) g,  p = p decay,
//   p = p - lr ((m / c1) / (sqrt(v / c2) + eps))
// (omb = 1 - b, c = 1 - b^t, decay = 1 - lr wd, given as fp32), then both
// moments are stored again with new block scales.
//
// One wave per block of 256 elements, four consecutive elements per lane;
// the block's new scales come from a wave max.
#include "qn_device.h"
#include "qn_internal.h"

namespace qn {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__global__ __launch_bounds__(256) void k_adamw8(float* __restrict__ p, const float* __restrict__ g,
                                                int64_t n, uint8_t* __restrict__ mq,
                                                float* __restrict__ ms, uint8_t* __restrict__ vq,
                                                float* __restrict__ vs, uint16_t* __restrict__ pb,
                                                AdamScalars h) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t i0 = blk * 256 + 4 * lane;
  if (blk * 256 >= n) return;  // whole wave: past the last block
  const bool full = i0 + 4 <= n;
  float pv[4], gv[4];
  uint32_t mc = 0, vc = 0;
  if (full) {
    const float4 a = *reinterpret_cast<const float4*>(p + i0);
    const float4 b = *reinterpret_cast<const float4*>(g + i0);
    pv[0] = a.x; pv[1] = a.y; pv[2] = a.z; pv[3] = a.w;
    gv[0] = b.x; gv[1] = b.y; gv[2] = b.z; gv[3] = b.w;
    mc = *reinterpret_cast<const uint32_t*>(mq + i0);
    vc = *reinterpret_cast<const uint32_t*>(vq + i0);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool in = i0 + k < n;
      pv[k] = in ? p[i0 + k] : 0.f;
      gv[k] = in ? g[i0 + k] : 0.f;
      mc |= (in ? (uint32_t)mq[i0 + k] : 0u) << (8 * k);
      vc |= (in ? (uint32_t)vq[i0 + k] : 0u) << (8 * k);
    }
  }
  const float sm = ms[blk], sv = vs[blk];
  float m[4], v[4], amax_m = 0.f, amax_v = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float mo = e4m3_to_f32((mc >> (8 * k)) & 0xffu) * sm;
    const float vo = e4m3_to_f32((vc >> (8 * k)) & 0xffu) * sv;
    m[k] = h.b1 * mo + h.omb1 * gv[k];
    v[k] = h.b2 * vo + (h.omb2 * gv[k]) * gv[k];
    float pi = pv[k] * h.decay;
    const float denom = __builtin_sqrtf(v[k] / h.c2) + h.eps;
    const float upd = (m[k] / h.c1) / denom;
    pv[k] = pi - h.lr * upd;
    if (i0 + k < n) {
      amax_m = fmaxf(amax_m, __builtin_fabsf(m[k]));
      amax_v = fmaxf(amax_v, __builtin_fabsf(v[k]));
    }
  }
  const float s_m = wave_max(amax_m) / kE4M3Max, s_v = wave_max(amax_v) / kE4M3Max;
  uint32_t mo = 0, vo = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    mo |= (s_m > 0.f ? f32_to_e4m3(m[k] / s_m) : 0u) << (8 * k);
    vo |= (s_v > 0.f ? f32_to_e4m3(v[k] / s_v) : 0u) << (8 * k);
  }
  if (full) {
    *reinterpret_cast<float4*>(p + i0) = make_float4(pv[0], pv[1], pv[2], pv[3]);
    *reinterpret_cast<uint32_t*>(mq + i0) = mo;
    *reinterpret_cast<uint32_t*>(vq + i0) = vo;
    if (pb)
      *reinterpret_cast<u32x2*>(pb + i0) = u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i0 + k < n) {
        p[i0 + k] = pv[k];
        mq[i0 + k] = (uint8_t)(mo >> (8 * k));
        vq[i0 + k] = (uint8_t)(vo >> (8 * k));
        if (pb) pb[i0 + k] = (uint16_t)(pack_bf16x2(pv[k], 0.f) & 0xffffu);
      }
  }
  if (lane == 0) {
    ms[blk] = s_m;
    vs[blk] = s_v;
  }
}

}  // namespace

hipError_t launch_adamw8(float* p, const float* g, int64_t n, uint8_t* mq, float* ms, uint8_t* vq,
                         float* vs, uint16_t* pb, const AdamScalars& h, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t nb = (n + 255) / 256;
  hipLaunchKernelGGL(k_adamw8, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, st, p, g, n, mq, ms,
                     vq, vs, pb, h);
  return hipGetLastError();
}

}  // namespace qn
