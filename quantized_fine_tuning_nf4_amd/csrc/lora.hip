// Rank-r adapter products of the QLoRA linear (page "QLoRA: NF4 storage,
// gradients and local integration", paragraph after the teaching listing):
//   u = X A^T and v = G B          -- "thin NT" products, reduction along a
//                                     row of both operands;
//   dB = s G^T u and dA = s v^T X  -- "thin TN" products, reduction over the
//                                     M rows, split in slices whose partial
//                                     sums are added in slice order.
// All use v_mfma_f32_16x16x32_bf16; fp32 operands (u, v) enter the MFMA as a
// bf16 high part plus a bf16 remainder, so they keep ~16 significant bits.
#include <algorithm>
#include <type_traits>

#include "qn_device.h"
#include "qn_internal.h"

namespace qn {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 consecutive bf16 of a row at column p (zero past the row end P).
__device__ __forceinline__ u32x4 load8(const uint16_t* row, int64_t p, int64_t P) {
  if (p + 8 <= P) return *reinterpret_cast<const u32x4*>(row + p);
  uint32_t w[4];
  for (int h = 0; h < 4; ++h) {
    uint32_t lo = p + 2 * h < P ? row[p + 2 * h] : 0u;
    uint32_t hi = p + 2 * h + 1 < P ? row[p + 2 * h + 1] : 0u;
    w[h] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// 8 bf16 values with the dropped ones zeroed: mb holds their 8 mask bits
// (the masks are bit-packed over the elements, bit e % 8 of byte e / 8 set:
// kept, so 8 elements starting at a multiple of 8 share one byte).
__device__ __forceinline__ u32x4 keep8(u32x4 v, uint32_t mb) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] &= (((mb >> (2 * q)) & 1u) * 0xffffu) | (((mb >> (2 * q + 1)) & 1u) * 0xffff0000u);
  return v;
}

// The first workgroup of a launch zeroes clr.n words at clr.p (the arrival
// counters a later kernel of the same call counts on).
__device__ __forceinline__ void clear_words(const Clear& clr) {
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < clr.n; i += blockDim.x) clr.p[i] = 0u;
}

}  // namespace

// out[M, r] = Z[M, P] T[r, P]^T over column slice s.  Workgroup (mt, s):
// rows 64mt .. 64mt+63, wave w rows 16w .. +15, all columns of the slice.
// MFMA lane l holds row l%16 and the eight columns 8(l/16).. of each 32-wide
// step of both operands (rows of Z and of T are contiguous along the
// reduction).  U steps' loads are issued before their MFMAs.  Columns past
// the slice load as zero (P is a multiple of 8).  NJ = ceil(r/16).
template <int NJ>
__global__ __launch_bounds__(kThreads) void k_thin_nt(const uint16_t* __restrict__ Z,
                                                      const uint16_t* __restrict__ T, int64_t M,
                                                      int64_t P, int r, int64_t slice,
                                                      float* __restrict__ out, Clear clr,
                                                      const uint8_t* __restrict__ zmask) {
  constexpr int U = NJ <= 2 ? 8 : 4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  clear_words(clr);
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t mw = (int64_t)blockIdx.x * 64 + 16 * wave;  // first row of the wave
  const int64_t m = min(mw + l16, M - 1);
  const int64_t pb = (int64_t)blockIdx.y * slice, pe = min(pb + slice, P);
  const int steps = (int)((pe - pb + 31) / 32);
  const uint16_t* zp = Z + m * P + pb + 8 * g;
  const uint16_t* tp[NJ];
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt) tp[jt] = T + (int64_t)min(16 * jt + l16, r - 1) * P + pb + 8 * g;
  const int64_t lim = pe - pb - 8 * g;  // in-slice columns left for this lane's chunk
  f32x4 acc[NJ] = {};
  for (int s0 = 0; s0 < steps; s0 += U) {
    u32x4 za[U], tb[U][NJ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = 32 * (int64_t)(s0 + u);
      const bool ok = off < lim;
      const int64_t o = ok ? off : 0;
      za[u] = *reinterpret_cast<const u32x4*>(zp + o);
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) tb[u][jt] = *reinterpret_cast<const u32x4*>(tp[jt] + o);
      if (zmask) za[u] = keep8(za[u], zmask[(m * P + pb + 8 * g + o) >> 3]);
      if (!ok) za[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        u32x4 b = tb[u][jt];
        if (16 * jt + l16 >= r) b = u32x4{0u, 0u, 0u, 0u};
        acc[jt] = mfma16(as_bf16x8(za[u]), as_bf16x8(b), acc[jt]);
      }
  }
  // lane l: column j = 16jt + l%16, rows mw + 4(l/16) + i
  float* dst = out + (int64_t)blockIdx.y * M * r;
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt) {
    const int j = 16 * jt + l16;
    if (j >= r) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = mw + 4 * g + i;
      if (row < M) dst[row * r + j] = acc[jt][i];
    }
  }
}

// r <= 16: the same product with T's slice (rows 0..15, zero past r)
// staged in LDS once per workgroup (row pitch 64 steps + 16 bytes, so the
// 16-byte reads of 8 consecutive rows fall in distinct bank groups), and Z
// streamed through registers two batches of TN1_U steps deep: the loads of
// batch b + 1 are in flight while batch b is multiplied.  Columns past the
// slice read as zero (selected at use, so no load waits at a branch).
constexpr int TN1_U = 4;
constexpr int64_t kThinNt1MaxSlice = 2048;
template <int TMODE>
__global__ __launch_bounds__(kThreads) void k_thin_nt1(const uint16_t* __restrict__ Z,
                                                       const uint16_t* __restrict__ T, int64_t M,
                                                       int64_t P, int r, int64_t slice,
                                                       float* __restrict__ out, Clear clr,
                                                       const uint8_t* __restrict__ zmask) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  clear_words(clr);
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t mw = (int64_t)blockIdx.x * 64 + 16 * wave;
  const int64_t m = min(mw + l16, M - 1);
  const int64_t pb = (int64_t)blockIdx.y * slice, pe = min(pb + slice, P);
  const int64_t width = pe - pb;
  const int steps = (int)((width + 31) / 32);
  const int nb = (steps + TN1_U - 1) / TN1_U;
  const int pitch = steps * 64 + 16;
  const uint16_t* zp = Z + m * P + pb + 8 * g;
  const int64_t lim = width - 8 * g;  // in-slice columns left for this lane's chunk
  u32x4 za[2][TN1_U];
  // the batch's mask bytes (dropout on Z), loaded beside it: row m's 16
  // bytes for the batch's 128 columns as two 8-byte halves (two steps each;
  // P % 64 == 0 and the slice starts on 128 columns, so each half is aligned
  // and lies in the row when its first column is in the slice; a half past
  // the slice reads the slice's first one instead, for steps zeroed at use)
  static_assert(TN1_U == 4, "two steps per 8-byte half of a batch's mask bytes");
  uint2 zk[2][2];
  auto load_batch = [&](int buf, int b) {
#pragma unroll
    for (int u = 0; u < TN1_U; ++u) {
      const int64_t off = 32 * (int64_t)(TN1_U * b + u);
      za[buf][u] = *reinterpret_cast<const u32x4*>(zp + (off < lim ? off : 0));
    }
    if (zmask) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t c = 128 * (int64_t)b + 64 * h;
        zk[buf][h] = *reinterpret_cast<const uint2*>(zmask + ((m * P + pb + (c < width ? c : 0)) >> 3));
      }
    }
  };
  if constexpr (TMODE == 0) {
    // stage T: eight 16-byte chunks per thread per pass, every load issued
    // before the first is used (clamped addresses; zero selected at the LDS
    // write for rows past r and columns past the slice); the first Z batch
    // goes out behind the first pass
    const int cpr = steps * 4;  // 16-byte chunks per staged row
    const int total = 16 * cpr;
    for (int e0 = 0; e0 < total; e0 += 8 * kThreads) {
      u32x4 tv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = min(e0 + q * kThreads + tid, total - 1);
        const int j = e / cpr, c = e - j * cpr;
        const int64_t col = min(8 * (int64_t)c, width - 8);
        tv[q] = *reinterpret_cast<const u32x4*>(T + (int64_t)min(j, r - 1) * P + pb + col);
      }
      if (e0 == 0) load_batch(0, 0);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = e0 + q * kThreads + tid;
        if (e < total) {
          const int j = e / cpr, c = e - j * cpr;
          const bool ok = j < r && 8 * (int64_t)c < width;
          *reinterpret_cast<u32x4*>(smem + j * pitch + 16 * c) = ok ? tv[q] : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  } else {
    // stage T given as its transpose Tr [P, r] (the adapter B as stored): a
    // thread takes a pair of columns (two rows of Tr, r <= 16 values each),
    // loads them (unconditional, clamped), sends the first Z batch, then
    // writes one word per rank (the pair's two values) to LDS; zero for
    // ranks >= r and columns past the slice
    const int pairs = steps * 16;
    for (int p0 = 0; p0 < pairs; p0 += 4 * kThreads) {
      uint32_t v[4][16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int pp = min(p0 + k * kThreads + tid, pairs - 1);
        const int64_t c0 = min(pb + 2 * (int64_t)pp, P - 1), c1 = min(c0 + 1, P - 1);
        if constexpr (TMODE == 1) {
          const u32x4* s0 = reinterpret_cast<const u32x4*>(T + c0 * 16);
          const u32x4* s1 = reinterpret_cast<const u32x4*>(T + c1 * 16);
          const u32x4 a0 = s0[0], a1 = s0[1], b0 = s1[0], b1 = s1[1];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[k][2 * q] = (a0[q] & 0xffffu) | (b0[q] << 16);
            v[k][2 * q + 1] = (a0[q] >> 16) | (b0[q] & 0xffff0000u);
            v[k][8 + 2 * q] = (a1[q] & 0xffffu) | (b1[q] << 16);
            v[k][8 + 2 * q + 1] = (a1[q] >> 16) | (b1[q] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int jj = min(j, r - 1);
            v[k][j] = (uint32_t)T[c0 * r + jj] | ((uint32_t)T[c1 * r + jj] << 16);
          }
        }
      }
      if (p0 == 0) load_batch(0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int pp = p0 + k * kThreads + tid;
        if (pp < pairs) {
          const int64_t col = 2 * (int64_t)pp;
          const uint32_t keep = (col < width ? 0xffffu : 0u) | (col + 1 < width ? 0xffff0000u : 0u);
#pragma unroll
          for (int j = 0; j < 16; ++j)
            *reinterpret_cast<uint32_t*>(smem + j * pitch + 4 * pp) = j < r ? (v[k][j] & keep) : 0u;
        }
      }
    }
  }
  // LDS-only barrier: the first Z batch stays in flight
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const uint8_t* trow = smem + l16 * pitch + 16 * g;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute_batch = [&](int buf, int b) {
#pragma unroll
    for (int u = 0; u < TN1_U; ++u) {
      const int st = TN1_U * b + u;
      if (st < steps) {
        u32x4 z = 32 * (int64_t)st < lim ? za[buf][u] : u32x4{0u, 0u, 0u, 0u};
        if (zmask) {  // byte g of the step's four: this lane's eight columns
          const uint32_t w = (u & 1) ? zk[buf][u >> 1].y : zk[buf][u >> 1].x;
          z = keep8(z, (w >> (8 * g)) & 0xffu);
        }
        const u32x4 t = *reinterpret_cast<const u32x4*>(trow + 64 * st);
        acc = mfma16(as_bf16x8(z), as_bf16x8(t), acc);
      }
    }
  };
  for (int b = 0; b < nb; b += 2) {
    if (b + 1 < nb) load_batch(1, b + 1);
    compute_batch(0, b);
    if (b + 1 < nb) {
      if (b + 2 < nb) load_batch(0, b + 2);
      compute_batch(1, b + 1);
    }
  }
  // lane l: column j = l%16, rows mw + 4(l/16) + i
  float* dst = out + (int64_t)blockIdx.y * M * r;
  if (l16 < r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = mw + 4 * g + i;
      if (row < M) dst[row * r + l16] = acc[i];
    }
  }
}

// out[i] = sum over s of part[s][i], added in slice order.
__global__ void k_sum_slices(const float* __restrict__ part, int64_t count, int S,
                             float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) out[i] = slice_sum(part, count, S, i);
}

// Column slice of launch_thin_nt (a multiple of 128).
int64_t thin_nt_slice(int64_t P, int S) {
  const int64_t slice = (P + S - 1) / S;
  return (slice + 127) / 128 * 128;
}

// Whether launch_thin_nt takes T as its transpose [P, r] for this shape.
bool thin_nt_rows_ok(int64_t M, int64_t P, int r) {
  return r <= 16 && thin_nt_slice(P, thin_nt_slices(M, P)) <= kThinNt1MaxSlice;
}

// Column slices (multiples of 128 columns) so that about 512 workgroups run.
int thin_nt_slices(int64_t M, int64_t P) {
  const int64_t mt = M > 0 ? (M + 63) / 64 : 1;
  int64_t S = (512 + mt - 1) / mt;
  const int64_t smax = (P + 127) / 128;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  return (int)S;
}

hipError_t launch_thin_nt(const uint16_t* Z, const uint16_t* T, int64_t M, int64_t P, int r,
                          float* out, float* part, int S, hipStream_t st, bool sum, bool t_rows,
                          Clear clr, const uint8_t* zmask) {
  const int64_t slice = thin_nt_slice(P, S);
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)S);
  float* dst = S > 1 ? part : out;
  if (r <= 16 && slice <= kThinNt1MaxSlice) {
    const int mode = !t_rows ? 0 : r == 16 ? 1 : 2;
    static const hipError_t attr[3] = {
        hipFuncSetAttribute(reinterpret_cast<const void*>(k_thin_nt1<0>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(16 * (kThinNt1MaxSlice * 2 + 16))),
        hipFuncSetAttribute(reinterpret_cast<const void*>(k_thin_nt1<1>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(16 * (kThinNt1MaxSlice * 2 + 16))),
        hipFuncSetAttribute(reinterpret_cast<const void*>(k_thin_nt1<2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(16 * (kThinNt1MaxSlice * 2 + 16)))};
    if (attr[mode] != hipSuccess) return attr[mode];
    const int steps = (int)((slice + 31) / 32);
    const size_t lds = (size_t)16 * (steps * 64 + 16);
    if (mode == 0)
      hipLaunchKernelGGL(k_thin_nt1<0>, grid, dim3(kThreads), lds, st, Z, T, M, P, r, slice, dst, clr, zmask);
    else if (mode == 1)
      hipLaunchKernelGGL(k_thin_nt1<1>, grid, dim3(kThreads), lds, st, Z, T, M, P, r, slice, dst, clr, zmask);
    else
      hipLaunchKernelGGL(k_thin_nt1<2>, grid, dim3(kThreads), lds, st, Z, T, M, P, r, slice, dst, clr, zmask);
  } else {
    if (t_rows) return hipErrorInvalidValue;  // the general kernel takes T as [r, P]
  switch ((r + 15) / 16) {
    case 1: hipLaunchKernelGGL(k_thin_nt<1>, grid, dim3(kThreads), 0, st, Z, T, M, P, r, slice, dst, clr, zmask); break;
    case 2: hipLaunchKernelGGL(k_thin_nt<2>, grid, dim3(kThreads), 0, st, Z, T, M, P, r, slice, dst, clr, zmask); break;
    case 3: hipLaunchKernelGGL(k_thin_nt<3>, grid, dim3(kThreads), 0, st, Z, T, M, P, r, slice, dst, clr, zmask); break;
    default: hipLaunchKernelGGL(k_thin_nt<4>, grid, dim3(kThreads), 0, st, Z, T, M, P, r, slice, dst, clr, zmask); break;
  }
  }
  if (S > 1 && sum) {
    const int64_t count = M * r;
    hipLaunchKernelGGL(k_sum_slices, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                       part, count, S, out);
  }
  return hipGetLastError();
}

__global__ void k_fill_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

__global__ void k_bwd_aux(BwdAux a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < bwd_aux_count(a)) bwd_aux_at(a, i);
}

hipError_t launch_bwd_aux(const BwdAux& a, hipStream_t st) {
  const int64_t count = bwd_aux_count(a);
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_aux, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rs(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, soff, 0, 0);
}

constexpr int TN_COLS = 128;             // columns of Z per workgroup
constexpr int TN_ROWB = TN_COLS * 2;     // 256 B per staged Z row
constexpr int TN_NST = 3;  // stages (two steps in flight; three: 1.5 us slower per backward)

}  // namespace

// part[z][p][j] = sum over the rows m of slice z of Z[m, p] * (s V)[m, j]
// (a transposed product: the reduction runs down the columns of Z).  Two
// independent products (dB and dA of one backward) share the launch: grid x
// runs over the column tiles of job 0, then those of job 1.  Workgroup
// (pt, z): columns 128 pt .. +127, wave w: 32w .. 32w+31 (two 16-column MFMA
// tiles).  A step is 32 rows: their Z (8 KB) and their (s V)^T high and
// remainder parts (2 x 16 NJ rows of 64 B) go global -> LDS by buffer loads
// into one stage, three stages deep, every wave issuing 2 + 2 NJ loads per
// step.
// Z row y's 16-byte chunk c sits at unit c ^ 2(y & 3); the A operand (16
// columns x 32 rows) is read transposed with ds_read_b64_tr_b16, lane t of a
// 16-lane group addressing row 4h + t/4, columns 4(t%4)..+3, so that lane t
// receives column t, four consecutive rows.  NJ = ceil(r/16).
struct TnJob {
  const uint16_t* Z;   // [M, P] bf16
  const uint16_t* vt;  // [2][16 NJ][Mp] (s V)^T high and remainder parts
  int64_t Mp;
  int64_t P;
  int64_t slice;       // rows per slice, a multiple of 32
  int S;               // slices
  int tiles;           // column tiles of 128
  float* part;         // [S, P, r]
  float* out;          // [P, r], or [r, P] when transposed
  int transposed;
  const uint8_t* zmask;  // keep bits of Z (dropout on x), or null
};

// Arrival counters of the column tiles of one launch (both jobs' tiles in
// grid order) sit in the caller's workspace: zero when the launch starts,
// left at zero by the workgroup that finishes a tile.
constexpr int kTnMaxTiles = kArrivalWords;
constexpr int kDeviceScope = 16;  // sc1: the level every XCD shares

// With arrivals != null the slices are also added here: each workgroup
// stores its slice with device-coherent stores, and the last of a column
// tile's S workgroups to arrive (an arrival counter per tile) adds the S
// slices of the tile in slice order with device-coherent loads and writes
// the output.
// vmcnt wait for the given count (an immediate of the instruction).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 4 && N <= 11, "counts of k_thin_tn's steps");
  if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if constexpr (N == 7) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
}

// MASK: a job may carry keep bits of Z (dropout on the adapter branch's
// input, for dA): the step's 32 rows x 16 bytes of bits go global -> LDS
// beside Z (one 4-byte-per-lane load in waves 0 and 1: rows 16w .. 16w+15;
// the direct-to-LDS path writes one dword per lane), and the dropped values
// are zeroed in the A operand after the transposed reads.
template <int NJ, bool MASK>
__global__ __launch_bounds__(kThreads) void k_thin_tn(TnJob j0, TnJob j1, int64_t M, int r,
                                                      unsigned* __restrict__ arrivals) {
  constexpr int ZB = 32 * TN_ROWB;             // Z bytes per stage
  constexpr int VB = 2 * 16 * NJ * 64;         // (sV)^T bytes per stage
  constexpr int KB = MASK ? 32 * 16 : 0;       // keep bits per stage
  constexpr int SB = ZB + VB + KB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool second = (int)blockIdx.x >= j0.tiles;
  const uint16_t* Z = second ? j1.Z : j0.Z;
  const uint16_t* vt = second ? j1.vt : j0.vt;
  const int64_t Mp = second ? j1.Mp : j0.Mp;
  const int64_t P = second ? j1.P : j0.P;
  const int64_t slice = second ? j1.slice : j0.slice;
  const int S = second ? j1.S : j0.S;
  float* part = second ? j1.part : j0.part;
  const uint8_t* zmask = MASK ? (second ? j1.zmask : j0.zmask) : nullptr;
  const bool hm = MASK && zmask != nullptr;  // workgroup-uniform
  if ((int)blockIdx.y >= S) return;
  const int64_t p0 = (int64_t)((int)blockIdx.x - (second ? j0.tiles : 0)) * TN_COLS;
  const int64_t mb = (int64_t)blockIdx.y * slice;
  const int64_t me = min(mb + slice, M);
  const int steps = (int)((me - mb + 31) / 32);

  // ---- Z loads: instruction i (0..7) of a step covers rows 4i..4i+3; wave w
  // issues i = 2w, 2w+1; lane l -> row 4i + l/16, unit l%16, source chunk
  // (l%16) ^ 2(row & 3).  Rows past M repeat row M-1 (their sV is zero);
  // columns past P repeat the last chunk (their outputs are not stored).
  // (sV)^T loads: 4 of its 64-byte rows per 4-byte-per-lane instruction
  // (lane l: row 4q + l/16, word l%16), instruction q = 2 NJ w + k of the
  // step (all lanes active: no branch around a load into LDS).
  // descriptors start at the slice's first row, so that only one slice's
  // bytes (below 2^31, thin_tn_slice_rows) are ever addressed by an offset
  const rsrc_t rz = make_rs(Z + mb * P, (uint32_t)((me - mb) * P * 2));
  const rsrc_t rv = make_rs(vt + mb, (uint32_t)((2 * 16 * NJ * Mp - mb) * 2));
  // keep bits from the slice's first row (P % 64 == 0: rows start on a byte);
  // bytes past the slice read as zero (columns past P are not stored)
  const rsrc_t rk = make_rs(hm ? zmask + mb * P / 8 : reinterpret_cast<const uint8_t*>(Z),
                            hm ? (uint32_t)((me - mb) * P / 8) : 0u);
  uint32_t zoff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 2 * wave + h, row = 4 * i + (lane >> 4);
    const int chunk = (lane & 15) ^ (2 * (row & 3));
    const int64_t col = min(p0 + 8 * chunk, P - 8);
    zoff[h] = (uint32_t)(col * 2);
  }
  uint32_t voff[2 * NJ];
#pragma unroll
  for (int k = 0; k < 2 * NJ; ++k) {
    const int q = 2 * NJ * wave + k, row = 4 * q + (lane >> 4);
    voff[k] = (uint32_t)(row * Mp * 2 + 4 * (lane & 15));
  }
  auto load_step = [&](int st, int stage) {
    uint8_t* base = smem + stage * SB;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * wave + h, row = 4 * i + (lane >> 4);
      const int64_t mm = min(mb + 32 * (int64_t)st + row, M - 1);
      dma16(rz, zoff[h] + (uint32_t)((mm - mb) * P * 2), 0, base + 1024 * i);
    }
#pragma unroll
    for (int k = 0; k < 2 * NJ; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(base + ZB + 256 * (2 * NJ * wave + k)),
                                               4, voff[k] + (uint32_t)(64 * st), 0, 0, 0);
    if constexpr (MASK) {
      if (hm && wave < 2) {  // lane l: row 16w + l/4, bytes 4(l%4) .. +3 of the tile's 16
        const int row = 16 * wave + (lane >> 2);
        const int64_t mm = min(mb + 32 * (int64_t)st + row, M - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (lds_void*)(base + ZB + VB + 256 * wave), 4,
            (uint32_t)((((mm - mb) * P + p0) >> 3) + 4 * (lane & 3)), 0, 0, 0);
      }
    }
  };
  // all but the newest step's loads (2 + 2 NJ per wave) have landed
  // (one more in waves 0 and 1 when the keep bits come along)
  auto wait_step = [&]() {
    static_assert(TN_NST == 3, "one step in flight beyond the next");
    if (MASK && hm && wave < 2)
      wait_vm<2 + 2 * NJ + (MASK ? 1 : 0)>();
    else
      wait_vm<2 + 2 * NJ>();
  };
  for (int k = 0; k < TN_NST - 1; ++k) load_step(min(k, steps - 1), k);
  wait_step();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // transposed-read addresses: lane l, group g = l/16, t = l%16; p-tile pt,
  // half h: row 8g + 4h + t/4, column 32w + 16pt + 4(t%4)
  const int g = lane >> 4, t = lane & 15;
  int aoff[2][2];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * g + 4 * h + (t >> 2);
      const int col = 32 * wave + 16 * pt + 4 * (t & 3);
      aoff[pt][h] = row * TN_ROWB + 16 * ((col >> 3) ^ (2 * (row & 3))) + 2 * (col & 7);
    }
  f32x4 acc[2][NJ] = {};
  // one step on stage P (a constant, so that the compiler sees the loads of
  // step st+2 and this step's LDS reads touch different stages)
  auto body = [&](auto p_t, int st) {
    constexpr int P = decltype(p_t)::value;
    load_step(min(st + TN_NST - 1, steps - 1), (P + TN_NST - 1) % TN_NST);
    const uint8_t* zs = smem + P * SB;
    // the four transposed reads in one block that also waits for them (the
    // compiler would otherwise treat them as possibly overlapping the loads
    // in flight to the other stages and wait for all of those first)
    const uint32_t zb = (uint32_t)reinterpret_cast<uintptr_t>(zs);
    u32x2 x00, x01, x10, x11;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        // early-clobber: a result must not share a register with an address
        // that a later read of the block still has to issue with
        : "=&v"(x00), "=&v"(x01), "=&v"(x10), "=&v"(x11)
        : "v"(zb + aoff[0][0]), "v"(zb + aoff[0][1]), "v"(zb + aoff[1][0]), "v"(zb + aoff[1][1])
        : "memory");
    u32x4 za[2] = {u32x4{x00[0], x00[1], x01[0], x01[1]}, u32x4{x10[0], x10[1], x11[0], x11[1]}};
    if constexpr (MASK) {
      if (hm) {
        // word i of za[pt] holds rows 8g + 2i, 8g + 2i + 1 of column
        // 32w + 16pt + t, whose keep bits are bit 16pt + t of the word at
        // byte 4w of each row's 16 bytes
        const uint8_t* ks = zs + ZB + VB + 4 * wave;
        uint32_t kw[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          kw[q] = *reinterpret_cast<const uint32_t*>(ks + 16 * (8 * g + q));
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const int sh = 16 * pt + t;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            za[pt][i] &= (((kw[2 * i] >> sh) & 1u) * 0xffffu) |
                         (((kw[2 * i + 1] >> sh) & 1u) * 0xffff0000u);
        }
      }
    }
    bf16x8 a[2];
    a[0] = as_bf16x8(za[0]);
    a[1] = as_bf16x8(za[1]);
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      // B operand: column j = 16jt + l%16, rows 8g..8g+7 of the step
      const uint8_t* vs = zs + ZB + (16 * jt + t) * 64 + 16 * g;
      const bf16x8 bh = as_bf16x8(*reinterpret_cast<const u32x4*>(vs));
      const bf16x8 bl = as_bf16x8(*reinterpret_cast<const u32x4*>(vs + 16 * NJ * 64));
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        acc[pt][jt] = mfma16(a[pt], bh, acc[pt][jt]);
        acc[pt][jt] = mfma16(a[pt], bl, acc[pt][jt]);
      }
    }
    // step st+1's loads (issued 2 steps ago) have landed everywhere before
    // anyone reads them or overwrites this stage
    wait_step();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  int st = 0;
  for (; st + 3 <= steps; st += 3) {
    body(S0{}, st);
    body(S1{}, st + 1);
    body(S2{}, st + 2);
  }
  if (st < steps) body(S0{}, st);
  if (st + 1 < steps) body(S1{}, st + 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // lane: column j = 16jt + l%16, rows p = 16pt + 4(l/16) + i of the wave
  const int S_ = S;
  const rsrc_t rp = make_rs(part, (uint32_t)((int64_t)S_ * P * r * 4));
  const int64_t sl_off = (int64_t)blockIdx.y * P * r;
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt) {
    const int j = 16 * jt + t;
    if (j >= r) continue;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t p = p0 + 32 * wave + 16 * pt + 4 * g + i;
        if (p < P)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[pt][jt][i]), rp,
                                                (uint32_t)((sl_off + p * r + j) * 4), 0,
                                                kDeviceScope);
      }
  }
  if (!arrivals) return;
  // ---- arrival: every wave's stores have completed before the barrier, so
  // they precede the count; the last workgroup reads them after it
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ int s_last;
  unsigned* ctr = arrivals + blockIdx.x;
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(S_ - 1);
  __syncthreads();
  if (!s_last) return;
  // ---- the tile's columns p0 .. p0 + np - 1: slice z holds them as np r
  // contiguous floats at (z P + p0) r; elements e, in chunks of 2048 (eight
  // per thread, every load of a chunk issued before the first add)
  const int np = (int)min((int64_t)TN_COLS, P - p0);
  const int cnt = np * r;
  const bool tr = second ? j1.transposed : j0.transposed;
  float* out = second ? j1.out : j0.out;
  const bool vec = (r % 4) == 0 && (P * r) % 4 == 0;
  const uint32_t zst = (uint32_t)((int64_t)P * r * 4);  // bytes between slices
  for (int c0 = 0; c0 < cnt; c0 += 8 * kThreads) {
    // a[q]: element c0 + 4 ((q / 4) kThreads + tid) + q % 4
    float a[8];
    if (vec) {
      uint32_t o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        o[h] = (uint32_t)(((int64_t)p0 * r + min(c0 + 4 * (h * kThreads + tid), cnt - 4)) * 4);
      f32x4 v[2];
      // one half at a time (registers), sixteen slices' loads in flight
      // (clamped: the extra ones are not added)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        for (int z0 = 0; z0 < S_; z0 += 16) {
          f32x4 w[16];
#pragma unroll
          for (int k = 0; k < 16; ++k)
            w[k] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rp, o[h] + (uint32_t)min(z0 + k, S_ - 1) * zst, 0, kDeviceScope));
          if (z0 == 0) v[h] = w[0];
#pragma unroll
          for (int k = 0; k < 16; ++k)
            if ((z0 > 0 || k > 0) && z0 + k < S_) v[h] += w[k];
        }
#pragma unroll
      for (int q = 0; q < 8; ++q) a[q] = v[q >> 2][q & 3];
    } else {
      uint32_t o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        o[q] = (uint32_t)(((int64_t)p0 * r +
                           min(c0 + 4 * ((q >> 2) * kThreads + tid) + (q & 3), cnt - 1)) * 4);
      for (int z0 = 0; z0 < S_; z0 += 8) {
        float w[8][8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int q = 0; q < 8; ++q)
            w[q][k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rp, o[q] + (uint32_t)min(z0 + k, S_ - 1) * zst, 0, kDeviceScope));
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (z0 == 0) a[q] = w[q][0];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((z0 > 0 || k > 0) && z0 + k < S_) a[q] += w[q][k];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = c0 + 4 * ((q >> 2) * kThreads + tid) + (q & 3);
      if (e >= cnt) continue;
      const int64_t p = p0 + e / r;
      const int j = e % r;
      if (tr)
        out[(int64_t)j * P + p] = a[q];
      else
        out[p * r + j] = a[q];
    }
  }
  if (tid == 0)  // every slice has arrived: ready for the next call
    __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// out = sum over slices of part, added in slice order (loads issued eight
// at a time), for the two products of one launch: threads 0 .. P0 r - 1
// produce job 0's output, the rest job 1's.  transposed: out[j][p], thread
// index running along p.
struct TnSum {
  const float* part;
  int64_t P;
  int S;
  bool transposed;
  float* out;
};
__global__ void k_sum_slices_tn(TnSum a, TnSum b, int r) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t count_a = a.P * r;
  const bool second = t >= count_a;
  const TnSum& J = second ? b : a;
  if (second) t -= count_a;
  const int64_t count = J.P * r;
  if (t >= count) return;
  // element index into part[s] ([P][r]) and into out
  const int64_t i = J.transposed ? (t % J.P) * r + t / J.P : t;
  J.out[t] = slice_sum(J.part, count, J.S, i);
}

// Slices of the M rows for the transposed products: enough workgroups to
// fill the chip (about 512 per product), a multiple of 32 rows each, and
// small enough that a slice of Z spans less than 2^31 bytes (the kernel
// addresses one slice through a 32-bit buffer offset).
// Rows per slice: about 512 workgroups per job, but at most 16 slices per
// column tile: the tile's last workgroup adds the slices, and with 64 of them
// (a 1024-column dB at M = 4096) that sum took longer than the products
// (the k_proj backward's dA/dB launch: 24 us).
int64_t thin_tn_slice_rows(int64_t M, int64_t P, int r) {
  (void)r;
  const int64_t pt = (P + TN_COLS - 1) / TN_COLS;
  const int64_t S = std::min<int64_t>((512 + pt - 1) / pt, 16);
  int64_t slice = (M + S - 1) / S;
  slice = (slice + 31) / 32 * 32;
  const int64_t cap = ((((int64_t)1 << 31) - 1) / (2 * P)) / 32 * 32;
  if (slice > cap) slice = cap;
  if (slice < 32) slice = 32;
  return slice;
}

int thin_tn_slices(int64_t M, int64_t P, int r) {
  const int64_t slice = thin_tn_slice_rows(M, P, r);
  return (int)((M + slice - 1) / slice);
}

// Row length of the staged (sV)^T: every slice's rows exist (zero past M).
int64_t thin_tn_rows_padded(int64_t M, int64_t P, int r) {
  return (int64_t)thin_tn_slices(M, P, r) * thin_tn_slice_rows(M, P, r);
}

hipError_t launch_thin_tn2(const ThinTn& a, const ThinTn& b, int64_t M, int r,
                           unsigned* arrivals, hipStream_t st) {
  const int nj = (r + 15) / 16;
  TnJob job[2];
  const ThinTn* in[2] = {&a, &b};
  int s_max = 1;
  for (int k = 0; k < 2; ++k) {
    const ThinTn& x = *in[k];
    TnJob& j = job[k];
    j.Z = x.Z;
    j.vt = x.vt;
    j.Mp = thin_tn_rows_padded(M, x.P, r);
    j.P = x.P;
    j.slice = thin_tn_slice_rows(M, x.P, r);
    j.S = thin_tn_slices(M, x.P, r);
    j.tiles = x.Z ? (int)((x.P + TN_COLS - 1) / TN_COLS) : 0;
    j.part = x.part;
    j.out = x.out;
    j.transposed = x.transposed ? 1 : 0;
    j.zmask = x.zmask;
    if (j.tiles > 0) s_max = std::max(s_max, j.S);
  }
  const int tiles = job[0].tiles + job[1].tiles;
  if (tiles == 0) return hipSuccess;
  // slices added by the last workgroup of each tile (one arrival counter per
  // tile), else by a second launch
  unsigned* ctr = tiles <= kTnMaxTiles ? arrivals : nullptr;
  const bool mask = (job[0].tiles > 0 && job[0].zmask) || (job[1].tiles > 0 && job[1].zmask);
  const size_t lds = (size_t)TN_NST * (32 * TN_ROWB + 2 * 16 * nj * 64 + (mask ? 32 * 16 : 0));
  const dim3 grid((unsigned)tiles, (unsigned)s_max);
#define QN_TN(NJ)                                                                              \
  if (mask)                                                                                    \
    hipLaunchKernelGGL((k_thin_tn<NJ, true>), grid, dim3(kThreads), lds, st, job[0], job[1], M, \
                       r, ctr);                                                                \
  else                                                                                         \
    hipLaunchKernelGGL((k_thin_tn<NJ, false>), grid, dim3(kThreads), lds, st, job[0], job[1], M, \
                       r, ctr)
  switch (nj) {
    case 1: QN_TN(1); break;
    case 2: QN_TN(2); break;
    case 3: QN_TN(3); break;
    default: QN_TN(4); break;
  }
#undef QN_TN
  if (ctr) return hipGetLastError();
  TnSum sum[2];
  int64_t count = 0;
  for (int k = 0; k < 2; ++k) {
    const ThinTn& x = *in[k];
    sum[k] = TnSum{x.part, x.Z ? x.P : 0, job[k].S, x.transposed, x.out};
    count += sum[k].P * r;
  }
  hipLaunchKernelGGL(k_sum_slices_tn, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                     sum[0], sum[1], r);
  return hipGetLastError();
}

}  // namespace qn
