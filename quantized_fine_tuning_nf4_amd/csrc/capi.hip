// C ABI of the QLoRA NF4 library: argument checks, workspace layout and
// launch order.  Every call checks its arguments on the host first and
// launches nothing on error.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/qlora_nf4.h"
#include "qn_device.h"
#include "qn_internal.h"

namespace {

using namespace qn;

// Carves 256-byte aligned pieces out of a caller workspace; with a null
// base it only measures.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    used = (used + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t blocks_of(int64_t n) { return (n + kBlock - 1) / kBlock; }
int64_t groups_of(int64_t nb) { return (nb + kGroup - 1) / kGroup; }
int64_t pow2_at_least(int64_t v) {
  int64_t p = 1;
  while (p < v) p *= 2;
  return p;
}

qn_status from_hip(hipError_t e) { return e == hipSuccess ? QN_OK : QN_EDEVICE; }

struct QuantWs {
  float* absmax;
  double* part;
  int64_t part_len;
  int* bad;   // [ng] per-group flags
  int* flag;  // the synchronous call's flag
  float* mean;  // the mean of a call without double quantization (unused)
};

QuantWs carve_quant(Carver& c, int64_t n) {
  const int64_t nb = blocks_of(n), ng = groups_of(nb);
  QuantWs w;
  c.take<unsigned>(kArrivalWords);  // left alone: a workspace may be shared with linear calls
  w.absmax = c.take<float>(nb);
  w.part_len = pow2_at_least(ng);
  w.part = c.take<double>(w.part_len);
  w.bad = c.take<int>(ng);
  w.flag = c.take<int>(1);
  w.mean = c.take<float>(1);
  return w;
}

qn_status check_state(const qn_nf4dq* w) {
  if (!w || !w->packed) return QN_EINVAL;
  if (w->codebook != QN_CODE_NF4 && w->codebook != QN_CODE_FP4) return QN_EINVAL;
  if (!w->absmax && (!w->qscale || !w->scale2 || !w->offset)) return QN_EINVAL;
  if (w->rows < 1 || w->cols < 1) return QN_EINVAL;
  if (w->rows > (INT64_MAX / 2) / w->cols) return QN_EINVAL;
  if (!aligned16(w->packed)) return QN_EALIGN;
  if (w->absmax ? !aligned16(w->absmax)
                : (!aligned16(w->qscale) || !aligned16(w->scale2) || !aligned16(w->offset)))
    return QN_EALIGN;
  return QN_OK;
}


// Largest M and weight dimension the linear calls take: the kernels address
// buffers through 32-bit offsets from a row or slice base, which these
// bounds keep below 2^31 bytes.
constexpr int64_t kMaxRowsM = (int64_t)1 << 23;
constexpr int64_t kMaxDim = (int64_t)1 << 20;

qn_status check_linear(const qn_nf4dq* w, int64_t M, int r) {
  qn_status s = check_state(w);
  if (s != QN_OK) return s;
  if (w->cols % kBlock != 0 || w->rows % 8 != 0) return QN_EINVAL;
  if (w->rows > kMaxDim || w->cols > kMaxDim) return QN_EINVAL;
  if (r < 1 || r > 64) return QN_EINVAL;
  if (M < 0 || M > kMaxRowsM) return QN_EINVAL;
  return QN_OK;
}

WState to_state(const qn_nf4dq* w) {
  return WState{w->packed, w->qscale, w->scale2, w->offset, w->rows, w->cols, w->absmax,
                w->codebook};
}

// Large batches (enough 128 x 128 output tiles to fill the chip) take the
// weight through a bf16 copy in the workspace and a plain bf16 GEMM (256 x 256
// tiles where there are enough of those, else 128 x 128); smaller ones
// dequantize inside the GEMM.  At the decoder layer's k_proj shape (M = 4096,
// 1024 x 4096) the dequantizing GEMM re-read its operands 6.5 times and ran
// at a tenth of the bf16 peak.
bool dense_path(int64_t M, int64_t out_cols) {
  return M > 0 && ((M + 127) / 128) * ((out_cols + 127) / 128) >= 240;
}
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

struct FwdWs {
  unsigned* arrivals;  // [kArrivalWords] arrival counters (zero between calls)
  float* u;      // [M, r] when the caller gives no u_out
  float* upart;  // [S, M, r] when S > 1
  int S;
  uint16_t* wd;  // [rows, cols] bf16 Qhat(W) (dense path)
  float* dpart;  // [dS, M, rows] decode partial sums (decode path)
  float* dupart; // [dS, M, r] decode partials of u
  int dS;
  DecodeTiles dt;  // one-kernel decode tiling (dt.rgt == 0: not used)
  float* tpart;    // [dt.S, M, rows] its partial sums
  float* tupart;   // [dt.bands, dt.S, 256] its partials of u
  int dbr;         // rows per band of the whole-row decode kernel (0: not used)
};

// dropout: the adapter branch reads a masked x, which the decode kernels
// (one set of x fragments for both products) do not take; such forwards use
// the GEMM routes.  Every route takes every state format.
FwdWs carve_fwd(Carver& c, int64_t M, int64_t rows, int64_t cols, int r, bool need_u,
                bool counters = true, bool dropout = false) {
  FwdWs f;
  f.arrivals = counters ? c.take<unsigned>(kArrivalWords) : nullptr;
  const bool dec = rows > 0 && !dropout;
  f.dbr = dec ? decode_rows_band(M, rows, cols, r) : 0;
  f.dt = dec && f.dbr == 0 ? decode_tiles(M, rows, cols, r) : DecodeTiles{0, 0, 0};
  f.dS = dec && f.dbr == 0 && f.dt.rgt == 0 ? decode_slices(M, rows, cols) : 0;
  const bool decode = f.dbr > 0 || f.dt.rgt > 0 || f.dS > 0;  // u from the decode kernels
  f.S = thin_nt_slices(M, cols);
  f.u = need_u ? c.take<float>((size_t)M * r) : nullptr;
  f.upart = f.S > 1 && !decode ? c.take<float>((size_t)f.S * M * r) : nullptr;
  f.wd = rows > 0 && M > 0 && !decode && dense_path(M, rows)
             ? c.take<uint16_t>((size_t)rows * cols)
             : nullptr;
  f.dpart = f.dS > 0 ? c.take<float>((size_t)f.dS * M * rows) : nullptr;
  f.dupart = f.dS > 0 ? c.take<float>((size_t)f.dS * M * r) : nullptr;
  f.tpart = f.dt.rgt > 0 ? c.take<float>((size_t)f.dt.S * M * round_up(rows, 4)) : nullptr;
  f.tupart = f.dt.rgt > 0 ? c.take<float>((size_t)f.dt.bands * f.dt.S * 256) : nullptr;
  return f;
}

struct BwdWs {
  unsigned* arrivals;  // [kArrivalWords] arrival counters
  FwdWs fu;      // recomputed u (if not saved)
  uint16_t* Bt;  // [r, rows]
  float* v;      // [M, r]
  float* vpart;  // [Sv, M, r]
  int Sv;
  float* dBpart;  // [Sb, rows, r]
  int Sb;
  uint16_t* su;   // [2][rp][Mpb] (s u)^T high and remainder parts
  float* dApart;  // [Sa, cols, r]
  int Sa;
  uint16_t* sv;   // [2][rp][Mpa] (s v)^T
  uint16_t* wt;   // [cols, ldt] bf16 Qhat(W)^T (dense path)
  int64_t ldt;
  uint16_t* At;   // [cols, r] A^T (dense path)
};

BwdWs carve_bwd(Carver& c, int64_t M, int64_t rows, int64_t cols, int r, bool need_u) {
  BwdWs b;
  b.arrivals = c.take<unsigned>(kArrivalWords);
  if (need_u) {
    b.fu = carve_fwd(c, M, 0, cols, r, true, false);
  } else {
    b.fu = FwdWs{};
    b.fu.S = 1;
  }
  b.Bt = c.take<uint16_t>((size_t)r * rows);
  b.Sv = thin_nt_slices(M, rows);
  b.v = c.take<float>((size_t)M * r);
  b.vpart = b.Sv > 1 ? c.take<float>((size_t)b.Sv * M * r) : nullptr;
  const int64_t rp = 16 * ((r + 15) / 16);
  b.Sb = thin_tn_slices(M, rows, r);
  b.dBpart = c.take<float>((size_t)b.Sb * rows * r);
  b.su = c.take<uint16_t>((size_t)2 * rp * thin_tn_rows_padded(M, rows, r));
  b.Sa = thin_tn_slices(M, cols, r);
  b.dApart = c.take<float>((size_t)b.Sa * cols * r);
  b.sv = c.take<uint16_t>((size_t)2 * rp * thin_tn_rows_padded(M, cols, r));
  b.ldt = round_up(rows, 64);
  const bool dense = M > 0 && dense_path(M, cols);
  b.wt = dense ? c.take<uint16_t>((size_t)cols * b.ldt) : nullptr;
  b.At = dense ? c.take<uint16_t>((size_t)cols * r) : nullptr;
  return b;
}

// The adapter branch's options (nullable: alpha / r, no dropout).
struct Lora {
  float s;               // branch scale
  const uint8_t* mask;   // dropout keep mask (nullable)
};

qn_status lora_options(const qn_lora_opts* o, float alpha, int r, Lora* out) {
  out->s = alpha / (float)r;
  out->mask = nullptr;
  if (!o) return QN_OK;
  if (o->rslora != 0 && o->rslora != 1) return QN_EINVAL;
  // rsLoRA: alpha / sqrt(r) (sqrtf is correctly rounded)
  if (o->rslora) out->s = alpha / sqrtf((float)r);
  if (o->dropout_mask) {
    const float p = o->dropout_p;
    if (!(p >= 0.f && p < 1.f)) return QN_EINVAL;
    if (!aligned16(o->dropout_mask)) return QN_EALIGN;  // read in 8- and 16-byte pieces
    out->mask = o->dropout_mask;
    out->s = out->s / (1.f - p);  // inverted dropout, folded into the scale
  } else if (o->dropout_p != 0.f) {
    return QN_EINVAL;
  }
  return QN_OK;
}

// The forward, on a workspace of ws_bytes at ws; clear: zero the arrival
// counters with a kernel before the launch that counts on them.
qn_status forward(const qn_nf4dq* w, const uint16_t* x, int64_t M, const uint16_t* A,
                  const uint16_t* B, int r, const Lora& lo, uint16_t* y, float* u_out,
                  void* workspace, size_t workspace_bytes, void* stream, bool clear) {
  qn_status s = check_linear(w, M, r);
  if (s != QN_OK) return s;
  if (M == 0) return QN_OK;
  if (!x || !A || !B || !y) return QN_EINVAL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) ||
      (u_out && !aligned16(u_out)))
    return QN_EALIGN;
  Carver probe(nullptr);
  const bool drop = lo.mask != nullptr;
  carve_fwd(probe, M, w->rows, w->cols, r, u_out == nullptr, true, drop);
  if (probe.used > 0) {
    if (!workspace) return QN_EINVAL;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return QN_EALIGN;
    if (workspace_bytes < probe.used) return QN_EWORKSPACE;
  }
  Carver c(workspace);
  FwdWs f = carve_fwd(c, M, w->rows, w->cols, r, u_out == nullptr, true, drop);
  float* u = u_out ? u_out : f.u;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float scale = lo.s;
  const int64_t N = w->rows, K = w->cols;
  if (f.dbr > 0)  // decode-sized batch, whole rows per workgroup
    return from_hip(launch_decode_rows(to_state(w), x, M, A, B, r, scale, y, u, f.dbr, st));
  if (f.dt.rgt > 0) {  // decode-sized batch, one kernel over column slices
    hipError_t e = hipSuccess;
    if (clear) e = launch_fill_zero(reinterpret_cast<float*>(f.arrivals), kArrivalWords, st);
    if (e == hipSuccess)
      e = launch_decode_tile(to_state(w), x, M, A, B, r, scale, y, u, f.dt, f.arrivals, f.tpart,
                             f.tupart, st);
    return from_hip(e);
  }
  if (f.dpart)  // decode-sized batch: u and the product in two kernels
    return from_hip(launch_decode_fwd(to_state(w), x, M, A, B, r, scale, y, u, f.dpart,
                                      f.dupart, f.dS, st));
  // dense path: the slices of u are added by spare workgroups of the
  // dequantization launch that follows
  const bool fold = f.wd && f.S > 1;
  hipError_t e = launch_thin_nt(x, A, M, K, r, u, f.upart, f.S, st, !fold, false,
                                Clear{nullptr, 0}, lo.mask);
  if (f.wd) {
    if (e == hipSuccess)
      e = launch_dequant(w->packed, w->qscale, w->scale2, w->offset, N * K, true, f.wd, st,
                         fold ? SliceSum{f.upart, M * (int64_t)r, f.S, u} : SliceSum{},
                         w->codebook, w->absmax);
    if (e == hipSuccess) e = launch_gemm_nt(x, K, K, f.wd, K, M, N, u, B, r, scale, y, st);
  } else if (e == hipSuccess) {
    e = launch_qgemm_fwd(to_state(w), x, M, u, B, r, scale, y, st);
  }
  return from_hip(e);
}

// Scratch of qlora_linear_fwd_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes its name to
// a kernel (on the host it is only a stand-in for the symbol): it uses the
// device address hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = QN_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of the scratch array (looked up once per device).
qn_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QN_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QN_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QN_OK;
}

}  // namespace

extern "C" {

static_assert(QN_ARRIVAL_BYTES == 4 * kArrivalWords, "arrival counter page");

int qn_abi_version(void) { return QN_ABI_VERSION; }

const char* qn_status_str(qn_status s) {
  switch (s) {
    case QN_OK: return "ok";
    case QN_EINVAL: return "invalid argument";
    case QN_ENONFINITE: return "non-finite value in the weight";
    case QN_EALIGN: return "pointer not 16-byte aligned";
    case QN_EWORKSPACE: return "workspace too small";
    case QN_EDEVICE: return "HIP runtime error";
  }
  return "unknown status";
}

void qn_nf4_codebook(float out[16]) {
  for (int k = 0; k < 16; ++k) {
    uint32_t b = kNF4Bits[k];
    std::memcpy(&out[k], &b, 4);
  }
}

void qn_fp4_codebook(float out[16]) {
  for (int k = 0; k < 16; ++k) {
    uint32_t b = kFP4Bits[k];
    std::memcpy(&out[k], &b, 4);
  }
}

size_t nf4_quantize_dq_workspace(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || rows > INT64_MAX / 2 / cols) return 0;
  Carver c(nullptr);
  carve_quant(c, rows * cols);
  return c.used;
}

qn_status nf4_quantize_dq(const float* W, int64_t rows, int64_t cols, uint8_t* packed,
                          uint8_t* qscale, float* scale2, float* offset, int* nonfinite,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return qn_quantize(W, rows, cols, QN_CODE_NF4, 1, packed, qscale, scale2, offset, nullptr,
                     nonfinite, workspace, workspace_bytes, stream);
}

qn_status qn_quantize(const float* W, int64_t rows, int64_t cols, int codebook,
                      int double_quant, uint8_t* packed, uint8_t* qscale, float* scale2,
                      float* offset, float* absmax, int* nonfinite, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (codebook != QN_CODE_NF4 && codebook != QN_CODE_FP4) return QN_EINVAL;
  if (!W || !packed || !workspace) return QN_EINVAL;
  if (double_quant ? (!qscale || !scale2 || !offset) : !absmax) return QN_EINVAL;
  if (rows < 1 || cols < 1 || rows > INT64_MAX / 2 / cols) return QN_EINVAL;
  if (!aligned16(W) || !aligned16(packed) || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      (reinterpret_cast<uintptr_t>(nonfinite) & 3u))
    return QN_EALIGN;
  if (double_quant ? (!aligned16(qscale) || !aligned16(scale2) || !aligned16(offset))
                   : !aligned16(absmax))
    return QN_EALIGN;
  const int64_t n = rows * cols;
  if (workspace_bytes < nf4_quantize_dq_workspace(rows, cols)) return QN_EWORKSPACE;
  Carver c(workspace);
  QuantWs ws = carve_quant(c, n);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_quantize(W, n, packed, qscale, scale2, offset, ws.absmax, ws.part,
                                 ws.part_len, ws.bad, nonfinite ? nonfinite : ws.flag, st,
                                 codebook, double_quant ? nullptr : absmax, ws.mean);
  if (e != hipSuccess) return QN_EDEVICE;
  if (nonfinite) return QN_OK;  // asynchronous: the caller reads the flag
  int bad = 0;
  e = hipMemcpyAsync(&bad, ws.flag, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return QN_EDEVICE;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return QN_EDEVICE;
  return bad ? QN_ENONFINITE : QN_OK;
}

qn_status nf4_dequantize(const qn_nf4dq* w, qn_dtype out_dtype, void* out, void* stream) {
  qn_status s = check_state(w);
  if (s != QN_OK) return s;
  if (!out || (out_dtype != QN_F32 && out_dtype != QN_BF16)) return QN_EINVAL;
  if (!aligned16(out)) return QN_EALIGN;
  return from_hip(launch_dequant(w->packed, w->qscale, w->scale2, w->offset, w->rows * w->cols,
                                 out_dtype == QN_BF16, out, static_cast<hipStream_t>(stream),
                                 SliceSum{}, w->codebook, w->absmax, /*nt=*/true));
}

size_t qlora_linear_workspace_ex(int64_t M, int64_t rows, int64_t cols, int r, int backward,
                                 const qn_lora_opts* opts) {
  if (M < 0 || rows < 1 || cols < 1 || r < 1 || r > 64) return 0;
  const bool drop = opts && opts->dropout_mask;
  Carver c(nullptr);
  if (backward)
    carve_bwd(c, M, rows, cols, r, true);
  else
    carve_fwd(c, M, rows, cols, r, true, true, drop);
  return c.used;
}

size_t qlora_linear_workspace(int64_t M, int64_t rows, int64_t cols, int r, int backward) {
  return qlora_linear_workspace_ex(M, rows, cols, r, backward, nullptr);
}

size_t qlora_linear_workspace_state(const qn_nf4dq* w, int64_t M, int r, int backward,
                                    const qn_lora_opts* opts) {
  if (!w || M < 0 || w->rows < 1 || w->cols < 1 || r < 1 || r > 64) return 0;
  const bool drop = opts && opts->dropout_mask;
  Carver c(nullptr);
  if (backward)
    carve_bwd(c, M, w->rows, w->cols, r, true);
  else
    carve_fwd(c, M, w->rows, w->cols, r, true, true, drop);
  return c.used;
}

qn_status qlora_linear_fwd(const qn_nf4dq* w, const uint16_t* x, int64_t M, const uint16_t* A,
                           const uint16_t* B, int r, float alpha, uint16_t* y, float* u_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return qlora_linear_fwd_ex(w, x, M, A, B, r, alpha, nullptr, y, u_out, workspace,
                             workspace_bytes, stream);
}

qn_status qlora_linear_fwd_ex(const qn_nf4dq* w, const uint16_t* x, int64_t M, const uint16_t* A,
                              const uint16_t* B, int r, float alpha, const qn_lora_opts* opts,
                              uint16_t* y, float* u_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (r < 1 || r > 64) return QN_EINVAL;
  Lora lo;
  qn_status s = lora_options(opts, alpha, r, &lo);
  if (s != QN_OK) return s;
  return forward(w, x, M, A, B, r, lo, y, u_out, workspace, workspace_bytes, stream, false);
}

qn_status qlora_linear_fwd_noalloc(const qn_nf4dq* w, const uint16_t* x, int64_t M,
                                   const uint16_t* A, const uint16_t* B, int r, float alpha,
                                   uint16_t* y, float* u_out, void* stream) {
  qn_status s = check_linear(w, M, r);
  if (s != QN_OK) return s;
  if (M == 0) return QN_OK;
  Carver probe(nullptr);
  carve_fwd(probe, M, w->rows, w->cols, r, u_out == nullptr);
  if (probe.used > kStaticScratchBytes) return QN_EWORKSPACE;
  void* ptr = nullptr;
  s = static_scratch(&ptr);
  if (s != QN_OK) return s;
  // the array keeps what the last call left in it: its counters are cleared
  // by a kernel before the launch that counts on them
  return forward(w, x, M, A, B, r, Lora{alpha / (float)r, nullptr}, y, u_out, ptr,
                 kStaticScratchBytes, stream, true);
}



qn_status qlora_linear_bwd(const qn_nf4dq* w, const uint16_t* x, const uint16_t* dY, int64_t M,
                           const uint16_t* A, const uint16_t* B, int r, float alpha,
                           const float* u_saved, uint16_t* dX, float* dA, float* dB,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return qlora_linear_bwd_ex(w, x, dY, M, A, B, r, alpha, nullptr, u_saved, dX, dA, dB,
                             workspace, workspace_bytes, stream);
}

qn_status qlora_linear_bwd_ex(const qn_nf4dq* w, const uint16_t* x, const uint16_t* dY,
                              int64_t M, const uint16_t* A, const uint16_t* B, int r, float alpha,
                              const qn_lora_opts* opts, const float* u_saved, uint16_t* dX,
                              float* dA, float* dB, void* workspace, size_t workspace_bytes,
                              void* stream) {
  qn_status s = check_linear(w, M, r);
  if (s != QN_OK) return s;
  Lora lo;
  s = lora_options(opts, alpha, r, &lo);
  if (s != QN_OK) return s;
  const bool drop = lo.mask != nullptr;
  if (!A || !B || !dA || !dB) return QN_EINVAL;
  if (M > 0 && (!x || !dY)) return QN_EINVAL;
  if (!aligned16(x) || !aligned16(dY) || !aligned16(A) || !aligned16(B) || !aligned16(dA) ||
      !aligned16(dB) || (dX && !aligned16(dX)) || (u_saved && !aligned16(u_saved)))
    return QN_EALIGN;
  const int64_t N = w->rows, K = w->cols;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (M == 0) {
    // empty batch: the gradients of the adapters are zero
    hipError_t e = launch_fill_zero(dA, (int64_t)r * K, st);
    if (e == hipSuccess) e = launch_fill_zero(dB, N * (int64_t)r, st);
    return from_hip(e);
  }
  Carver probe(nullptr);
  carve_bwd(probe, M, N, K, r, u_saved == nullptr);
  if (!workspace) return QN_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return QN_EALIGN;
  if (workspace_bytes < probe.used) return QN_EWORKSPACE;
  Carver c(workspace);
  BwdWs b = carve_bwd(c, M, N, K, r, u_saved == nullptr);
  const float scale = lo.s;
  hipError_t e = hipSuccess;
  const float* u = u_saved;
  // an early launch of the call zeroes the arrival counters the adapter
  // gradients' launch counts on, so the backward never depends on what the
  // workspace held before
  Clear clr{b.arrivals, kArrivalWords};
  if (!u && e == hipSuccess) {
    e = launch_thin_nt(x, A, M, K, r, b.fu.u, b.fu.upart, b.fu.S, st, true, false, clr, lo.mask);
    clr = Clear{nullptr, 0};
    u = b.fu.u;
  }
  // v = G B as slices (added below); the product takes B as stored when it
  // can, else B^T made first
  const bool b_rows = thin_nt_rows_ok(M, N, r);
  if (e == hipSuccess && !b_rows) {
    if (clr.n) {  // (no earlier launch: a kernel, not a memset, for graph capture)
      e = launch_fill_zero(reinterpret_cast<float*>(clr.p), clr.n, st);
      clr = Clear{nullptr, 0};
    }
    BwdAux t{};
    t.B = B;
    t.Bt = b.Bt;
    t.N = N;
    t.r = r;
    e = launch_bwd_aux(t, st);
  }
  if (e == hipSuccess)
    e = launch_thin_nt(dY, b_rows ? B : b.Bt, M, N, r, b.v, b.vpart, b.Sv, st, false, b_rows,
                       clr);
  // the small jobs: v's slice sum, (s u)^T and (s v)^T split for the
  // transposed products, A^T for the dense dX product; in spare workgroups of
  // the transposed dequantization when there is one
  const bool dense_dx = dX && b.wt;
  BwdAux aux{};
  aux.A = A;
  aux.At = dense_dx ? b.At : nullptr;
  aux.K = K;
  aux.u = u;
  aux.su = b.su;
  aux.Mpu = thin_tn_rows_padded(M, N, r);
  aux.vpart = b.vpart;
  aux.Sv = b.Sv;
  aux.v = b.v;
  aux.sv = b.sv;
  aux.Mpv = thin_tn_rows_padded(M, K, r);
  aux.M = M;
  aux.r = r;
  aux.s = scale;
  if (e == hipSuccess) {
    if (dense_dx)
      e = launch_dequant_t(w->packed, w->qscale, w->scale2, w->offset, N, K, b.wt, b.ldt, aux,
                           st, w->codebook, w->absmax);
    else
      e = launch_bwd_aux(aux, st);
  }
  if (e == hipSuccess && dX) {
    // under dropout the branch's share is added masked after the base product
    const float sx = drop ? 0.f : scale;
    if (dense_dx)
      e = launch_gemm_nt(dY, N, N, b.wt, b.ldt, M, K, b.v, b.At, r, sx, dX, st);
    else
      e = launch_qgemm_dx(to_state(w), dY, M, b.v, A, r, sx, dX, st);
    if (e == hipSuccess && drop) e = launch_lora_masked_add(dX, b.v, A, lo.mask, M, K, r, scale, st);
  }
  // dB = s G^T u and dA = s v^T X in one launch (and their slice sums in one)
  if (e == hipSuccess)
    e = launch_thin_tn2(ThinTn{dY, b.su, N, dB, false, b.dBpart},
                        ThinTn{x, b.sv, K, dA, true, b.dApart, lo.mask}, M, r, b.arrivals,
                        st);
  return from_hip(e);
}

qn_status nf4_merge_lora(const qn_nf4dq* w, const uint16_t* A, const uint16_t* B, int r,
                         float alpha, float* out, void* stream) {
  qn_status s = check_state(w);
  if (s != QN_OK) return s;
  if (r < 1 || r > 64 || w->rows > kMaxDim * 64 || w->cols > kMaxDim * 64) return QN_EINVAL;
  if (!A || !B || !out) return QN_EINVAL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(out)) return QN_EALIGN;
  return from_hip(launch_merge(to_state(w), A, B, r, alpha / (float)r, out,
                               static_cast<hipStream_t>(stream), w->codebook, w->absmax));
}

qn_status adamw8_step(float* p, const float* g, int64_t n, uint8_t* m_codes, float* m_scales,
                      uint8_t* v_codes, float* v_scales, uint16_t* p_bf16,
                      const qn_adamw_hparams* h, void* stream) {
  if (n < 0 || !h || h->step < 1) return QN_EINVAL;
  if (n == 0) return QN_OK;
  if (!p || !g || !m_codes || !m_scales || !v_codes || !v_scales) return QN_EINVAL;
  if (!aligned16(p) || !aligned16(g) || !aligned16(m_codes) || !aligned16(v_codes) ||
      !aligned16(m_scales) || !aligned16(v_scales) || (p_bf16 && !aligned16(p_bf16)))
    return QN_EALIGN;
  if (!(h->beta1 >= 0.f && h->beta1 < 1.f && h->beta2 >= 0.f && h->beta2 < 1.f)) return QN_EINVAL;
  // the derived scalars in fp64 from the fp32 hyperparameters, rounded once
  const double b1 = h->beta1, b2 = h->beta2, t = (double)h->step;
  AdamScalars s;
  s.lr = h->lr;
  s.b1 = h->beta1;
  s.b2 = h->beta2;
  s.omb1 = (float)(1.0 - b1);
  s.omb2 = (float)(1.0 - b2);
  s.eps = h->eps;
  s.c1 = (float)(1.0 - std::pow(b1, t));
  s.c2 = (float)(1.0 - std::pow(b2, t));
  s.decay = (float)(1.0 - (double)h->lr * (double)h->weight_decay);
  return from_hip(launch_adamw8(p, g, n, m_codes, m_scales, v_codes, v_scales, p_bf16, s,
                                static_cast<hipStream_t>(stream)));
}

int qlora_linear_route(int64_t M, int64_t rows, int64_t cols, int r, int backward) {
  if (M < 1 || M > kMaxRowsM || rows < 8 || cols < kBlock || rows % 8 != 0 ||
      cols % kBlock != 0 || rows > kMaxDim || cols > kMaxDim || r < 1 || r > 64)
    return -1;
  const int64_t out_cols = backward ? cols : rows;
  if (!backward) {
    if (decode_rows_band(M, rows, cols, r) > 0) return QN_ROUTE_DECODE_ROWS;
    if (decode_tiles(M, rows, cols, r).rgt > 0) return QN_ROUTE_DECODE_TILES;
    if (decode_slices(M, rows, cols) > 0) return QN_ROUTE_DECODE_SPLIT;
  }
  if (dense_path(M, out_cols)) return QN_ROUTE_DENSE;
  return M <= 32 ? QN_ROUTE_FUSED_SMALL : QN_ROUTE_FUSED;
}

qn_status lora_linear_bf16(const uint16_t* x, int64_t M, const uint16_t* W, int64_t rows,
                           int64_t cols, const float* V, const uint16_t* L, int r, float alpha,
                           uint16_t* y, void* stream) {
  if (rows < 1 || cols < 1 || M < 0 || r < 1 || r > 64) return QN_EINVAL;
  if (cols % kBlock != 0 || rows % 8 != 0) return QN_EINVAL;
  if (M == 0) return QN_OK;
  if (!x || !W || !V || !L || !y) return QN_EINVAL;
  if (!aligned16(x) || !aligned16(W) || !aligned16(V) || !aligned16(L) || !aligned16(y))
    return QN_EALIGN;
  return from_hip(launch_gemm_nt(x, cols, cols, W, cols, M, rows, V, L, r, alpha / (float)r, y,
                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"
