"""QLoRA NF4 hot path on one AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libqlora_nf4.so`` (C ABI in
``include/qlora_nf4.h``).  The functions carry the C names and do argument
marshalling only -- shape/dtype checks, output and workspace allocation
through PyTorch, the current HIP stream -- every step of the computation
runs in the library's HIP kernels.  There is no CPU fallback: if the library
is missing or no GPU is present, calls raise.

    st = nf4_quantize_dq(W)                       # W: fp32 [d_out, d_in] on cuda
    Wd = nf4_dequantize(st, torch.bfloat16)
    y, u = qlora_linear_fwd(st, x, A, B, alpha)   # y = x Qhat(W)^T + (alpha/r) x A^T B^T
    dX, dA, dB = qlora_linear_bwd(st, x, dY, A, B, alpha, u)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")

QN_OK, QN_EINVAL, QN_ENONFINITE, QN_EALIGN, QN_EWORKSPACE, QN_EDEVICE = range(6)
QN_F32, QN_BF16 = 0, 1

EXPORTS = ["qn_abi_version", "qn_status_str", "qn_nf4_codebook", "nf4_quantize_dq_workspace",
           "nf4_quantize_dq", "nf4_dequantize", "qlora_linear_workspace", "qlora_linear_fwd",
           "qlora_linear_bwd", "lora_linear_bf16", "qlora_linear_route",
           "qlora_linear_fwd_noalloc", "nf4_merge_lora", "qlora_linear_workspace_ex",
           "qlora_linear_fwd_ex", "qlora_linear_bwd_ex", "qn_quantize",
           "qlora_linear_workspace_state", "qn_fp4_codebook", "adamw8_step"]
ROUTES = {1: "decode_rows", 2: "decode_tiles", 3: "decode_split", 4: "fused_small", 5: "fused",
          6: "dense"}


class QNError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class _LoraOpts(ctypes.Structure):
    _fields_ = [("rslora", ctypes.c_int), ("dropout_mask", ctypes.c_void_p),
                ("dropout_p", ctypes.c_float)]


class _AdamHP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("step", ctypes.c_int64)]


class _NF4DQ(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("qscale", ctypes.c_void_p),
                ("scale2", ctypes.c_void_p), ("offset", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("absmax", ctypes.c_void_p), ("codebook", ctypes.c_int32)]


CODEBOOKS = {"nf4": 0, "fp4": 1}


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with "
                           "`python quantized_fine_tuning_nf4_amd/build.py`")
    L = ctypes.CDLL(path)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.qn_abi_version.restype = ctypes.c_int
    L.qn_status_str.argtypes = [ctypes.c_int]
    L.qn_status_str.restype = ctypes.c_char_p
    L.qn_nf4_codebook.argtypes = [P]
    L.qn_fp4_codebook.argtypes = [P]
    L.nf4_quantize_dq_workspace.argtypes = [I64, I64]
    L.nf4_quantize_dq_workspace.restype = SZ
    L.nf4_quantize_dq.argtypes = [P, I64, I64, P, P, P, P, P, P, SZ, P]
    L.nf4_quantize_dq.restype = ctypes.c_int
    L.qn_quantize.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P, P, SZ,
                              P]
    L.qn_quantize.restype = ctypes.c_int
    L.nf4_dequantize.argtypes = [ctypes.POINTER(_NF4DQ), ctypes.c_int, P, P]
    L.nf4_dequantize.restype = ctypes.c_int
    L.qlora_linear_workspace.argtypes = [I64, I64, I64, ctypes.c_int, ctypes.c_int]
    L.qlora_linear_workspace.restype = SZ
    L.qlora_linear_fwd.argtypes = [ctypes.POINTER(_NF4DQ), P, I64, P, P, ctypes.c_int,
                                   ctypes.c_float, P, P, P, SZ, P]
    L.qlora_linear_fwd.restype = ctypes.c_int
    L.qlora_linear_bwd.argtypes = [ctypes.POINTER(_NF4DQ), P, P, I64, P, P, ctypes.c_int,
                                   ctypes.c_float, P, P, P, P, P, SZ, P]
    L.qlora_linear_bwd.restype = ctypes.c_int
    L.lora_linear_bf16.argtypes = [P, I64, P, I64, I64, P, P, ctypes.c_int, ctypes.c_float, P, P]
    L.lora_linear_bf16.restype = ctypes.c_int
    L.qlora_linear_fwd_noalloc.argtypes = [ctypes.POINTER(_NF4DQ), P, I64, P, P, ctypes.c_int,
                                           ctypes.c_float, P, P, P]
    L.qlora_linear_fwd_noalloc.restype = ctypes.c_int
    OP = ctypes.POINTER(_LoraOpts)
    L.qlora_linear_workspace_ex.argtypes = [I64, I64, I64, ctypes.c_int, ctypes.c_int, OP]
    L.qlora_linear_workspace_ex.restype = SZ
    L.qlora_linear_workspace_state.argtypes = [ctypes.POINTER(_NF4DQ), I64, ctypes.c_int,
                                               ctypes.c_int, OP]
    L.qlora_linear_workspace_state.restype = SZ
    L.qlora_linear_fwd_ex.argtypes = [ctypes.POINTER(_NF4DQ), P, I64, P, P, ctypes.c_int,
                                      ctypes.c_float, OP, P, P, P, SZ, P]
    L.qlora_linear_fwd_ex.restype = ctypes.c_int
    L.qlora_linear_bwd_ex.argtypes = [ctypes.POINTER(_NF4DQ), P, P, I64, P, P, ctypes.c_int,
                                      ctypes.c_float, OP, P, P, P, P, P, SZ, P]
    L.qlora_linear_bwd_ex.restype = ctypes.c_int
    L.nf4_merge_lora.argtypes = [ctypes.POINTER(_NF4DQ), P, P, ctypes.c_int, ctypes.c_float, P, P]
    L.adamw8_step.argtypes = [P, P, I64, P, P, P, P, P, ctypes.POINTER(_AdamHP), P]
    L.adamw8_step.restype = ctypes.c_int
    L.nf4_merge_lora.restype = ctypes.c_int
    L.qlora_linear_route.argtypes = [I64, I64, I64, ctypes.c_int, ctypes.c_int]
    L.qlora_linear_route.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != QN_OK:
        msg = load_library().qn_status_str(status).decode()
        raise QNError(status, msg)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


@dataclass
class NF4State:
    """Quantized weight on the device: packed 4-bit codes and either the
    double-quantized block scales (E4M3 scale codes, second-level scales and
    the mean offset) or, with double quantization off, the fp32 block scales
    (absmax).  codebook: 0 NF4, 1 FP4."""
    packed: torch.Tensor                  # uint8 [32*nb]
    qscale: torch.Tensor | None           # uint8 [nb]
    scale2: torch.Tensor | None           # float32 [ng]
    offset: torch.Tensor | None           # float32 [1]
    rows: int
    cols: int
    absmax: torch.Tensor | None = None    # float32 [nb] (double quantization off)
    codebook: int = 0

    def c_struct(self) -> _NF4DQ:
        return _NF4DQ(self.packed.data_ptr(), _ptr(self.qscale), _ptr(self.scale2),
                      _ptr(self.offset), self.rows, self.cols, _ptr(self.absmax), self.codebook)

    @property
    def device(self):
        return self.packed.device

    def nbytes(self) -> int:
        if self.absmax is not None:
            return self.packed.numel() + 4 * self.absmax.numel()
        return (self.packed.numel() + self.qscale.numel() + 4 * self.scale2.numel()
                + 4 * self.offset.numel())


def codebook(name: str = "nf4") -> list:
    out = (ctypes.c_float * 16)()
    L = load_library()
    (L.qn_fp4_codebook if name == "fp4" else L.qn_nf4_codebook)(out)
    return list(out)


def state_sizes(rows: int, cols: int):
    n = rows * cols
    nb = (n + 63) // 64
    ng = (nb + 255) // 256
    return nb, ng


def empty_state(rows: int, cols: int, device) -> NF4State:
    nb, ng = state_sizes(rows, cols)
    return NF4State(torch.empty(32 * nb, dtype=torch.uint8, device=device),
                    torch.empty(nb, dtype=torch.uint8, device=device),
                    torch.empty(ng, dtype=torch.float32, device=device),
                    torch.empty(1, dtype=torch.float32, device=device), rows, cols)


def nf4_quantize_dq(W: torch.Tensor, out: NF4State | None = None,
                    workspace: torch.Tensor | None = None,
                    nonfinite: torch.Tensor | None = None) -> NF4State:
    """NF4 block-64 quantisation + double quantisation of an fp32 weight
    [d_out, d_in] (a 1-D tensor is one row).  Without `nonfinite` the call
    synchronizes and raises QNError on NaN/Inf; with `nonfinite` (an int32
    CUDA tensor of one element) it stays asynchronous and writes 1 or 0 there."""
    L = load_library()
    W = _dev(W, torch.float32, "W")
    rows, cols = (W.shape[0], W.shape[1]) if W.dim() == 2 else (1, W.numel())
    if W.dim() not in (1, 2):
        raise ValueError("W must be 1-D or 2-D")
    st = out if out is not None else empty_state(rows, cols, W.device)
    ws_bytes = L.nf4_quantize_dq_workspace(rows, cols)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 1), dtype=torch.uint8,
                                                             device=W.device)
    if nonfinite is not None:
        _dev(nonfinite, torch.int32, "nonfinite")
        if nonfinite.numel() != 1:
            raise ValueError("nonfinite must hold one int32")
    _check(L.nf4_quantize_dq(W.data_ptr(), rows, cols, st.packed.data_ptr(),
                             st.qscale.data_ptr(), st.scale2.data_ptr(), st.offset.data_ptr(),
                             _ptr(nonfinite), ws.data_ptr(), ws.numel(), _stream(W.device)))
    return st


def qn_quantize(W: torch.Tensor, codebook: str = "nf4", double_quant: bool = True,
                workspace: torch.Tensor | None = None,
                nonfinite: torch.Tensor | None = None) -> NF4State:
    """Block-64 4-bit quantisation with NF4 or FP4 codes, with or without
    double quantisation of the block scales (see nf4_quantize_dq for the
    rest)."""
    L = load_library()
    W = _dev(W, torch.float32, "W")
    if W.dim() not in (1, 2):
        raise ValueError("W must be 1-D or 2-D")
    rows, cols = (W.shape[0], W.shape[1]) if W.dim() == 2 else (1, W.numel())
    cb = CODEBOOKS[codebook]
    nb, ng = state_sizes(rows, cols)
    dev = W.device
    if double_quant:
        st = NF4State(torch.empty(32 * nb, dtype=torch.uint8, device=dev),
                      torch.empty(nb, dtype=torch.uint8, device=dev),
                      torch.empty(ng, dtype=torch.float32, device=dev),
                      torch.empty(1, dtype=torch.float32, device=dev), rows, cols, None, cb)
    else:
        st = NF4State(torch.empty(32 * nb, dtype=torch.uint8, device=dev), None, None, None,
                      rows, cols, torch.empty(nb, dtype=torch.float32, device=dev), cb)
    ws_bytes = L.nf4_quantize_dq_workspace(rows, cols)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 1), dtype=torch.uint8,
                                                             device=dev)
    if nonfinite is not None:
        _dev(nonfinite, torch.int32, "nonfinite")
    _check(L.qn_quantize(W.data_ptr(), rows, cols, cb, int(bool(double_quant)),
                         st.packed.data_ptr(), _ptr(st.qscale), _ptr(st.scale2), _ptr(st.offset),
                         _ptr(st.absmax), _ptr(nonfinite), ws.data_ptr(), ws.numel(),
                         _stream(dev)))
    return st


def nf4_dequantize(st: NF4State, dtype=torch.bfloat16, out: torch.Tensor | None = None):
    L = load_library()
    code = {torch.float32: QN_F32, torch.bfloat16: QN_BF16}[dtype]
    if out is None:
        out = torch.empty((st.rows, st.cols), dtype=dtype, device=st.device)
    _dev(out, dtype, "out")
    s = st.c_struct()
    _check(L.nf4_dequantize(ctypes.byref(s), code, out.data_ptr(), _stream(st.device)))
    return out


def nf4_merge_lora(st: NF4State, A: torch.Tensor, B: torch.Tensor, alpha: float,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """Qhat(W) + (alpha/r) B A as an fp32 [d_out, d_in] tensor (the merged
    weight; requantize it with nf4_quantize_dq)."""
    L = load_library()
    A = _dev(A, torch.bfloat16, "A")
    B = _dev(B, torch.bfloat16, "B")
    r = A.shape[0]
    if A.dim() != 2 or A.shape[1] != st.cols or B.shape != (st.rows, r):
        raise ValueError(f"A must be [r, {st.cols}] and B [{st.rows}, r]")
    if out is None:
        out = torch.empty((st.rows, st.cols), dtype=torch.float32, device=st.device)
    _dev(out, torch.float32, "out")
    s = st.c_struct()
    _check(L.nf4_merge_lora(ctypes.byref(s), A.data_ptr(), B.data_ptr(), r, float(alpha),
                            out.data_ptr(), _stream(st.device)))
    return out


def nf4_merge_requantize(st: NF4State, A: torch.Tensor, B: torch.Tensor,
                         alpha: float) -> NF4State:
    """The merged weight quantized again: the state of Qhat(Qhat(W) + s B A)."""
    return nf4_quantize_dq(nf4_merge_lora(st, A, B, alpha))


class Adam8:
    """8-bit AdamW state for one fp32 parameter tensor (moments as E4M3
    codes with one fp32 scale per 256 elements) and its step."""

    def __init__(self, param: torch.Tensor, lr=2e-4, betas=(0.9, 0.999), eps=1e-8,
                 weight_decay=0.0):
        p = _dev(param, torch.float32, "param")
        n, nb = p.numel(), (p.numel() + 255) // 256
        dev = p.device
        self.p = p
        self.mq = torch.zeros(max(n, 16), dtype=torch.uint8, device=dev)
        self.vq = torch.zeros(max(n, 16), dtype=torch.uint8, device=dev)
        self.ms = torch.zeros(max(nb, 4), dtype=torch.float32, device=dev)
        self.vs = torch.zeros(max(nb, 4), dtype=torch.float32, device=dev)
        self.lr, self.betas, self.eps, self.wd = lr, betas, eps, weight_decay
        self.t = 0

    def step(self, grad: torch.Tensor, p_bf16: torch.Tensor | None = None):
        g = _dev(grad, torch.float32, "grad")
        if g.numel() != self.p.numel():
            raise ValueError("grad must have the parameter's size")
        if p_bf16 is not None:
            _dev(p_bf16, torch.bfloat16, "p_bf16")
        self.t += 1
        h = _AdamHP(self.lr, self.betas[0], self.betas[1], self.eps, self.wd, self.t)
        _check(load_library().adamw8_step(self.p.data_ptr(), g.data_ptr(), self.p.numel(),
                                          self.mq.data_ptr(), self.ms.data_ptr(),
                                          self.vq.data_ptr(), self.vs.data_ptr(), _ptr(p_bf16),
                                          ctypes.byref(h), _stream(self.p.device)))


def route(M: int, rows: int, cols: int, r: int, backward: bool = False) -> str:
    """Name of the kernel route of the forward (or of the backward's dX) for
    these sizes on the current device."""
    code = load_library().qlora_linear_route(M, rows, cols, r, int(bool(backward)))
    if code < 0:
        raise ValueError("sizes the linear calls reject")
    return ROUTES[code]


def linear_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace for the linear calls: zeroed, because its first 4 KB are
    arrival counters that must be zero before first use (every call leaves
    them at zero).  One workspace may serve calls of any shape on one
    stream, sized for the largest."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _linear_args(st, x, A, B):
    M = x.shape[0]
    r = A.shape[0]
    if x.dim() != 2 or x.shape[1] != st.cols:
        raise ValueError(f"x must be [M, {st.cols}]")
    if A.dim() != 2 or A.shape[1] != st.cols:
        raise ValueError(f"A must be [r, {st.cols}]")
    if B.dim() != 2 or B.shape != (st.rows, r):
        raise ValueError(f"B must be [{st.rows}, {r}]")
    return M, r


def _bits(t):
    return t.data_ptr()


def dropout_mask(M: int, cols: int, p: float, device="cuda", generator=None) -> torch.Tensor:
    """A keep mask for dropout with probability p on the adapter branch's
    input x [M, cols], bit-packed as the library takes it (element e kept
    when bit e % 8 of byte e / 8 is set): uint8 [M * cols / 8].  The random
    draw itself is torch's."""
    if (M * cols) % 8:
        raise ValueError("M * cols must be a multiple of 8")
    keep = torch.rand(M * cols, device=device, generator=generator) >= p
    w = torch.tensor([1, 2, 4, 8, 16, 32, 64, 128], dtype=torch.int32, device=device)
    return (keep.view(-1, 8).to(torch.int32) * w).sum(dim=1).to(torch.uint8)


def _opts(rslora, mask, p):
    if not rslora and mask is None and not p:
        return None
    if mask is not None:
        _dev(mask, torch.uint8, "dropout_mask")
    return _LoraOpts(int(bool(rslora)), _ptr(mask), float(p))


def qlora_linear_fwd(st: NF4State, x: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                     alpha: float, save_u: bool = True, y: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, rslora: bool = False,
                     dropout_mask: torch.Tensor | None = None, dropout_p: float = 0.0):
    """y = x Qhat(W)^T + s (x A^T) B^T with s = alpha / r (alpha / sqrt(r)
    with rslora); dropout_mask / dropout_p: dropout on the adapter branch's
    input (see dropout_mask()).  Returns (y bf16 [M, d_out], u fp32 [M, r] or
    None; u is the branch's x A^T, masked under dropout)."""
    L = load_library()
    x = _dev(x, torch.bfloat16, "x")
    A = _dev(A, torch.bfloat16, "A")
    B = _dev(B, torch.bfloat16, "B")
    M, r = _linear_args(st, x, A, B)
    if y is None:
        y = torch.empty((M, st.rows), dtype=torch.bfloat16, device=x.device)
    u = torch.empty((M, r), dtype=torch.float32, device=x.device) if save_u else None
    o = _opts(rslora, dropout_mask, dropout_p)
    op = ctypes.byref(o) if o is not None else None
    sc = st.c_struct()
    ws_bytes = L.qlora_linear_workspace_state(ctypes.byref(sc), M, r, 0, op)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = linear_workspace(ws_bytes, x.device)
    s = st.c_struct()
    _check(L.qlora_linear_fwd_ex(ctypes.byref(s), x.data_ptr(), M, A.data_ptr(), B.data_ptr(), r,
                                 float(alpha), op, y.data_ptr(), _ptr(u), workspace.data_ptr(),
                                 workspace.numel(), _stream(x.device)))
    return y, u


def qlora_linear_bwd(st: NF4State, x: torch.Tensor, dY: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, alpha: float, u: torch.Tensor | None = None,
                     need_dx: bool = True, workspace: torch.Tensor | None = None,
                     rslora: bool = False, dropout_mask: torch.Tensor | None = None,
                     dropout_p: float = 0.0):
    """Returns (dX bf16 [M, d_in] or None, dA fp32 [r, d_in], dB fp32 [d_out, r])."""
    L = load_library()
    x = _dev(x, torch.bfloat16, "x")
    dY = _dev(dY, torch.bfloat16, "dY")
    A = _dev(A, torch.bfloat16, "A")
    B = _dev(B, torch.bfloat16, "B")
    M, r = _linear_args(st, x, A, B)
    if dY.shape != (M, st.rows):
        raise ValueError(f"dY must be [{M}, {st.rows}]")
    if u is not None:
        _dev(u, torch.float32, "u")
        if u.shape != (M, r):
            raise ValueError(f"u must be [{M}, {r}]")
    dX = torch.empty((M, st.cols), dtype=torch.bfloat16, device=x.device) if need_dx else None
    dA = torch.empty((r, st.cols), dtype=torch.float32, device=x.device)
    dB = torch.empty((st.rows, r), dtype=torch.float32, device=x.device)
    o = _opts(rslora, dropout_mask, dropout_p)
    op = ctypes.byref(o) if o is not None else None
    sc = st.c_struct()
    ws_bytes = L.qlora_linear_workspace_state(ctypes.byref(sc), M, r, 1, op)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = linear_workspace(ws_bytes, x.device)
    s = st.c_struct()
    _check(L.qlora_linear_bwd_ex(ctypes.byref(s), x.data_ptr(), dY.data_ptr(), M, A.data_ptr(),
                                 B.data_ptr(), r, float(alpha), op, _ptr(u), _ptr(dX),
                                 dA.data_ptr(), dB.data_ptr(), workspace.data_ptr(),
                                 workspace.numel(), _stream(x.device)))
    return dX, dA, dB


def lora_linear_bf16(x: torch.Tensor, W: torch.Tensor, V: torch.Tensor, L_: torch.Tensor,
                     alpha: float, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = x W^T + (alpha/r) V L_^T on a bf16 weight W [d_out, d_in] (for
    example nf4_dequantize's output); V fp32 [M, r] (u), L_ bf16 [d_out, r]."""
    L = load_library()
    x = _dev(x, torch.bfloat16, "x")
    W = _dev(W, torch.bfloat16, "W")
    V = _dev(V, torch.float32, "V")
    L_ = _dev(L_, torch.bfloat16, "L")
    if x.dim() != 2 or W.dim() != 2 or x.shape[1] != W.shape[1]:
        raise ValueError("x must be [M, d_in] and W [d_out, d_in]")
    M, (rows, cols) = x.shape[0], W.shape
    r = V.shape[1] if V.dim() == 2 else -1
    if V.shape != (M, r) or L_.shape != (rows, r):
        raise ValueError("V must be [M, r] and L [d_out, r]")
    if y is None:
        y = torch.empty((M, rows), dtype=torch.bfloat16, device=x.device)
    _check(L.lora_linear_bf16(x.data_ptr(), M, W.data_ptr(), rows, cols, V.data_ptr(),
                              L_.data_ptr(), r, float(alpha), y.data_ptr(), _stream(x.device)))
    return y


class _QLoRAFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, A, B, st, alpha, rslora, mask, p):
        y, u = qlora_linear_fwd(st, x, A, B, alpha, rslora=rslora, dropout_mask=mask,
                                dropout_p=p)
        ctx.save_for_backward(x, A, B, u, mask)
        ctx.st, ctx.alpha, ctx.rslora, ctx.p = st, alpha, rslora, p
        return y

    @staticmethod
    def backward(ctx, dY):
        x, A, B, u, mask = ctx.saved_tensors
        dX, dA, dB = qlora_linear_bwd(ctx.st, x, dY.contiguous(), A, B, ctx.alpha, u,
                                      need_dx=ctx.needs_input_grad[0], rslora=ctx.rslora,
                                      dropout_mask=mask, dropout_p=ctx.p)
        return dX, dA.to(A.dtype), dB.to(B.dtype), None, None, None, None, None


class QLoRALinear(torch.nn.Module):
    """Frozen NF4+DQ base weight with a rank-r adapter: y = x Qhat(W)^T +
    s x A^T B^T, s = alpha/r (alpha/sqrt(r) with rslora), and dropout with
    probability `dropout` on the adapter branch's input in training mode.
    A: (r, d_in), B: (d_out, r), bf16 (B starts at zero, A Kaiming-uniform,
    as in the course notebook's LoRALinear)."""

    def __init__(self, weight: torch.Tensor, r: int = 16, alpha: float = 32.0,
                 dropout: float = 0.0, rslora: bool = False):
        super().__init__()
        d_out, d_in = weight.shape
        self.st = nf4_quantize_dq(weight.detach().float().contiguous())
        self.r, self.alpha, self.dropout, self.rslora = r, alpha, float(dropout), bool(rslora)
        A = torch.empty(r, d_in, dtype=torch.float32, device=weight.device)
        torch.nn.init.kaiming_uniform_(A, a=5 ** 0.5)
        self.lora_A = torch.nn.Parameter(A.to(torch.bfloat16))
        self.lora_B = torch.nn.Parameter(torch.zeros(d_out, r, dtype=torch.bfloat16,
                                                     device=weight.device))

    def forward(self, x):
        shp = x.shape
        x2 = x.reshape(-1, shp[-1]).contiguous()
        p = self.dropout if self.training else 0.0
        mask = dropout_mask(x2.shape[0], x2.shape[1], p, x2.device) if p > 0 else None
        y = _QLoRAFn.apply(x2, self.lora_A, self.lora_B, self.st, self.alpha, self.rslora, mask,
                           p)
        return y.reshape(*shp[:-1], y.shape[-1])
