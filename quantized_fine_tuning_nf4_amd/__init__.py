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
           "qlora_linear_bwd", "lora_linear_bf16"]


class QNError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class _NF4DQ(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("qscale", ctypes.c_void_p),
                ("scale2", ctypes.c_void_p), ("offset", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


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
    L.nf4_quantize_dq_workspace.argtypes = [I64, I64]
    L.nf4_quantize_dq_workspace.restype = SZ
    L.nf4_quantize_dq.argtypes = [P, I64, I64, P, P, P, P, P, P, SZ, P]
    L.nf4_quantize_dq.restype = ctypes.c_int
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
    """Quantized weight, format v1: packed codes, E4M3 scale codes, second-
    level scales and the mean offset, all on the device."""
    packed: torch.Tensor  # uint8 [32*nb]
    qscale: torch.Tensor  # uint8 [nb]
    scale2: torch.Tensor  # float32 [ng]
    offset: torch.Tensor  # float32 [1]
    rows: int
    cols: int

    def c_struct(self) -> _NF4DQ:
        return _NF4DQ(self.packed.data_ptr(), self.qscale.data_ptr(), self.scale2.data_ptr(),
                      self.offset.data_ptr(), self.rows, self.cols)

    @property
    def device(self):
        return self.packed.device

    def nbytes(self) -> int:
        return (self.packed.numel() + self.qscale.numel() + 4 * self.scale2.numel()
                + 4 * self.offset.numel())


def codebook() -> list:
    out = (ctypes.c_float * 16)()
    load_library().qn_nf4_codebook(out)
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


def nf4_dequantize(st: NF4State, dtype=torch.bfloat16, out: torch.Tensor | None = None):
    L = load_library()
    code = {torch.float32: QN_F32, torch.bfloat16: QN_BF16}[dtype]
    if out is None:
        out = torch.empty((st.rows, st.cols), dtype=dtype, device=st.device)
    _dev(out, dtype, "out")
    s = st.c_struct()
    _check(L.nf4_dequantize(ctypes.byref(s), code, out.data_ptr(), _stream(st.device)))
    return out


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


def qlora_linear_fwd(st: NF4State, x: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                     alpha: float, save_u: bool = True, y: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None):
    """y = x Qhat(W)^T + (alpha/r) (x A^T) B^T; returns (y bf16 [M, d_out],
    u fp32 [M, r] or None)."""
    L = load_library()
    x = _dev(x, torch.bfloat16, "x")
    A = _dev(A, torch.bfloat16, "A")
    B = _dev(B, torch.bfloat16, "B")
    M, r = _linear_args(st, x, A, B)
    if y is None:
        y = torch.empty((M, st.rows), dtype=torch.bfloat16, device=x.device)
    u = torch.empty((M, r), dtype=torch.float32, device=x.device) if save_u else None
    ws_bytes = L.qlora_linear_workspace(M, st.rows, st.cols, r, 0)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    s = st.c_struct()
    _check(L.qlora_linear_fwd(ctypes.byref(s), x.data_ptr(), M, A.data_ptr(), B.data_ptr(), r,
                              float(alpha), y.data_ptr(), _ptr(u), workspace.data_ptr(),
                              workspace.numel(), _stream(x.device)))
    return y, u


def qlora_linear_bwd(st: NF4State, x: torch.Tensor, dY: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, alpha: float, u: torch.Tensor | None = None,
                     need_dx: bool = True, workspace: torch.Tensor | None = None):
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
    ws_bytes = L.qlora_linear_workspace(M, st.rows, st.cols, r, 1)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    s = st.c_struct()
    _check(L.qlora_linear_bwd(ctypes.byref(s), x.data_ptr(), dY.data_ptr(), M, A.data_ptr(),
                              B.data_ptr(), r, float(alpha), _ptr(u), _ptr(dX), dA.data_ptr(),
                              dB.data_ptr(), workspace.data_ptr(), workspace.numel(),
                              _stream(x.device)))
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
    def forward(ctx, x, A, B, st, alpha):
        y, u = qlora_linear_fwd(st, x, A, B, alpha)
        ctx.save_for_backward(x, A, B, u)
        ctx.st, ctx.alpha = st, alpha
        return y

    @staticmethod
    def backward(ctx, dY):
        x, A, B, u = ctx.saved_tensors
        dX, dA, dB = qlora_linear_bwd(ctx.st, x, dY.contiguous(), A, B, ctx.alpha, u,
                                      need_dx=ctx.needs_input_grad[0])
        return dX, dA.to(A.dtype), dB.to(B.dtype), None, None


class QLoRALinear(torch.nn.Module):
    """Frozen NF4+DQ base weight with a rank-r adapter: y = x Qhat(W)^T +
    (alpha/r) x A^T B^T.  A: (r, d_in), B: (d_out, r), bf16 (B starts at
    zero, A Kaiming-uniform, as in the course notebook's LoRALinear)."""

    def __init__(self, weight: torch.Tensor, r: int = 16, alpha: float = 32.0):
        super().__init__()
        d_out, d_in = weight.shape
        self.st = nf4_quantize_dq(weight.detach().float().contiguous())
        self.r, self.alpha = r, alpha
        A = torch.empty(r, d_in, dtype=torch.float32, device=weight.device)
        torch.nn.init.kaiming_uniform_(A, a=5 ** 0.5)
        self.lora_A = torch.nn.Parameter(A.to(torch.bfloat16))
        self.lora_B = torch.nn.Parameter(torch.zeros(d_out, r, dtype=torch.bfloat16,
                                                     device=weight.device))

    def forward(self, x):
        shp = x.shape
        y = _QLoRAFn.apply(x.reshape(-1, shp[-1]).contiguous(), self.lora_A, self.lora_B,
                           self.st, self.alpha)
        return y.reshape(*shp[:-1], y.shape[-1])
