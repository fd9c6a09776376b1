"""CPU oracle for the QLoRA NF4 hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never imports it
and shares no code with it.

This module is a thin ctypes layer over ``qlora_oracle.c`` (plain C, fp64
GEMM loops, fp32 quantiser written step by step from the pages).  Citations
of the passages each step follows are in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qlora_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared"]

OK, EINVAL, ENONFINITE = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no HIP, no SIMD intrinsics, no BLAS)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.orc_codebook.argtypes = [_P]
        L.orc_nf4_code.argtypes = [ctypes.c_float]
        L.orc_nf4_code.restype = ctypes.c_int
        L.orc_nf4_codes.argtypes = [_P, _I64, _P]
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_float
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_scale_mean.argtypes = [_P, _I64]
        L.orc_scale_mean.restype = ctypes.c_float
        L.orc_quantize.argtypes = [_P, _I64, ctypes.c_int, _P, _P, _P, _P, _P]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_quantize_cb.argtypes = [_P, _I64, ctypes.c_int, ctypes.c_int, _P, _P, _P, _P, _P]
        L.orc_quantize_cb.restype = ctypes.c_int
        L.orc_dequantize.argtypes = [_P, _I64, ctypes.c_int, _P, _P, _P, _P, _P, _P]
        L.orc_dequantize_cb.argtypes = [_P, _I64, ctypes.c_int, ctypes.c_int, _P, _P, _P, _P,
                                        _P, _P]
        L.orc_fp4_codebook.argtypes = [_P]
        L.orc_fp4_code.argtypes = [ctypes.c_float]
        L.orc_fp4_code.restype = ctypes.c_int
        L.orc_lora_down.argtypes = [_P, _P, _I64, ctypes.c_int, _P, _I64, _P]
        L.orc_qlora_fwd.argtypes = [_P, _I64, _I64, _P, _P, _P, ctypes.c_int,
                                    ctypes.c_double, _P, _I64, _P, _P]
        L.orc_lora_up_grad.argtypes = [_P, _P, _I64, ctypes.c_int, _P, _I64, _P]
        L.orc_qlora_dx.argtypes = [_P, _I64, _I64, _P, _P, _P, ctypes.c_int,
                                   ctypes.c_double, _P, _I64, _P, _P]
        L.orc_adapter_grads.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64,
                                        ctypes.c_int, ctypes.c_double, _P, _P]
        L.orc_merge.argtypes = [_P, _I64, _I64, _P, _P, ctypes.c_int, ctypes.c_float, _P]
        F = ctypes.c_float
        L.orc_adamw8_step.argtypes = [_P, _P, _I64, _P, _P, _P, _P, _P] + [F] * 9
        L.orc_dropout_apply.argtypes = [_P, _P, _I64, _I64, _P]
        L.orc_qlora_dx_dropout.argtypes = [_P, _I64, _I64, _P, _P, _P, ctypes.c_int,
                                           ctypes.c_double, _P, _P, _I64, _P, _P]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


def _bf16_bits(a) -> np.ndarray:
    """bf16 data as uint16 bit patterns (numpy uint16 or a torch bf16 tensor)."""
    if isinstance(a, np.ndarray):
        assert a.dtype == np.uint16
        return np.ascontiguousarray(a)
    import torch  # only to read torch bf16 tensors handed over by tests
    assert a.dtype == torch.bfloat16
    return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on."""
    lib().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- codebook
def codebook() -> np.ndarray:
    out = np.zeros(16, np.float32)
    lib().orc_codebook(_ptr(out))
    return out


def fp4_codebook() -> np.ndarray:
    """The 16 FP4 code values (code c: sign bit 3, magnitude index c & 7)."""
    out = np.zeros(16, np.float32)
    lib().orc_fp4_codebook(_ptr(out))
    return out


def fp4_codes(n: np.ndarray) -> np.ndarray:
    n = np.ascontiguousarray(n, dtype=np.float32).ravel()
    return np.array([lib().orc_fp4_code(float(v)) for v in n], np.uint8)


def nf4_codes(n: np.ndarray) -> np.ndarray:
    n = np.ascontiguousarray(n, dtype=np.float32)
    out = np.empty(n.size, np.uint8)
    lib().orc_nf4_codes(_ptr(n), n.size, _ptr(out))
    return out.reshape(n.shape)


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def e4m3_decode(q: int) -> float:
    return float(lib().orc_e4m3_decode(int(q)))


def bf16_rne(v: float) -> int:
    return int(lib().orc_bf16_rne(float(v)))


def scale_mean(absmax: np.ndarray) -> np.float32:
    a = np.ascontiguousarray(absmax, dtype=np.float32)
    return np.float32(lib().orc_scale_mean(_ptr(a), a.size))


# ---------------------------------------------------------------- quantize
@dataclass
class State:
    packed: np.ndarray   # uint8 [32*nb]
    absmax: np.ndarray   # float32 [nb]   first-level scales (DQ-off state)
    qscale: np.ndarray   # uint8 [nb]     E4M3FN codes (DQ state)
    scale2: np.ndarray   # float32 [ng]
    offset: np.float32   # mean of the first-level scales
    rows: int
    cols: int
    double_quant: bool
    codebook: int = 0    # 0 NF4, 1 FP4

    @property
    def n(self) -> int:
        return self.rows * self.cols


CODEBOOKS = {"nf4": 0, "fp4": 1}


def quantize(W: np.ndarray, double_quant: bool = True, codebook: str = "nf4") -> State:
    """Block-64 4-bit quantisation (NF4 or FP4 codes, + double quantisation)
    of an fp32 array.

    Raises ValueError on empty or non-finite input, like the page's listing.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    rows, cols = (W.shape if W.ndim == 2 else (1, W.size))
    n = W.size
    nb = max((n + 63) // 64, 1)
    ng = (nb + 255) // 256
    packed = np.zeros(32 * nb, np.uint8)
    absmax = np.zeros(nb, np.float32)
    qscale = np.zeros(nb, np.uint8)
    scale2 = np.zeros(ng, np.float32)
    offset = np.zeros(1, np.float32)
    cb = CODEBOOKS[codebook]
    st = lib().orc_quantize_cb(_ptr(W), n, cb, int(bool(double_quant)), _ptr(packed),
                               _ptr(absmax), _ptr(qscale), _ptr(scale2), _ptr(offset))
    if st == EINVAL:
        raise ValueError("quantizer input: empty")
    if st == ENONFINITE:
        raise ValueError("quantizer input: non-finite")
    return State(packed, absmax, qscale, scale2, offset[0], rows, cols, bool(double_quant), cb)


def dequantize(s: State, want_f32: bool = True, want_bf16: bool = True):
    """Returns (fp32 [rows, cols] or None, bf16 bits uint16 [rows, cols] or None)."""
    n = s.n
    f32 = np.empty(n, np.float32) if want_f32 else None
    b16 = np.empty(n, np.uint16) if want_bf16 else None
    off = np.array([s.offset], np.float32)
    lib().orc_dequantize_cb(_ptr(s.packed), n, s.codebook, int(s.double_quant), _ptr(s.absmax),
                            _ptr(s.qscale), _ptr(s.scale2), _ptr(off), _ptr(f32), _ptr(b16))
    shape = (s.rows, s.cols)
    return (f32.reshape(shape) if f32 is not None else None,
            b16.reshape(shape) if b16 is not None else None)


def codes_of(s: State) -> np.ndarray:
    """Unpacked 4-bit codes (uint8 [32*nb*2]) of a state."""
    p = s.packed
    c = np.empty(2 * p.size, np.uint8)
    c[0::2] = p & 15
    c[1::2] = p >> 4
    return c


# ---------------------------------------------------------------- linear
def _rows_arg(rows):
    if rows is None:
        return None
    return np.ascontiguousarray(rows, dtype=np.int64)


def lora_down(X, A, rows=None) -> np.ndarray:
    Xb, Ab = _bf16_bits(X), _bf16_bits(A)
    M, K = Xb.shape
    r = Ab.shape[0]
    rr = _rows_arg(rows)
    nrows = M if rr is None else rr.size
    u = np.empty((nrows, r), np.float64)
    lib().orc_lora_down(_ptr(Xb), _ptr(Ab), K, r, _ptr(rr), nrows, _ptr(u))
    return u


def qlora_fwd(Wd: np.ndarray, X, A, B, s: float, rows=None):
    """Y = X W'^T + s (X A^T) B^T in fp64 for the listed rows (all if None).

    Returns (Y [nrows, N] fp64, u [nrows, r] fp64)."""
    Wd = np.ascontiguousarray(Wd, dtype=np.float32)
    Xb, Ab, Bb = _bf16_bits(X), _bf16_bits(A), _bf16_bits(B)
    N, K = Wd.shape
    M = Xb.shape[0]
    r = Ab.shape[0]
    assert Xb.shape[1] == K and Ab.shape == (r, K) and Bb.shape == (N, r)
    rr = _rows_arg(rows)
    nrows = M if rr is None else rr.size
    Y = np.empty((nrows, N), np.float64)
    u = np.empty((nrows, r), np.float64)
    lib().orc_qlora_fwd(_ptr(Wd), N, K, _ptr(Xb), _ptr(Ab), _ptr(Bb), r, float(s), _ptr(rr),
                        nrows, _ptr(Y), _ptr(u))
    return Y, u


def lora_up_grad(G, B, rows=None) -> np.ndarray:
    Gb, Bb = _bf16_bits(G), _bf16_bits(B)
    M, N = Gb.shape
    r = Bb.shape[1]
    rr = _rows_arg(rows)
    nrows = M if rr is None else rr.size
    v = np.empty((nrows, r), np.float64)
    lib().orc_lora_up_grad(_ptr(Gb), _ptr(Bb), N, r, _ptr(rr), nrows, _ptr(v))
    return v


def qlora_dx(Wd: np.ndarray, G, A, B, s: float, rows=None):
    """dX = G W' + s (G B) A in fp64 for the listed rows.  Returns (dX, v)."""
    Wd = np.ascontiguousarray(Wd, dtype=np.float32)
    Gb, Ab, Bb = _bf16_bits(G), _bf16_bits(A), _bf16_bits(B)
    N, K = Wd.shape
    M = Gb.shape[0]
    r = Ab.shape[0]
    assert Gb.shape[1] == N and Ab.shape == (r, K) and Bb.shape == (N, r)
    rr = _rows_arg(rows)
    nrows = M if rr is None else rr.size
    dX = np.empty((nrows, K), np.float64)
    v = np.empty((nrows, r), np.float64)
    lib().orc_qlora_dx(_ptr(Wd), N, K, _ptr(Gb), _ptr(Ab), _ptr(Bb), r, float(s), _ptr(rr),
                       nrows, _ptr(dX), _ptr(v))
    return dX, v


def adapter_grads(X, G, A, B, s: float):
    """dA = s (G B)^T X [r, K] and dB = s G^T (X A^T) [N, r], fp64, over all rows."""
    Xb, Gb, Ab, Bb = _bf16_bits(X), _bf16_bits(G), _bf16_bits(A), _bf16_bits(B)
    M, K = Xb.shape
    N = Gb.shape[1]
    r = Ab.shape[0]
    u = lora_down(Xb, Ab)
    v = lora_up_grad(Gb, Bb)
    dA = np.empty((r, K), np.float64)
    dB = np.empty((N, r), np.float64)
    lib().orc_adapter_grads(_ptr(Xb), _ptr(Gb), _ptr(u), _ptr(v), M, N, K, r, float(s),
                            _ptr(dA), _ptr(dB))
    return dA, dB


# ---------------------------------------------------------------- adapter variants
def lora_scale(alpha: float, r: int, rslora: bool = False, dropout_p: float = 0.0) -> float:
    """The adapter branch's scale in fp32: alpha / r, or alpha / sqrt(r) for
    rsLoRA (course notebook FT-02, "Exercise 4: alpha/r vs alpha/sqrt(r)
    scaling (rsLoRA)"), divided by 1 - p when dropout with probability p acts
    on the branch's input (inverted dropout, folded into the scale)."""
    a, rf = np.float32(alpha), np.float32(r)
    s = a / np.sqrt(rf, dtype=np.float32) if rslora else a / rf
    if dropout_p:
        s = np.float32(s) / (np.float32(1.0) - np.float32(dropout_p))
    return float(np.float32(s))


def dropout_apply(X, mask: np.ndarray) -> np.ndarray:
    """The adapter branch's input: X with dropped elements zeroed (mask
    bit-packed over the row-major elements, bit e % 8 of byte e / 8)."""
    Xb = _bf16_bits(X)
    M, K = Xb.shape
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    assert mask.size * 8 >= M * K
    out = np.empty_like(Xb)
    lib().orc_dropout_apply(_ptr(Xb), _ptr(mask), M, K, _ptr(out))
    return out


def qlora_dx_dropout(Wd: np.ndarray, G, A, B, s: float, mask: np.ndarray, rows=None):
    """dX = G W' + s ((G B) A) (.) mask in fp64 for the listed rows.  Returns (dX, v)."""
    Wd = np.ascontiguousarray(Wd, dtype=np.float32)
    Gb, Ab, Bb = _bf16_bits(G), _bf16_bits(A), _bf16_bits(B)
    N, K = Wd.shape
    M = Gb.shape[0]
    r = Ab.shape[0]
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    assert mask.size * 8 >= M * K
    rr = _rows_arg(rows)
    nrows = M if rr is None else rr.size
    dX = np.empty((nrows, K), np.float64)
    v = np.empty((nrows, r), np.float64)
    lib().orc_qlora_dx_dropout(_ptr(Wd), N, K, _ptr(Gb), _ptr(Ab), _ptr(Bb), r, float(s),
                               _ptr(mask), _ptr(rr), nrows, _ptr(dX), _ptr(v))
    return dX, v


def qlora_fwd_dropout(Wd: np.ndarray, X, A, B, s: float, mask: np.ndarray, rows=None):
    """y = X W'^T + s ((mask (.) X) A^T) B^T for the listed rows; returns (y, u)
    with u = (mask (.) X) A^T."""
    Xb = _bf16_bits(X)
    Xd = dropout_apply(Xb, mask)
    base, _ = qlora_fwd(Wd, Xb, A, np.zeros_like(_bf16_bits(B)), 0.0, rows=rows)
    u = lora_down(Xd, A, rows=rows)
    return base + s * (u @ _bf16_f64(B).T), u


def adapter_grads_dropout(X, G, A, B, s: float, mask: np.ndarray):
    """dA = s (G B)^T (mask (.) X), dB = s G^T ((mask (.) X) A^T), over all rows."""
    return adapter_grads(dropout_apply(X, mask), G, A, B, s)


@dataclass
class Adam8State:
    """8-bit AdamW state of one parameter tensor: E4M3 codes and fp32 block
    scales (256 elements per block) of the two moments."""
    mq: np.ndarray
    ms: np.ndarray
    vq: np.ndarray
    vs: np.ndarray

    @staticmethod
    def zeros(n: int) -> "Adam8State":
        nb = (n + 255) // 256
        return Adam8State(np.zeros(n, np.uint8), np.zeros(nb, np.float32),
                          np.zeros(n, np.uint8), np.zeros(nb, np.float32))


def adamw_scalars(lr, beta1, beta2, eps, weight_decay, step):
    """The fp32 scalars of AdamW step `step` (>= 1).  The hyperparameters are
    fp32 values (rounded from what is given); from them, in fp64 and rounded
    once to fp32: 1 - b1, 1 - b2, the bias corrections 1 - b^t and the
    decoupled decay 1 - lr wd."""
    f = lambda x: float(np.float32(x))
    lr, b1, b2, eps, wd = f(lr), f(beta1), f(beta2), f(eps), f(weight_decay)
    return (lr, b1, b2, f(1.0 - b1), f(1.0 - b2), eps, f(1.0 - b1 ** int(step)),
            f(1.0 - b2 ** int(step)), f(1.0 - lr * wd))


def adamw8_step(p: np.ndarray, g: np.ndarray, st: Adam8State, lr=2e-4, beta1=0.9,
                beta2=0.999, eps=1e-8, weight_decay=0.0, step=1, want_bf16=False):
    """One 8-bit AdamW step in place on p (fp32) and st; returns bf16(p)
    bits when want_bf16."""
    assert p.dtype == np.float32 and g.dtype == np.float32 and p.flags["C_CONTIGUOUS"]
    g = np.ascontiguousarray(g)
    pb = np.empty(p.size, np.uint16) if want_bf16 else None
    lib().orc_adamw8_step(_ptr(p), _ptr(g), p.size, _ptr(st.mq), _ptr(st.ms), _ptr(st.vq),
                          _ptr(st.vs), _ptr(pb),
                          *adamw_scalars(lr, beta1, beta2, eps, weight_decay, step))
    return pb


def _bf16_f64(a) -> np.ndarray:
    b = _bf16_bits(a)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def merge(Wd: np.ndarray, A, B, s: float) -> np.ndarray:
    """Qhat(W) + s B A as fp32 [rows, cols] from the dequantized fp32 weight
    (fp64 rank sum, one fp32 rounding at the end; see orc_merge)."""
    Wd = np.ascontiguousarray(Wd, dtype=np.float32)
    Ab, Bb = _bf16_bits(A), _bf16_bits(B)
    rows, cols = Wd.shape
    r = Ab.shape[0]
    assert Ab.shape == (r, cols) and Bb.shape == (rows, r)
    out = np.empty((rows, cols), np.float32)
    lib().orc_merge(_ptr(Wd), rows, cols, _ptr(Ab), _ptr(Bb), r, float(np.float32(s)), _ptr(out))
    return out


def rel_frobenius(out, ref) -> float:
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(out - ref)
    return float(num / den) if den > 0 else float(num)
