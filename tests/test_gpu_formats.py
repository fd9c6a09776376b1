"""GPU parity of the format variants with the CPU oracle (course notebook
FT-02: "Guided example 3: double quantization" on/off and "Exercise 3: NF4
vs FP4 at equal memory"): quantize and dequantize bit-exact for NF4 and FP4
codes with and without double quantization; merge bit-exact; the linear
calls within 5e-3 of fp64 on every route (each takes every format); an
exact one-hot pin through the decode kernels for every format."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import REL_TOL, bf16_dev, bf16_host_f64, f32_dev, needs_gpu, rel_err, say

pytestmark = [pytest.mark.gpu, needs_gpu]

FORMATS = [("nf4", False), ("fp4", True), ("fp4", False)]


@pytest.fixture(scope="module")
def qn():
    import quantized_fine_tuning_nf4_amd as qn
    qn.load_library()
    return qn


def _check_state(qn, st, ref):
    torch.cuda.synchronize()
    assert np.array_equal(st.packed.cpu().numpy(), ref.packed)
    if ref.double_quant:
        assert np.array_equal(st.qscale.cpu().numpy(), ref.qscale)
        assert np.array_equal(st.scale2.cpu().numpy().view(np.uint32), ref.scale2.view(np.uint32))
        assert st.offset.cpu().numpy()[0] == ref.offset
    else:
        assert np.array_equal(st.absmax.cpu().numpy().view(np.uint32), ref.absmax.view(np.uint32))
    f32 = qn.nf4_dequantize(st, torch.float32).cpu().numpy()
    b16 = qn.nf4_dequantize(st, torch.bfloat16).cpu().contiguous().view(torch.int16).numpy()
    rf32, rb16 = oracle.dequantize(ref)
    assert np.array_equal(f32.view(np.uint32), rf32.view(np.uint32))
    assert np.array_equal(b16.view(np.uint16), rb16)


@pytest.mark.parametrize("codebook,dq", FORMATS)
@pytest.mark.parametrize("rows,cols", [(256, 256), (37, 16448), (1, 1), (1000, 1000)])
def test_quantize_formats_bit_exact(qn, codebook, dq, rows, cols):
    say(f"[formats] quantize {codebook} dq={dq} {rows}x{cols}")
    W = wl.weight(rows, cols, 1100 + rows)
    if W.size >= 192:  # a zero block and a constant block
        W.ravel()[64:128] = 0.0
        W.ravel()[128:192] = -0.03
    st = qn.qn_quantize(f32_dev(W), codebook=codebook, double_quant=dq)
    _check_state(qn, st, oracle.quantize(W, double_quant=dq, codebook=codebook))


@pytest.mark.parametrize("codebook,dq", FORMATS)
def test_quantize_formats_outlier_workload(qn, codebook, dq):
    W = wl.outlier_weight()
    st = qn.qn_quantize(f32_dev(W), codebook=codebook, double_quant=dq)
    _check_state(qn, st, oracle.quantize(W, double_quant=dq, codebook=codebook))


def test_fp4_codes_near_every_threshold(qn):
    """Unit-scale blocks of weights within a few ulps of every FP4 midpoint
    (both signs): the codes are the exact nearest magnitude, ties lower."""
    cb = oracle.fp4_codebook()
    vals = []
    for k in range(7):
        m = np.float32((float(cb[k]) + float(cb[k + 1])) / 2)
        for d in range(-20, 21):
            v = m
            for _ in range(abs(d)):
                v = np.nextafter(v, np.float32(np.inf if d > 0 else -np.inf))
            vals += [v, -v]
    vals = np.array(vals, np.float32)
    pad = (-vals.size) % 63
    vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 63)
    W = np.concatenate([np.ones((vals.shape[0], 1), np.float32), vals], axis=1)  # absmax 1
    st = qn.qn_quantize(f32_dev(W), codebook="fp4", double_quant=False)
    _check_state(qn, st, oracle.quantize(W, double_quant=False, codebook="fp4"))


def _thresholds(cb):
    """The decision thresholds in quotient space: the largest fp32 not above
    each midpoint of adjacent levels (NF4: all sixteen levels; FP4: the
    eight magnitudes)."""
    L = (oracle.codebook() if cb == "nf4" else oracle.fp4_codebook()[:8]).astype(np.float64)
    m = (L[:-1] + L[1:]) / 2
    t = m.astype(np.float32)
    return np.where(t.astype(np.float64) > m, np.nextafter(t, np.float32(-np.inf)), t)


@pytest.mark.parametrize("codebook", ["nf4", "fp4"])
@pytest.mark.parametrize("lo,hi", [(-100, -80), (100, 127)])
def test_codes_near_thresholds_at_extreme_scales(qn, codebook, lo, hi):
    """Weights within a few ulps of every threshold times the block scale, at
    block scales from 2^lo to 2^hi: tiny scales on both sides of 2^-90 (the
    waves mix the code search's fp32 and fp64 forms) and scales up to the top
    of the fp32 range.  Both signs; the codes are the oracle's."""
    rng = np.random.default_rng(500 + lo)
    nblk = 4096
    t = _thresholds(codebook)
    scales = (rng.uniform(0.5, 1.0, nblk) * 2.0 ** rng.integers(lo, hi, nblk)).astype(np.float32)
    W = np.zeros((nblk, 64), np.float32)
    W[:, 0] = scales
    W[1::3, 0] *= -1
    ks = rng.integers(0, t.size, (nblk, 63))
    base = (t[ks].astype(np.float64) * scales[:, None].astype(np.float64)).astype(np.float32)
    d = rng.integers(-4, 5, (nblk, 63)).astype(np.int32)
    bits = base.view(np.int32)
    bits = np.where(base >= 0, bits + d, bits - d).astype(np.int32)
    v = bits.view(np.float32)
    v = np.where(rng.random((nblk, 63)) < 0.5, -v, v)
    W[:, 1:] = np.clip(v, -np.abs(W[:, :1]), np.abs(W[:, :1]))
    say(f"[formats] {codebook} near thresholds, scales 2^{lo}..2^{hi}")
    st = qn.qn_quantize(f32_dev(W), codebook=codebook, double_quant=False)
    _check_state(qn, st, oracle.quantize(W, double_quant=False, codebook=codebook))


@pytest.mark.parametrize("codebook,dq", FORMATS)
@pytest.mark.parametrize("rows,cols,M,r", [(264, 192, 4, 8), (520, 576, 300, 16),
                                           (3848, 3840, 4100, 16)])
def test_linear_formats(qn, codebook, dq, rows, cols, M, r):
    say(f"[formats] linear {codebook} dq={dq} rows={rows} cols={cols} M={M} r={r}")
    W, x, A, B, G = (wl.weight(rows, cols, 1200 + rows), wl.normal_bf16((M, cols), 1201, 1.0),
                     wl.normal_bf16((r, cols), 1202, 0.05), wl.normal_bf16((rows, r), 1203, 0.05),
                     wl.normal_bf16((M, rows), 1204, 1.0))
    alpha = 2.0 * r
    st = qn.qn_quantize(f32_dev(W), codebook=codebook, double_quant=dq)
    xd, Ad, Bd, Gd = (bf16_dev(a) for a in (x, A, B, G))
    y, u = qn.qlora_linear_fwd(st, xd, Ad, Bd, alpha)
    dX, dA, dB = qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, alpha, u)
    torch.cuda.synchronize()
    s = float(np.float32(alpha) / np.float32(r))
    Wd, _ = oracle.dequantize(oracle.quantize(W, double_quant=dq, codebook=codebook),
                              want_bf16=False)
    rng = np.random.default_rng(M)
    sel = np.arange(M) if M <= 48 else np.sort(rng.choice(M, 48, replace=False))
    Y_ref, _ = oracle.qlora_fwd(Wd, x, A, B, s, rows=sel)
    dX_ref, _ = oracle.qlora_dx(Wd, G, A, B, s, rows=sel)
    dA_ref, dB_ref = oracle.adapter_grads(x, G, A, B, s)
    errs = dict(y=rel_err(bf16_host_f64(y)[sel], Y_ref), dX=rel_err(bf16_host_f64(dX)[sel], dX_ref),
                dA=rel_err(dA.cpu().numpy(), dA_ref), dB=rel_err(dB.cpu().numpy(), dB_ref))
    say("  rel err", {k: f"{v:.2e}" for k, v in errs.items()})
    assert all(e <= REL_TOL for e in errs.values()), errs


@pytest.mark.parametrize("codebook,dq", FORMATS)
@pytest.mark.parametrize("rows,cols,M,r,route", [
    (14336, 4096, 1, 16, "decode_rows"), (14336, 4096, 16, 16, "decode_rows"),
    (14336, 2048, 5, 16, "decode_rows"), (4096, 4096, 4, 16, "decode_tiles"),
    (4104, 3072, 3, 8, "decode_tiles"), (2048, 2048, 2, 32, "decode_split"),
])
def test_decode_formats(qn, codebook, dq, rows, cols, M, r, route):
    """Decode-sized forwards of every format on each decode route: y and u
    against the fp64 oracle on every row."""
    assert qn.route(M, rows, cols, r) == route
    say(f"[formats] decode {codebook} dq={dq} rows={rows} cols={cols} M={M} r={r}")
    W, x, A, B = (wl.weight(rows, cols, 1400 + rows + M), wl.normal_bf16((M, cols), 1401, 1.0),
                  wl.normal_bf16((r, cols), 1402, 0.05), wl.normal_bf16((rows, r), 1403, 0.05))
    alpha = 2.0 * r
    st = qn.qn_quantize(f32_dev(W), codebook=codebook, double_quant=dq)
    y, u = qn.qlora_linear_fwd(st, bf16_dev(x), bf16_dev(A), bf16_dev(B), alpha)
    torch.cuda.synchronize()
    s = float(np.float32(alpha) / np.float32(r))
    Wd, _ = oracle.dequantize(oracle.quantize(W, double_quant=dq, codebook=codebook),
                              want_bf16=False)
    Y_ref, U_ref = oracle.qlora_fwd(Wd, x, A, B, s)
    errs = dict(y=rel_err(bf16_host_f64(y), Y_ref), u=rel_err(u.cpu().numpy(), U_ref))
    say("  rel err", {k: f"{v:.2e}" for k, v in errs.items()})
    assert errs["y"] <= REL_TOL and errs["u"] <= 1e-5, errs


@pytest.mark.parametrize("codebook,dq", FORMATS)
@pytest.mark.parametrize("rows,cols,r,route", [
    (14336, 4096, 16, "decode_rows"),
    (4096, 4096, 16, "decode_tiles"),
    (2048, 2048, 32, "decode_split"),
])
def test_decode_formats_one_hot_exact(qn, codebook, dq, rows, cols, r, route):
    """x rows = e_k (16 per call, every column k over the calls), B = 0:
    y[m, :] = bf16(W'[:, k]) exactly through the decode kernels for every
    format (the block scale 0.25 is a power of two)."""
    assert qn.route(16, rows, cols, r) == route
    say(f"[formats] decode one-hot {codebook} dq={dq} route={route}")
    W = wl.equal_absmax_weight(rows, cols, seed=rows + cols + 7)
    ref = oracle.quantize(W, double_quant=dq, codebook=codebook)
    if dq:
        assert ref.offset == np.float32(0.25) and not ref.scale2.any()
    else:
        assert np.all(ref.absmax == np.float32(0.25))
    _, Wb = oracle.dequantize(ref, want_f32=False)
    st = qn.qn_quantize(f32_dev(W), codebook=codebook, double_quant=dq)
    A = bf16_dev(wl.normal_bf16((r, cols), 7, 0.01))
    B = torch.zeros((rows, r), dtype=torch.bfloat16, device="cuda")
    eye = torch.zeros((cols, cols), dtype=torch.bfloat16, device="cuda")
    eye.fill_diagonal_(1.0)
    got = torch.empty((cols, rows), dtype=torch.bfloat16, device="cuda")
    L = qn.load_library()
    ws = qn.linear_workspace(L.qlora_linear_workspace_state(qn.ctypes.byref(st.c_struct()), 16,
                                                            r, 0, None))
    for k0 in range(0, cols, 16):
        qn.qlora_linear_fwd(st, eye[k0:k0 + 16], A, B, 2.0 * r, y=got[k0:k0 + 16], workspace=ws)
    torch.cuda.synchronize()
    want = wl.bf16_bits_to_f32(np.ascontiguousarray(Wb.T))
    assert np.array_equal(got.float().cpu().numpy(), want)


@pytest.mark.parametrize("codebook,dq", FORMATS)
def test_merge_formats_bit_exact(qn, codebook, dq):
    rows, cols, r = 520, 576, 16
    W = wl.weight(rows, cols, 1300)
    A = wl.normal_bf16((r, cols), 1301, 0.05)
    B = wl.normal_bf16((rows, r), 1302, 0.05)
    st = qn.qn_quantize(f32_dev(W), codebook=codebook, double_quant=dq)
    merged = qn.nf4_merge_lora(st, bf16_dev(A), bf16_dev(B), 32.0).cpu().numpy()
    Wd, _ = oracle.dequantize(oracle.quantize(W, double_quant=dq, codebook=codebook),
                              want_bf16=False)
    ref = oracle.merge(Wd, A, B, np.float32(2.0))
    assert np.array_equal(merged.view(np.uint32), ref.view(np.uint32))
