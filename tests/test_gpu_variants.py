"""GPU parity of the adapter-branch variants with the CPU oracle: rsLoRA's
alpha / sqrt(r) scale and dropout on the branch's input (course notebook
FT-02: "Exercise 4: alpha/r vs alpha/sqrt(r) scaling (rsLoRA)" and the
LoraConfig's lora_dropout), forward and backward within 5e-3 of fp64, plus
the exact special cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import REL_TOL, bf16_dev, bf16_host_f64, f32_dev, needs_gpu, rel_err, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def qn():
    import quantized_fine_tuning_nf4_amd as qn
    qn.load_library()
    return qn


def _inputs(rows, cols, M, r, seed):
    W = wl.weight(rows, cols, seed)
    x = wl.normal_bf16((M, cols), seed + 1, 1.0)
    A = wl.normal_bf16((r, cols), seed + 2, 0.05)
    B = wl.normal_bf16((rows, r), seed + 3, 0.05)
    G = wl.normal_bf16((M, rows), seed + 4, 1.0)
    return W, x, A, B, G


def _sample(M, k=48, seed=0):
    if M <= k:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), k - 2, False)]))


def _mask(M, K, p, seed):
    keep = np.random.default_rng(seed).random(M * K) >= p
    return np.packbits(keep, bitorder="little")


@pytest.mark.parametrize("rows,cols,M,r", [
    (4096, 4096, 4, 16),     # decode route (rsLoRA only changes the scale)
    (520, 576, 300, 16),     # dequantization inside the GEMM tiles
    (3848, 3840, 4100, 8),   # bf16 weight copy + dense GEMM
])
def test_rslora_matches_oracle(qn, rows, cols, M, r):
    say(f"[variants] rsLoRA rows={rows} cols={cols} M={M} r={r}")
    W, x, A, B, G = _inputs(rows, cols, M, r, seed=900 + rows)
    alpha = 16.0
    st = qn.nf4_quantize_dq(f32_dev(W))
    xd, Ad, Bd, Gd = (bf16_dev(a) for a in (x, A, B, G))
    y, u = qn.qlora_linear_fwd(st, xd, Ad, Bd, alpha, rslora=True)
    dX, dA, dB = qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, alpha, u, rslora=True)
    torch.cuda.synchronize()
    s = oracle.lora_scale(alpha, r, rslora=True)
    Wd, _ = oracle.dequantize(oracle.quantize(W), want_bf16=False)
    sel = _sample(M, seed=r)
    Y_ref, _ = oracle.qlora_fwd(Wd, x, A, B, s, rows=sel)
    dX_ref, _ = oracle.qlora_dx(Wd, G, A, B, s, rows=sel)
    dA_ref, dB_ref = oracle.adapter_grads(x, G, A, B, s)
    errs = dict(y=rel_err(bf16_host_f64(y)[sel], Y_ref), dX=rel_err(bf16_host_f64(dX)[sel], dX_ref),
                dA=rel_err(dA.cpu().numpy(), dA_ref), dB=rel_err(dB.cpu().numpy(), dB_ref))
    say("  rel err", {k: f"{v:.2e}" for k, v in errs.items()})
    assert all(e <= REL_TOL for e in errs.values()), errs
    # alpha / sqrt(16) = (4 alpha) / 16: the same scale, the same bits
    if r == 16:
        y2, _ = qn.qlora_linear_fwd(st, xd, Ad, Bd, 4 * alpha)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)


@pytest.mark.parametrize("rows,cols,M,r,p", [
    (264, 192, 24, 8, 0.05),     # 32-row fused GEMM (a decode-sized batch with dropout)
    (4096, 4096, 4, 16, 0.05),   # decode-sized: dropout takes the fused GEMM route
    (520, 576, 300, 16, 0.3),    # 128 x 128 fused GEMM
    (3848, 3840, 4100, 16, 0.05),  # dense GEMM, masked dX add after it
    (1032, 320, 130, 64, 0.5),   # rank 64
    (4096, 4096, 8192, 16, 0.05),  # the training shape with dropout (as the benchmark times it)
])
def test_dropout_matches_oracle(qn, rows, cols, M, r, p):
    say(f"[variants] dropout rows={rows} cols={cols} M={M} r={r} p={p} "
        f"route fwd={qn.route(M, rows, cols, r)}")
    W, x, A, B, G = _inputs(rows, cols, M, r, seed=950 + rows + r)
    alpha = 2.0 * r
    mask = _mask(M, cols, p, seed=M + cols)
    st = qn.nf4_quantize_dq(f32_dev(W))
    xd, Ad, Bd, Gd = (bf16_dev(a) for a in (x, A, B, G))
    md = torch.from_numpy(mask).cuda()
    y, u = qn.qlora_linear_fwd(st, xd, Ad, Bd, alpha, dropout_mask=md, dropout_p=p)
    dX, dA, dB = qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, alpha, u, dropout_mask=md, dropout_p=p)
    # u recomputed inside the backward (masked the same way)
    dX2, dA2, dB2 = qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, alpha, None, dropout_mask=md,
                                        dropout_p=p)
    torch.cuda.synchronize()
    s = oracle.lora_scale(alpha, r, dropout_p=p)
    Wd, _ = oracle.dequantize(oracle.quantize(W), want_bf16=False)
    sel = _sample(M, seed=r + 1)
    Y_ref, u_ref = oracle.qlora_fwd_dropout(Wd, x, A, B, s, mask, rows=sel)
    dX_ref, _ = oracle.qlora_dx_dropout(Wd, G, A, B, s, mask, rows=sel)
    dA_ref, dB_ref = oracle.adapter_grads_dropout(x, G, A, B, s, mask)
    errs = dict(y=rel_err(bf16_host_f64(y)[sel], Y_ref), u=rel_err(u.cpu().numpy()[sel], u_ref),
                dX=rel_err(bf16_host_f64(dX)[sel], dX_ref),
                dA=rel_err(dA.cpu().numpy(), dA_ref), dB=rel_err(dB.cpu().numpy(), dB_ref))
    say("  rel err", {k: f"{v:.2e}" for k, v in errs.items()})
    assert all(e <= REL_TOL for e in errs.values()), errs
    assert torch.equal(dX2, dX) and torch.equal(dA2, dA)
    assert rel_err(dB2.cpu().numpy(), dB.cpu().numpy().astype(np.float64)) <= 1e-5


@pytest.mark.parametrize("rows,cols,M,r", [(520, 576, 300, 16), (3848, 3840, 4100, 16)])
def test_dropout_all_dropped(qn, rows, cols, M, r):
    """Every element dropped: y is the base output bit for bit, dA and dB are
    exactly zero, dX equals the base input gradient bit for bit."""
    W, x, A, B, G = _inputs(rows, cols, M, r, seed=990 + rows)
    st = qn.nf4_quantize_dq(f32_dev(W))
    xd, Ad, Bd, Gd = (bf16_dev(a) for a in (x, A, B, G))
    md = torch.zeros(M * cols // 8, dtype=torch.uint8, device="cuda")
    y, u = qn.qlora_linear_fwd(st, xd, Ad, Bd, 32.0, dropout_mask=md, dropout_p=0.05)
    y0, _ = qn.qlora_linear_fwd(st, xd, Ad, Bd, 0.0)
    dX, dA, dB = qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, 32.0, u, dropout_mask=md,
                                     dropout_p=0.05)
    dX0, _, _ = qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, 0.0, None)
    torch.cuda.synchronize()
    assert not u.any()
    assert torch.equal(y, y0) and torch.equal(dX, dX0)
    assert not dA.any() and not dB.any()


def test_options_are_checked_on_the_host(qn):
    import ctypes
    L = qn.load_library()
    W, x, A, B, _ = _inputs(64, 128, 8, 4, seed=5)
    st = qn.nf4_quantize_dq(f32_dev(W))
    xd, Ad, Bd = (bf16_dev(a) for a in (x, A, B))
    md = torch.ones(8 * 128 // 8, dtype=torch.uint8, device="cuda")
    s = st.c_struct()
    y = torch.empty((8, 64), dtype=torch.bfloat16, device="cuda")
    ws = qn.linear_workspace(1 << 20)
    for opts in [qn._LoraOpts(2, None, 0.0), qn._LoraOpts(0, md.data_ptr(), 1.0),
                 qn._LoraOpts(0, md.data_ptr(), -0.1), qn._LoraOpts(0, None, 0.5)]:
        rc = L.qlora_linear_fwd_ex(ctypes.byref(s), xd.data_ptr(), 8, Ad.data_ptr(),
                                   Bd.data_ptr(), 4, 8.0, ctypes.byref(opts), y.data_ptr(), None,
                                   ws.data_ptr(), ws.numel(), None)
        assert rc == qn.QN_EINVAL
    # the mask is read in 8- and 16-byte pieces: a misaligned one is refused
    # before anything is launched
    bad = qn._LoraOpts(0, md.data_ptr() + 1, 0.05)
    rc = L.qlora_linear_fwd_ex(ctypes.byref(s), xd.data_ptr(), 8, Ad.data_ptr(), Bd.data_ptr(), 4,
                               8.0, ctypes.byref(bad), y.data_ptr(), None, ws.data_ptr(),
                               ws.numel(), None)
    assert rc == qn.QN_EALIGN
