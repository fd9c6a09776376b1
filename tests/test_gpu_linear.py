"""GPU parity of qlora_linear_fwd / qlora_linear_bwd with the fp64 CPU oracle
(relative Frobenius error <= 5e-3), plus exact special cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import (REL_TOL, bf16_bits, bf16_dev, bf16_host_f64, f32_dev, needs_gpu, rel_err,
                        say)

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def qn():
    import quantized_fine_tuning_nf4_amd as qn
    qn.load_library()
    return qn


class Case:
    """Seeded inputs of one linear; the oracle quantizes W itself."""

    def __init__(self, rows, cols, M, r, alpha, seed, adapter_std=0.01):
        self.rows, self.cols, self.M, self.r, self.alpha = rows, cols, M, r, alpha
        self.s = float(np.float32(alpha) / np.float32(r))
        self.W = wl.weight(rows, cols, seed)
        self.x = wl.normal_bf16((M, cols), seed + 1, 1.0)
        self.A = wl.normal_bf16((r, cols), seed + 2, adapter_std)
        self.B = wl.normal_bf16((rows, r), seed + 3, adapter_std)
        self.G = wl.normal_bf16((M, rows), seed + 4, 1.0)
        self._Wd = None

    @property
    def Wd(self):
        if self._Wd is None:
            self._Wd, _ = oracle.dequantize(oracle.quantize(self.W))
        return self._Wd

    def dev(self, qn):
        st = qn.nf4_quantize_dq(f32_dev(self.W))
        return st, bf16_dev(self.x), bf16_dev(self.A), bf16_dev(self.B), bf16_dev(self.G)


def sample_rows(M, k=48, seed=0):
    """Rows checked at full size: first, last (ragged tail) and random."""
    if M <= k:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    fixed = np.array([0, 1, M - 2, M - 1])
    rest = rng.choice(np.arange(2, M - 2), k - 4, replace=False)
    return np.sort(np.concatenate([fixed, rest]))


def check_fwd_bwd(qn, c: Case, label: str, rows=None, bwd=True):
    say(f"[linear] {label}: rows={c.rows} cols={c.cols} M={c.M} r={c.r}")
    st, x, A, B, G = c.dev(qn)
    y, u = qn.qlora_linear_fwd(st, x, A, B, c.alpha)
    torch.cuda.synchronize()
    sel = np.arange(c.M) if rows is None else rows
    Y_ref, u_ref = oracle.qlora_fwd(c.Wd, c.x, c.A, c.B, c.s, rows=sel)
    ey = rel_err(bf16_host_f64(y)[sel], Y_ref)
    eu = rel_err(u.cpu().numpy()[sel], u_ref)
    say(f"  fwd rel err y={ey:.2e} u={eu:.2e}")
    assert ey <= REL_TOL and eu <= 1e-5
    if not bwd:
        return
    dX, dA, dB = qn.qlora_linear_bwd(st, x, G, A, B, c.alpha, u)
    torch.cuda.synchronize()
    dX_ref, _ = oracle.qlora_dx(c.Wd, c.G, c.A, c.B, c.s, rows=sel)
    dA_ref, dB_ref = oracle.adapter_grads(c.x, c.G, c.A, c.B, c.s)
    ex = rel_err(bf16_host_f64(dX)[sel], dX_ref)
    ea = rel_err(dA.cpu().numpy(), dA_ref)
    eb = rel_err(dB.cpu().numpy(), dB_ref)
    say(f"  bwd rel err dX={ex:.2e} dA={ea:.2e} dB={eb:.2e}")
    assert ex <= REL_TOL and ea <= REL_TOL and eb <= REL_TOL
    # recomputing u inside the backward: dX and dA do not involve u and are
    # bit-equal; dB = s G^T u matches to u's fp32 precision (the decode-sized
    # forward sums u in another order than the backward's recomputation)
    dX2, dA2, dB2 = qn.qlora_linear_bwd(st, x, G, A, B, c.alpha, None)
    torch.cuda.synchronize()
    assert torch.equal(dX2, dX) and torch.equal(dA2, dA)
    assert rel_err(dB2.cpu().numpy(), dB.cpu().numpy().astype(np.float64)) <= 1e-5


def test_tiny_config(qn):
    cfg = wl.TINY
    c = Case(cfg["rows"], cfg["cols"], cfg["M"], cfg["r"], cfg["alpha"], wl.SEED_W + cfg["seed"])
    check_fwd_bwd(qn, c, "tiny")


@pytest.mark.parametrize("rows,cols,M,r", [
    (264, 192, 37, 5),      # 32-row tiles, ragged everything, rank not a multiple of 8
    (8, 64, 1, 1),          # smallest legal shapes
    (520, 576, 300, 16),    # 128x128 tiles, ragged M / N / K tiles
    (1032, 320, 130, 64),   # rank 64: four 16-wide adapter steps
    (7680, 256, 2085, 8),   # forward through the bf16 copy + dense GEMM, ragged M
    (3848, 3840, 4100, 5),  # dense forward and dX: ragged M, N % 32 == 8, rank 5
    (2056, 3904, 4100, 20), # dense dX: K % 256 == 64 (a partial column group in the
                            # transposed dequantization), rank 20 (B^T made first)
    (4096, 4096, 32832, 16),  # a long batch: u and v in one column slice each (no slice
                              # sums), 129 GEMM row tiles with a 64-row last one
])
def test_ragged_shapes(qn, rows, cols, M, r):
    c = Case(rows, cols, M, r, 2.0 * r, seed=rows + cols + M)
    check_fwd_bwd(qn, c, "ragged", rows=sample_rows(M, 64, seed=M))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_config(qn, M):
    cfg = wl.DECODE
    c = Case(cfg["rows"], cfg["cols"], M, cfg["r"], cfg["alpha"], wl.SEED_W + cfg["seed"])
    check_fwd_bwd(qn, c, f"decode M={M}", bwd=(M == 16))


@pytest.mark.parametrize("rows,cols,M,r", [
    (4096, 14336, 3, 16),   # sliced decode: 14 slices, 240-row bands
    (8200, 2048, 7, 5),     # whole-row decode, 2048 columns: 40-row bands
    (16384, 4096, 16, 16),  # whole-row decode: 64-row bands, M = 16
    (9000, 4096, 2, 13),    # whole-row decode: 40-row bands (a partial third group), rank 13
    (20000, 4096, 1, 16),   # whole-row decode: more bands than compute units, ragged last band
    (10008, 4096, 4, 1),    # whole-row decode: an 8-row last band, rank 1
    (9000, 2048, 16, 16),   # whole-row decode, 2048 columns, M = 16
    (1040, 3072, 1, 1),     # sliced decode: one row group per band, rank 1
    (1000, 1024, 5, 7),     # sliced decode: one slice, partial row group, odd rank
    (2048, 2048, 8, 32),    # rank 32: the two-kernel decode (u by extra workgroups)
    (264, 192, 9, 5),       # cols % 1024 != 0: the 32-row fused GEMM instead
    (3000, 8192, 1, 16),    # sliced decode: one row, eight column slices
    (776, 64, 1, 5),        # one row, one block per row, partial row group, rank 5 (fused GEMM)
    (2056, 4096, 2, 16),    # sliced decode: 16-row bands (too few rows for whole-row bands)
    (1000, 1536, 2, 3),     # two rows, 24 blocks per row (fused GEMM), rank 3
])
def test_decode_shapes(qn, rows, cols, M, r):
    c = Case(rows, cols, M, r, 2.0 * r, seed=rows + 3 * cols + M)
    check_fwd_bwd(qn, c, "decode", bwd=False)


def test_train_config_full_size(qn):
    cfg = wl.TRAIN
    c = Case(cfg["rows"], cfg["cols"], cfg["M"], cfg["r"], cfg["alpha"], wl.SEED_W + cfg["seed"])
    check_fwd_bwd(qn, c, "train 8192x4096x4096", rows=sample_rows(cfg["M"], 48, seed=4))


@pytest.mark.parametrize("rows,cols,M,r", [
    (264, 192, 37, 5),      # one partial tile, scalar adapter loads
    (3848, 3840, 4100, 16),  # the size at which the forward itself takes this product
    (1000, 1088, 1960, 16),  # 128 x 128 tiles (too few 256 x 256 ones), ragged edges
    (1024, 4096, 4096, 16),  # the decoder layer's k_proj shape: 128 x 128 tiles
    (648, 320, 3000, 7),    # 128 x 128 tiles, scalar adapter loads
    (7000, 1088, 4000, 16),  # 256 x 224 tiles (448 of 256 would need 2 rounds of 256 wide),
                             # a 56-column last tile
    (7168, 576, 4000, 7),   # 256 x 224 tiles, scalar adapter loads
])
def test_dense_lora_linear_bf16(qn, rows, cols, M, r):
    """lora_linear_bf16 on nf4_dequantize's bf16 weight: against the oracle,
    and bit-equal to qlora_linear_fwd where the forward runs this product."""
    say(f"[linear] lora_linear_bf16 rows={rows} cols={cols} M={M} r={r}")
    c = Case(rows, cols, M, r, 2.0 * r, seed=17 + rows)
    st, x, A, B, _ = c.dev(qn)
    y_fwd, u = qn.qlora_linear_fwd(st, x, A, B, c.alpha)
    Wb = qn.nf4_dequantize(st, torch.bfloat16)
    y = qn.lora_linear_bf16(x, Wb, u, B, c.alpha)
    torch.cuda.synchronize()
    sel = sample_rows(M, 48, seed=M)
    Y_ref, _ = oracle.qlora_fwd(c.Wd, c.x, c.A, c.B, c.s, rows=sel)
    ey = rel_err(bf16_host_f64(y)[sel], Y_ref)
    say(f"  rel err y={ey:.2e}")
    assert ey <= REL_TOL
    if qn.route(M, rows, cols, r) == "dense":
        assert torch.equal(y, y_fwd)


def test_lora_b_zero_is_exactly_base(qn):
    """B = 0: y equals the alpha = 0 output bit for bit; dA is exactly 0."""
    c = Case(520, 576, 300, 16, 32.0, seed=11)
    c.B[:] = 0
    st, x, A, B, G = c.dev(qn)
    y, u = qn.qlora_linear_fwd(st, x, A, B, c.alpha)
    y0, _ = qn.qlora_linear_fwd(st, x, A, B, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    _, dA, dB = qn.qlora_linear_bwd(st, x, G, A, B, c.alpha, u)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dA)) == 0 and float(dB.abs().sum()) > 0


def test_zero_weight_isolates_lora_term(qn):
    """W = 0 (all zero blocks): y is the adapter term alone, so an error in
    the LoRA path cannot hide under the base product."""
    c = Case(264, 192, 40, 8, 16.0, seed=12, adapter_std=0.05)
    c.W[:] = 0
    check_fwd_bwd(qn, c, "zero weight")


@pytest.mark.parametrize("rows,cols,M", [
    (1024, 512, 300),    # dequantization inside the GEMM
    (4096, 4096, 3840),  # bf16 copies of the weight and its transpose + dense GEMM
])
def test_one_hot_rows_read_dequantized_weight_exactly(qn, rows, cols, M):
    """B = 0 and x rows = e_k: y[m, :] = bf16(W'[:, k]) exactly; A = 0 and G
    rows = e_n: dX[m, :] = bf16(W'[n, :]) exactly (through the MFMA path)."""
    say(f"[linear] one-hot rows={rows} cols={cols} M={M}")
    c = Case(rows, cols, M, 16, 32.0, seed=13)
    _, Wb = oracle.dequantize(oracle.quantize(c.W))
    ks = np.arange(M) * 7 % cols
    x = np.zeros((M, cols), np.uint16)
    x[np.arange(M), ks] = 0x3F80  # bf16 1.0
    c.x = x
    c.B[:] = 0
    st, xd, A, B, G = c.dev(qn)
    y, _ = qn.qlora_linear_fwd(st, xd, A, B, c.alpha)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    want = wl.bf16_bits_to_f32(Wb[:, ks].T)
    assert np.array_equal(got, want)
    ns = np.arange(M) * 5 % rows
    g = np.zeros((M, rows), np.uint16)
    g[np.arange(M), ns] = 0x3F80
    c.A[:] = 0
    st, xd, A, B, _ = c.dev(qn)
    dX, _, _ = qn.qlora_linear_bwd(st, xd, bf16_dev(g), A, bf16_dev(c.B), c.alpha, None)
    torch.cuda.synchronize()
    assert np.array_equal(dX.float().cpu().numpy(), wl.bf16_bits_to_f32(Wb[ns, :]))


def test_empty_batch(qn):
    c = Case(64, 128, 1, 4, 8.0, seed=14)
    st, _, A, B, _ = c.dev(qn)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    G = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    y, u = qn.qlora_linear_fwd(st, x, A, B, c.alpha)
    assert y.shape == (0, 64)
    dX, dA, dB = qn.qlora_linear_bwd(st, x, G, A, B, c.alpha, None)
    torch.cuda.synchronize()
    assert dX.shape == (0, 128) and not dA.any() and not dB.any()


@pytest.mark.parametrize("rows,cols,M,r", [
    (1024, 1024, 4100, 20),  # transposed products: 96-row slices (3-step tail), two rank groups
    (2056, 1024, 4100, 17),  # 160-row slices (5 steps: tail after the unrolled loop)
])
def test_adapter_grads_repeat_identical(qn, rows, cols, M, r):
    """dA and dB of repeated backward calls are bit-identical and match the
    oracle (slice tails of the transposed products with more than 16 ranks)."""
    c = Case(rows, cols, M, r, 2.0 * r, seed=rows + cols + r)
    say(f"[linear] adapter-grad repeats: rows={rows} cols={cols} M={M} r={r}")
    st, x, A, B, G = c.dev(qn)
    _, u = qn.qlora_linear_fwd(st, x, A, B, c.alpha)
    outs = [qn.qlora_linear_bwd(st, x, G, A, B, c.alpha, u) for _ in range(3)]
    torch.cuda.synchronize()
    for dX, dA, dB in outs[1:]:
        assert torch.equal(dA, outs[0][1]) and torch.equal(dB, outs[0][2])
    dA_ref, dB_ref = oracle.adapter_grads(c.x, c.G, c.A, c.B, c.s)
    ea, eb = rel_err(outs[0][1].cpu().numpy(), dA_ref), rel_err(outs[0][2].cpu().numpy(), dB_ref)
    say(f"  rel err dA={ea:.2e} dB={eb:.2e}")
    assert ea <= REL_TOL and eb <= REL_TOL


@pytest.mark.parametrize("rows,cols,M,r", [
    (4096, 4096, 8192, 16),  # the training shape: 16 slices per column tile, vector finish
    (1024, 1024, 4100, 13),  # scalar finish (r % 4 != 0), 96-row slices
])
def test_backward_in_a_graph_replays_exactly(qn, rows, cols, M, r):
    """The backward captured in a HIP graph: every replay, with eager
    backward calls between replays (their own workspaces), equals the eager
    result bit for bit: the slices of dA and dB are added in slice order by
    whichever workgroup of a column tile arrives last, and the arrival
    counters are cleared by the call's first kernel."""
    c = Case(rows, cols, M, r, 2.0 * r, seed=rows + 5 * r)
    say(f"[linear] backward graph replays: rows={rows} cols={cols} M={M} r={r}")
    st, x, A, B, G = c.dev(qn)
    _, u = qn.qlora_linear_fwd(st, x, A, B, c.alpha)
    dX_ref, dA_ref, dB_ref = qn.qlora_linear_bwd(st, x, G, A, B, c.alpha, u)
    dX, dA, dB = torch.empty_like(dX_ref), torch.empty_like(dA_ref), torch.empty_like(dB_ref)
    L = qn.load_library()
    ws = torch.empty(L.qlora_linear_workspace(M, rows, cols, r, 1), dtype=torch.uint8,
                     device="cuda")
    s = st.c_struct()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.qlora_linear_bwd(qn.ctypes.byref(s), x.data_ptr(), G.data_ptr(), M, A.data_ptr(),
                           B.data_ptr(), r, float(c.alpha), u.data_ptr(), dX.data_ptr(),
                           dA.data_ptr(), dB.data_ptr(), ws.data_ptr(), ws.numel(),
                           torch.cuda.current_stream().cuda_stream)
    for k in range(3):
        dX.zero_()
        dA.zero_()
        dB.zero_()
        qn.qlora_linear_bwd(st, x, G, A, B, 1.0, u)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dX, dX_ref) and torch.equal(dA, dA_ref) and torch.equal(dB, dB_ref), k


def test_deterministic_repeat(qn):
    c = Case(520, 576, 300, 16, 32.0, seed=15)
    st, x, A, B, G = c.dev(qn)
    outs = []
    for _ in range(2):
        y, u = qn.qlora_linear_fwd(st, x, A, B, c.alpha)
        dX, dA, dB = qn.qlora_linear_bwd(st, x, G, A, B, c.alpha, u)
        torch.cuda.synchronize()
        outs.append((y.clone(), dX.clone(), dA.clone(), dB.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_autograd_module(qn):
    """QLoRALinear's autograd matches the oracle's gradients for L = sum(Y*G)."""
    c = Case(264, 192, 37, 8, 16.0, seed=16, adapter_std=0.05)
    W = f32_dev(c.W)
    mod = qn.QLoRALinear(W, r=8, alpha=16.0)
    with torch.no_grad():
        mod.lora_A.copy_(bf16_dev(c.A))
        mod.lora_B.copy_(bf16_dev(c.B))
    x = bf16_dev(c.x).requires_grad_(True)
    y = mod(x)
    (y.float() * bf16_dev(c.G).float()).sum().backward()
    torch.cuda.synchronize()
    Y_ref, _ = oracle.qlora_fwd(c.Wd, c.x, c.A, c.B, c.s)
    dX_ref, _ = oracle.qlora_dx(c.Wd, c.G, c.A, c.B, c.s)
    dA_ref, dB_ref = oracle.adapter_grads(c.x, c.G, c.A, c.B, c.s)
    assert rel_err(bf16_host_f64(y), Y_ref) <= REL_TOL
    assert rel_err(bf16_host_f64(x.grad), dX_ref) <= REL_TOL
    assert rel_err(mod.lora_A.grad.float().cpu().numpy(), dA_ref) <= 1e-2
    assert rel_err(mod.lora_B.grad.float().cpu().numpy(), dB_ref) <= 1e-2


@pytest.mark.parametrize("rows,M", [(14336, 4), (4096, 16), (1040, 1)])
def test_decode_calls_sharing_a_workspace_see_fresh_inputs(qn, rows, M):
    """Successive decode forwards through one workspace (partial sums of the
    previous call still in it) give exactly what separate workspaces give."""
    c = Case(rows, 4096, M, 16, 32.0, seed=33)
    st, x1, A, B, _ = c.dev(qn)
    x2 = bf16_dev(wl.normal_bf16((M, 4096), 34, 1.0))
    ref1, _ = qn.qlora_linear_fwd(st, x1, A, B, c.alpha)
    ref2, _ = qn.qlora_linear_fwd(st, x2, A, B, c.alpha)
    L = qn.load_library()
    ws = qn.linear_workspace(L.qlora_linear_workspace(M, rows, 4096, 16, 0))
    for xin, ref in ((x1, ref1), (x2, ref2), (x1, ref1), (x2, ref2)):
        y, _ = qn.qlora_linear_fwd(st, xin, A, B, c.alpha, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


@pytest.mark.parametrize("rows", [4096, 14336])
def test_decode_forward_in_a_graph_replays_exactly(qn, rows):
    """The decode forward captured in a HIP graph: every replay, with eager
    work between replays, equals the eager result bit for bit (the band sums
    do not depend on the order in which tiles arrive)."""
    c = Case(rows, 4096, 4, 16, 32.0, seed=21)
    st, x, A, B, _ = c.dev(qn)
    y_ref, u_ref = qn.qlora_linear_fwd(st, x, A, B, c.alpha)
    y = torch.empty_like(y_ref)
    u = torch.empty_like(u_ref)
    L = qn.load_library()
    ws = qn.linear_workspace(L.qlora_linear_workspace(4, rows, 4096, 16, 0))
    s = st.c_struct()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.qlora_linear_fwd(qn.ctypes.byref(s), x.data_ptr(), 4, A.data_ptr(), B.data_ptr(), 16,
                           32.0, y.data_ptr(), u.data_ptr(), ws.data_ptr(), ws.numel(),
                           torch.cuda.current_stream().cuda_stream)
    for k in range(3):
        y.zero_()
        u.zero_()
        qn.qlora_linear_fwd(st, x, A, B, 8.0)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(u, u_ref), k
