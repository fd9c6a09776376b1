"""GPU parity of nf4_quantize_dq / nf4_dequantize with the CPU oracle:
bit-exact codes, scale codes, second-level scales, offset and dequantized
weights (fp32 and bf16)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import bf16_bits, f32_dev, needs_gpu, say, state_np

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def qn():
    import quantized_fine_tuning_nf4_amd as qn
    qn.load_library()
    return qn


def check_quant(qn, W: np.ndarray, label: str):
    say(f"[quant] {label} shape={W.shape}")
    ref = oracle.quantize(W, double_quant=True)
    st = qn.nf4_quantize_dq(f32_dev(W))
    got = state_np(st)
    assert got["packed"].size == ref.packed.size
    nbad = int(np.count_nonzero(got["packed"] != ref.packed))
    assert nbad == 0, f"{nbad} packed bytes differ"
    assert np.array_equal(got["qscale"], ref.qscale)
    assert np.array_equal(got["scale2"].view(np.uint32), ref.scale2.view(np.uint32))
    assert np.float32(got["offset"]).view(np.uint32) == np.float32(ref.offset).view(np.uint32)
    # dequantize from the GPU state, compare with the oracle's dequant bits
    f32_ref, b16_ref = oracle.dequantize(ref)
    f = qn.nf4_dequantize(st, torch.float32)
    b = qn.nf4_dequantize(st, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(f.cpu().numpy().view(np.uint32), f32_ref.view(np.uint32))
    assert np.array_equal(bf16_bits(b), b16_ref)
    return st


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 77), (7, 1000), (2, 64), (1000, 1000),
                                       (37, 16384 + 64)])
def test_quant_parity_ragged(qn, rows, cols):
    W = wl.weight(rows, cols, seed=rows * 7 + cols, std=0.02)
    check_quant(qn, W, "ragged")


def test_quant_parity_tiny_config(qn):
    c = wl.TINY
    W = wl.weight(c["rows"], c["cols"], wl.SEED_W + c["seed"])
    check_quant(qn, W, "tiny 256x256")


def test_quant_parity_outlier_config(qn):
    W = wl.outlier_weight()
    st = check_quant(qn, W, "4096x4096 outliers, zero and constant blocks")
    # the zero blocks decode to zero, the constant blocks to +-s'
    Wd = qn.nf4_dequantize(st, torch.float32).cpu().numpy()
    assert np.all(Wd[0, 0:64] == 0) and np.all(Wd[4095, 63 * 64:] == 0)
    assert np.all(Wd[2048, 33 * 64:34 * 64] == Wd[2048, 33 * 64]) and Wd[2048, 33 * 64] > 0


@pytest.mark.parametrize("rows,cols", [(4104, 4096), (8192, 4096)])
def test_quant_parity_mid_mean_tree(qn, rows, cols):
    """1024 < ng <= 2048 groups: the scale pass forms the mean from eight
    partials per thread (1026 and 2048 groups)."""
    W = wl.weight(rows, cols, seed=rows + 3)
    check_quant(qn, W, f"{rows}x{cols}")


def test_quant_parity_long_mean_tree(qn):
    """ng > 4096 groups: the mean's tree runs two levels in global memory."""
    W = wl.weight(8192, 8320, seed=77)
    check_quant(qn, W, "8192x8320")


def test_quant_parity_decode_weight(qn):
    W = wl.weight(wl.FFN, wl.HIDDEN, wl.SEED_W + wl.DECODE["seed"])
    check_quant(qn, W, "14336x4096")


def _round_down_thresholds():
    L = oracle.codebook().astype(np.float64)
    m = (L[:-1] + L[1:]) / 2
    t = m.astype(np.float32)
    t = np.where(t.astype(np.float64) > m, np.nextafter(t, np.float32(-np.inf)), t)
    return t


def test_quant_near_thresholds_many_scales(qn):
    """Weights within a few ulps of every decision boundary, at 4096 random
    block scales: the GPU's division-free search must match RN32(w/s)."""
    rng = np.random.default_rng(123)
    nblk = 4096
    t = _round_down_thresholds()
    scales = (rng.uniform(0.5, 1.0, nblk) * 2.0 ** rng.integers(-30, 20, nblk)).astype(np.float32)
    W = np.zeros((nblk, 64), np.float32)
    W[:, 0] = scales
    W[::2, 0] *= -1
    ks = rng.integers(0, 15, (nblk, 63))
    base = (t[ks] * scales[:, None]).astype(np.float32)
    # step d ulps toward +inf (bits move up for positive, down for negative)
    d = rng.integers(-4, 5, (nblk, 63)).astype(np.int32)
    bits = base.view(np.int32)
    bits = np.where(base >= 0, bits + d, bits - d).astype(np.int32)
    W[:, 1:] = np.clip(bits.view(np.float32), -scales[:, None], scales[:, None])
    check_quant(qn, W, "near thresholds")


def test_quant_near_thresholds_subnormal_scales(qn):
    """As above with subnormal block scales (absmax below 2^-126): the
    weights near each boundary sit on the subnormal grid."""
    rng = np.random.default_rng(321)
    nblk = 2048
    t = _round_down_thresholds()
    scales = (rng.uniform(0.5, 1.0, nblk) * 2.0 ** rng.integers(-140, -126, nblk)).astype(np.float32)
    assert (scales < np.float32(2.0 ** -126)).all() and (scales > 0).all()
    W = np.zeros((nblk, 64), np.float32)
    W[:, 0] = scales
    W[1::2, 0] *= -1
    ks = rng.integers(0, 15, (nblk, 63))
    base = (t[ks].astype(np.float64) * scales[:, None].astype(np.float64)).astype(np.float32)
    d = rng.integers(-3, 4, (nblk, 63)).astype(np.int32)
    bits = base.view(np.int32)
    bits = np.where(base >= 0, bits + d, bits - d).astype(np.int32)
    W[:, 1:] = np.clip(bits.view(np.float32), -np.abs(W[:, :1]), np.abs(W[:, :1]))
    check_quant(qn, W, "near thresholds, subnormal scales")


def test_quant_unit_scale_sweep(qn):
    """Every 97th fp32 in [-1, 1] (about 22 M values) in blocks whose absmax
    is 1 (one element per block is +-1)."""
    one = int(np.float32(1.0).view(np.uint32))
    pos = np.arange(0, one + 1, 97, dtype=np.uint32)
    vals = np.concatenate([pos.view(np.float32), (pos | np.uint32(0x80000000)).view(np.float32)])
    nblk = (vals.size + 62) // 63
    W = np.zeros((nblk, 64), np.float32)
    W[:, 0] = 1.0
    flat = np.zeros(nblk * 63, np.float32)
    flat[:vals.size] = vals
    W[:, 1:] = flat.reshape(nblk, 63)
    check_quant(qn, W, "unit-scale sweep")


def test_quant_rejects_nonfinite(qn):
    for bad in (np.nan, np.inf, -np.inf):
        W = wl.weight(64, 256, seed=5)
        W[17, 100] = bad
        say(f"[quant] non-finite {bad}")
        with pytest.raises(qn.QNError) as e:
            qn.nf4_quantize_dq(f32_dev(W))
        assert e.value.status == qn.QN_ENONFINITE
    # a good weight after a failure still works (the flag is cleared)
    check_quant(qn, wl.weight(64, 256, seed=6), "after non-finite")


def test_quant_async_flag(qn):
    """With a device flag the call does not synchronize; the flag reads 1 for
    non-finite input, 0 otherwise, and the state equals the synchronous one."""
    import torch
    flag = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    W = wl.weight(512, 1024, seed=8)
    st_sync = qn.nf4_quantize_dq(f32_dev(W))
    st = qn.nf4_quantize_dq(f32_dev(W), nonfinite=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    a, b = state_np(st_sync), state_np(st)
    for k in ("packed", "qscale", "scale2", "offset"):
        assert np.array_equal(a[k], b[k]), k
    for bad in (np.nan, np.inf):
        Wb = W.copy()
        Wb[300, 1000] = bad
        qn.nf4_quantize_dq(f32_dev(Wb), nonfinite=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 1
    qn.nf4_quantize_dq(f32_dev(W), nonfinite=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0


def test_quant_deterministic(qn):
    W = f32_dev(wl.weight(2048, 4096, seed=9))
    a = state_np(qn.nf4_quantize_dq(W))
    b = state_np(qn.nf4_quantize_dq(W))
    for k in ("packed", "qscale", "scale2"):
        assert np.array_equal(a[k], b[k])
    assert a["offset"] == b["offset"]


def test_storage_bits_per_weight(qn):
    """4096 x 4096: 4 + 8/64 + 32/(64*256) bits per weight (offset excluded)."""
    st = qn.nf4_quantize_dq(f32_dev(wl.weight(4096, 4096, seed=1)))
    bits = 8 * (st.packed.numel() + st.qscale.numel()) + 32 * st.scale2.numel()
    assert bits / (4096 * 4096) == 4.126953125
