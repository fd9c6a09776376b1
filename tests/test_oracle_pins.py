"""Pins of the CPU oracle against facts the pages and the mathematics fix.

None of these re-types the oracle's own code: each compares it with a page
value (tests/golden, cited there), an exact rational or brute-force rule, a
library routine (torch's float8/bf16 casts, numpy fp64 matmul, torch
autograd), or an invariant that a plausible mistake would break.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests import _golden

LIT = np.array(_golden.values("nf4_codebook_page2.txt"), dtype=np.float64)


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


# --------------------------------------------------------------- codebook
def test_codebook_equals_page_literals(orc):
    cb = orc.codebook()
    assert cb.dtype == np.float32 and cb.size == 16
    # every page literal is exactly an fp32 value, and the oracle holds it
    assert np.array_equal(LIT.astype(np.float32).astype(np.float64), LIT)
    assert np.array_equal(cb.astype(np.float64), LIT)


def test_codebook_structure_page2(orc):
    g = _golden.table("page2_listing_checks.txt")
    cb = orc.codebook().astype(np.float64)
    assert (cb < 0).sum() == g["negative_levels"]
    assert (cb == 0).sum() == g["zero_levels"]
    assert (cb > 0).sum() == g["positive_levels"]
    assert ((cb >= -0.2) & (cb <= 0.2)).sum() == g["levels_in_0p2"]
    assert not np.allclose(cb, -cb[::-1])
    assert np.all(np.diff(cb) > 0) and cb[0] == -1.0 and cb[-1] == 1.0


def test_codebook_against_rounded_table_page5(orc):
    cb = orc.codebook().astype(np.float64)
    p5 = np.array(_golden.values("nf4_codebook_4dp_page5.txt"))
    close = np.abs(cb - p5) <= 0.5e-4 + 1e-12
    assert sorted(np.nonzero(~close)[0].tolist()) == [3, 8]


# --------------------------------------------------------------- code search
def exact_midpoints():
    """Midpoints of adjacent levels; exact in fp64 (sum of two fp32)."""
    m = (LIT[:-1] + LIT[1:]) / 2.0
    for k in range(15):
        assert Fraction(m[k]) == (Fraction(LIT[k]) + Fraction(LIT[k + 1])) / 2
    return m


def nearest_exact(n):
    """Nearest level of fp32 values n, ties to the lower code (exact rule)."""
    return np.searchsorted(exact_midpoints(), np.asarray(n, np.float64), side="left").astype(np.uint8)


def fp32_window(center: float, half: int):
    """All fp32 values within +-half ulps of center (sign-aware)."""
    c = np.float32(center)
    out = [c]
    up = dn = c
    for _ in range(half):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    return np.array(out, np.float32)


def test_code_search_near_every_midpoint(orc):
    vals = np.concatenate([fp32_window(m, 3000) for m in exact_midpoints()])
    assert np.array_equal(orc.nf4_codes(vals), nearest_exact(vals))


def test_code_search_random_and_special(orc):
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.uniform(-1, 1, 2_000_000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-38, -1e-38], np.float32),
        LIT.astype(np.float32),
    ])
    assert np.array_equal(orc.nf4_codes(vals), nearest_exact(vals))


def test_code_search_exhaustive_fp32(orc):
    """Every fp32 in [-1, 1] (about 2.13e9 values; ~30 s on 8 cores)."""
    one = int(np.float32(1.0).view(np.uint32))
    chunk = 1 << 25
    for sign in (0, 0x80000000):
        for start in range(0, one + 1, chunk):
            bits = np.arange(start, min(start + chunk, one + 1), dtype=np.uint32) | np.uint32(sign)
            vals = bits.view(np.float32)
            assert np.array_equal(orc.nf4_codes(vals), nearest_exact(vals)), start


def test_exact_ties_go_to_lower_code(orc):
    ties = [(k, m) for k, m in enumerate(exact_midpoints()) if float(np.float32(m)) == m]
    # exactly six midpoints are fp32 values
    assert [k for k, _ in ties] == [2, 6, 7, 9, 11, 13]
    for k, m in ties:
        assert orc.nf4_codes(np.array([m], np.float32))[0] == k


def brute_codes(W):
    """Codes by the page's rule, brute force: fp32 blocks of 64 (tail zero),
    absmax, fp32 division (zero block: divide by 1), exact nearest level with
    rational distances, ties to the lower code."""
    flat = np.asarray(W, np.float32).ravel()
    pad = (-flat.size) % 64
    blocks = np.concatenate([flat, np.zeros(pad, np.float32)]).reshape(-1, 64)
    lv = [Fraction(float(v)) for v in LIT]
    codes = []
    for blk in blocks:
        s = np.float32(np.max(np.abs(blk)))
        d = s if s > 0 else np.float32(1.0)
        for w in blk:
            n = Fraction(float(np.float32(w) / d))
            dist = [abs(n - L) for L in lv]
            codes.append(dist.index(min(dist)))
    return np.array(codes, np.uint8)


@pytest.mark.parametrize("shape", [(3, 64), (5, 77), (1, 1), (2, 33), (11, 13)])
def test_quantize_against_brute_force(orc, shape):
    rng = np.random.default_rng(sum(shape))
    W = (rng.standard_normal(shape) * rng.uniform(0.01, 3.0, size=(shape[0], 1))).astype(np.float32)
    if W.size > 70:
        W.ravel()[64:128] = 0.0  # a zero block
    st = orc.quantize(W, double_quant=False)
    codes = orc.codes_of(st)
    bc = brute_codes(W)
    assert codes.size == bc.size == 64 * ((W.size + 63) // 64)
    assert np.array_equal(codes, bc)
    # nibble order: element 2j is the low nibble of byte j
    assert np.array_equal(st.packed, (bc[0::2] | (bc[1::2] << 4)).astype(np.uint8))
    # first-level scale = fp32 absmax of each block
    flat = np.concatenate([W.ravel(), np.zeros((-W.size) % 64, np.float32)]).reshape(-1, 64)
    assert np.array_equal(st.absmax, np.abs(flat).max(axis=1))


# --------------------------------------------------------------- page-2 listing checks
def test_page2_listing_checks(orc):
    g = _golden.table("page2_listing_checks.txt")
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.2, (8, 8)).astype(np.float32)
    st = orc.quantize(w, double_quant=False)
    assert st.packed.size == g["pack_8x8_bytes"]
    assert st.absmax.nbytes == g["pack_8x8_scale_bytes"]
    z = orc.quantize(np.zeros((g["zeros_rows"], g["zeros_cols"]), np.float32), double_quant=True)
    f32, b16 = orc.dequantize(z)
    assert f32.shape == (3, 7) and np.count_nonzero(f32) == 0 and np.count_nonzero(b16 & 0x7FFF) == 0


@pytest.mark.parametrize("dq", [False, True])
def test_levels_round_trip_in_unit_block(orc, dq):
    lv = LIT.astype(np.float32)
    blk = np.concatenate([lv, lv[::-1], lv, np.zeros(16, np.float32)])
    st = orc.quantize(blk.reshape(1, 64), double_quant=dq)
    codes = orc.codes_of(st)
    assert np.array_equal(codes[:16], np.arange(16))
    assert np.array_equal(codes[16:32], np.arange(16)[::-1])
    assert np.all(codes[48:] == 7)
    f32, _ = orc.dequantize(st)
    assert np.array_equal(f32.ravel(), blk)


def test_errors_like_page_listing(orc):
    with pytest.raises(ValueError):
        orc.quantize(np.zeros((0,), np.float32))
    for bad in (np.nan, np.inf, -np.inf):
        w = np.ones((4, 64), np.float32)
        w[2, 5] = bad
        with pytest.raises(ValueError):
            orc.quantize(w)


# --------------------------------------------------------------- block conventions
def test_zero_and_constant_blocks(orc):
    W = np.random.default_rng(3).standard_normal((4, 256)).astype(np.float32) * 0.02
    W[0, 0:64] = 0.0
    W[1, 64:128] = 0.5
    W[2, 128:192] = -1e-3
    W[3, 192:256] = -0.0
    for dq in (False, True):
        st = orc.quantize(W, double_quant=dq)
        c = orc.codes_of(st).reshape(-1, 64)
        assert np.all(c[0] == 7) and np.all(c[4 * 3 + 3] == 7)
        assert np.all(c[1 * 4 + 1] == 15) and np.all(c[2 * 4 + 2] == 0)
        f32, _ = orc.dequantize(st)
        assert np.all(f32[0, 0:64] == 0) and np.all(f32[3, 192:256] == 0)
        if not dq:  # without DQ a constant block is exact
            assert np.all(f32[1, 64:128] == np.float32(0.5))
            assert np.all(f32[2, 128:192] == np.float32(-1e-3))
        else:  # with DQ it is the DQ'd scale, with the block's sign
            sp = np.float32(f32[1, 64])
            assert np.all(f32[1, 64:128] == sp) and sp > 0
            assert np.all(f32[2, 128:192] < 0)


def test_absmax_invariant(orc):
    W = np.random.default_rng(4).standard_normal((64, 320)).astype(np.float32) * 0.02
    st = orc.quantize(W)
    c = orc.codes_of(st).reshape(-1, 64)
    nonzero = st.absmax > 0
    assert np.all(((c == 0) | (c == 15)).any(axis=1)[nonzero])


# --------------------------------------------------------------- E4M3 and bf16
def torch_e4m3(x):
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_matches_torch(orc):
    ref = e4m3_values()
    for q in range(256):
        v = orc.e4m3_decode(q)
        if (q & 0x7F) == 0x7F:
            assert math.isnan(v) and math.isnan(ref[q])
        else:
            assert v == ref[q] and math.copysign(1, v) == math.copysign(1, ref[q])


def test_e4m3_encode_matches_torch(orc):
    vals = e4m3_values()
    fin = np.unique(vals[np.isfinite(vals) & (vals >= 0)]).astype(np.float64)
    mids = (fin[:-1] + fin[1:]) / 2.0
    xs = [np.float32(v) for v in fin]
    for m in mids:
        for w in fp32_window(m, 2):
            xs.append(w)
    rng = np.random.default_rng(11)
    xs += list(rng.uniform(-460, 460, 20000).astype(np.float32))
    xs += list((rng.standard_normal(20000) * 3).astype(np.float32))
    xs = np.array(xs + [-x for x in xs], np.float32)
    xs = xs[np.abs(xs) < 464]
    ours = np.array([orc.e4m3_encode(x) for x in xs], np.uint8)
    assert np.array_equal(ours, torch_e4m3(xs))


def test_e4m3_spot_values(orc):
    # round to nearest, ties to even mantissa; 449 and 463.9 round to 448
    assert orc.e4m3_decode(orc.e4m3_encode(1.0625)) == 1.0
    assert orc.e4m3_decode(orc.e4m3_encode(1.1875)) == 1.25
    assert orc.e4m3_decode(orc.e4m3_encode(449.0)) == 448.0
    assert orc.e4m3_decode(orc.e4m3_encode(463.9)) == 448.0
    # saturation reading beyond the format's range
    assert orc.e4m3_decode(orc.e4m3_encode(1000.0)) == 448.0
    assert orc.e4m3_decode(orc.e4m3_encode(-1000.0)) == -448.0
    assert orc.e4m3_decode(orc.e4m3_encode(2.0 ** -10)) == 0.0
    assert orc.e4m3_decode(orc.e4m3_encode(3 * 2.0 ** -11)) == 2.0 ** -9


def test_bf16_matches_torch(orc):
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10,
                         (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32)[:0x7F00],
                         np.array([0.0, -0.0, 1e-40, -1e-40], np.float32)])
    ref = torch.tensor(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([orc.bf16_rne(x) for x in xs], np.uint16)
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------- double quantisation
def test_scale_mean_exact_rational(orc):
    rng = np.random.default_rng(6)
    for nb in (1, 3, 255, 256, 257, 1000, 4096 + 17):
        s = rng.uniform(0.01, 2.0, nb).astype(np.float32)
        mu = orc.scale_mean(s)
        exact = sum(Fraction(float(v)) for v in s) / nb
        lo = np.nextafter(mu, np.float32(-np.inf))
        hi = np.nextafter(mu, np.float32(np.inf))
        # mu is the fp32 nearest the exact mean (the fp64 tree's error is far
        # below half an fp32 ulp for these sizes)
        assert abs(Fraction(float(mu)) - exact) <= abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(float(mu)) - exact) <= abs(Fraction(float(hi)) - exact)
    # exact cases
    assert orc.scale_mean(np.full(777, 0.375, np.float32)) == np.float32(0.375)
    assert orc.scale_mean(np.array([1.0, 2.0, 4.0, 8.0], np.float32)) == np.float32(3.75)


def test_dq_group_absmax_maps_to_448(orc):
    W = np.random.default_rng(8).standard_normal((512, 512)).astype(np.float32) * 0.02
    st = orc.quantize(W)
    vals = np.array([orc.e4m3_decode(q) for q in st.qscale], np.float64).reshape(-1, 256)
    for g in range(vals.shape[0]):
        assert st.scale2[g] > 0
        assert np.max(np.abs(vals[g])) == 448.0


def test_dq_constant_scales_give_zero_codes(orc):
    # every block has absmax 0.25 -> all scales equal the mean -> C2 = 0
    W = np.random.default_rng(9).uniform(-0.2, 0.2, (8, 1024)).astype(np.float32)
    W[:, ::64] = 0.25
    st = orc.quantize(W)
    assert st.offset == np.float32(0.25)
    assert np.all(st.scale2 == 0) and np.all(st.qscale == 0)
    f32, _ = orc.dequantize(st)
    st0 = orc.quantize(W, double_quant=False)
    f0, _ = orc.dequantize(st0)
    assert np.array_equal(f32, f0)  # s' = mu = s exactly


def test_dq_scale_error_bound(orc):
    W = np.random.default_rng(10).standard_normal((256, 1024)).astype(np.float32) * 0.02
    W[:, 3] *= 20
    st = orc.quantize(W)
    for b in range(0, st.absmax.size, 37):
        g = b // 256
        s2 = float(st.scale2[g])
        q = st.qscale[b]
        xv = orc.e4m3_decode(q)
        sp = float(np.float32(xv * s2 + float(st.offset))) if s2 > 0 else float(st.offset)
        # half an E4M3 step at |x| (step 2^(e-3), subnormal 2^-9) plus rounding
        x = (float(st.absmax[b]) - float(st.offset)) / s2
        e = max(math.floor(math.log2(abs(x))), -6) if x != 0 else -6
        bound = s2 * 2.0 ** (e - 3) / 2 * (1 + 1e-6) + 2 * abs(sp) * 2 ** -24
        assert abs(sp - float(st.absmax[b])) <= bound


def _dq_from_numpy(W):
    """The double-quantisation inputs recomputed from W with numpy alone
    (no oracle code): block absmax s_b of the flattened, zero-padded weight;
    the mean of the scales as the fp32 nearest the exact rational mean
    (math.fsum is exact before its one fp64 rounding, far below an fp32 half
    ulp); d_b = RN32(s_b - mu), C2_g = max |d_b| per 256 blocks,
    s2_g = RN32(C2_g / 448) (page "QLoRA Deep Dive: 4-bit NormalFloat &
    Double Quantization Internals", section "2. Squeezing More Memory:
    Double Quantization (DQ)": normalise the constants by their group
    absmax, then an 8-bit float code)."""
    flat = np.asarray(W, np.float32).ravel()
    pad = (-flat.size) % 64
    s = np.abs(np.concatenate([flat, np.zeros(pad, np.float32)]).reshape(-1, 64)).max(axis=1)
    nb = s.size
    mu = np.float32(math.fsum(s.astype(np.float64).tolist()) / nb)
    d = (s - mu).astype(np.float32)
    ng = (nb + 255) // 256
    dpad = np.concatenate([np.abs(d), np.zeros(ng * 256 - nb, np.float32)]).reshape(ng, 256)
    s2 = (dpad.max(axis=1) / np.float32(448.0)).astype(np.float32)
    return s, mu, d, s2


def _observed_block_scales(orc, st):
    """s'_b as the oracle's dequantize writes it: the value at the element of
    block b whose code is 15 (level +1) or 0 (level -1); NaN for blocks with
    neither (all-zero blocks)."""
    f32, _ = orc.dequantize(st, want_bf16=False)
    nb = st.absmax.size
    flat = np.concatenate([f32.ravel(), np.zeros(64 * nb - f32.size, np.float32)]).reshape(nb, 64)
    codes = orc.codes_of(st)[:64 * nb].reshape(nb, 64)
    sp = np.full(nb, np.nan, np.float64)
    for level_code, sign in ((15, 1.0), (0, -1.0)):
        has = (codes == level_code).any(axis=1) & np.isnan(sp)
        idx = np.argmax(codes == level_code, axis=1)
        sp[has] = sign * flat[np.nonzero(has)[0], idx[has]].astype(np.float64)
    return sp


def _dq_scale_bound(s, d, s2, sp):
    """|s'_b - s_b| bound: half an E4M3 step at x_b = d_b/s2_g (step 2^(e-3)
    in the binade [2^e, 2^(e+1)), 2^-9 below 2^-6) times s2_g, plus the fp32
    roundings of d_b, of x_b and of s' itself."""
    s2b = np.repeat(s2.astype(np.float64), 256)[:s.size]
    x = np.divide(d.astype(np.float64), s2b, out=np.zeros_like(s2b), where=s2b > 0)
    e = np.where(x != 0, np.floor(np.log2(np.abs(x), where=x != 0, out=np.zeros_like(x))), -6)
    e = np.maximum(e, -6)
    return s2b * 2.0 ** (e - 3) / 2 * (1 + 1e-6) + 2.0 ** -23 * (np.abs(d) + np.abs(sp))


def _check_dq_dequant_scale(orc, W):
    st = orc.quantize(W)
    s, mu, d, s2 = _dq_from_numpy(W)
    # the state's second level agrees with the independent recomputation
    assert st.offset == mu
    assert np.array_equal(st.scale2, s2)
    # the 8-bit scale codes are torch's E4M3FN rounding of RN32(d_b / s2_g)
    s2b = np.repeat(s2, 256)[:s.size]
    x = np.where(s2b > 0, d / np.where(s2b > 0, s2b, 1), 0).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(st.qscale, ref)
    # s'_b read back from the dequantized weight stays within the DQ error
    # of the exact block scale s_b, block by block
    sp = _observed_block_scales(orc, st)
    seen = ~np.isnan(sp)
    assert seen[s > 0].all()
    bound = _dq_scale_bound(s, d, s2, sp)
    err = np.abs(sp - s.astype(np.float64))
    bad = np.nonzero(seen & (err > bound))[0]
    assert bad.size == 0, (bad[:8], err[bad[:8]], bound[bad[:8]])
    return st, sp, s


def test_dq_dequant_scale_outlier_workload(orc):
    """Every block of the 4096x4096 quantize workload (N(0, 0.02), 1% of the
    columns x20, zero and constant blocks): the dequant scale s'_b that the
    oracle's dequantize applies is within the DQ error bound of s_b."""
    import workloads as wl
    _check_dq_dequant_scale(orc, wl.outlier_weight())


def test_dq_dequant_scale_groups_differ_tenfold(orc):
    """Groups of 256 blocks whose absmax differ 10x in turn (and a mean far
    from every group's scales): a dequant that took another group's s2, or
    left out the mean offset on some blocks, lands far outside the bound."""
    rng = np.random.default_rng(15)
    W = rng.standard_normal((16, 8 * 16384 // 16)).astype(np.float32) * np.float32(0.02)
    W = W.reshape(8, 16384)
    W *= np.float32(10.0) ** (np.arange(8) % 2).astype(np.float32)[:, None]
    W = W.reshape(64, -1)
    st, sp, s = _check_dq_dequant_scale(orc, W)
    # the construction really separates the groups and the mean
    g = s.reshape(8, 256)
    assert g[1].min() > 2 * g[0].max() and abs(float(st.offset) - g[0].mean()) > 10 * g[0].std()
    assert np.all(np.diff(st.scale2[:2]) > 0)


def test_storage_closed_form(orc):
    g = _golden.table("storage_bits.txt")
    for rows, cols in [(4096, 4096), (1024, 4096), (14336, 4096), (128, 128)]:
        n = rows * cols
        assert n % 16384 == 0
        nb, ng = n // 64, n // 16384
        st = orc.quantize(np.zeros((1, 64), np.float32))  # shape only of formats
        overhead = (8 * nb + 32 * ng) / n
        assert overhead == g["dq_overhead"]
        assert 4 + overhead == g["bits_dq"]
        assert 4 + 32 / 64 == g["bits_no_dq"]
        assert g["bits_no_dq"] - g["bits_dq"] == g["saving"]
    # the oracle's state really has those sizes
    W = np.zeros((128, 128), np.float32)
    st = orc.quantize(W)
    bits = 8 * (st.packed.size + st.qscale.size) + 32 * st.scale2.size
    assert bits / W.size == g["bits_dq"]


# --------------------------------------------------------------- dequantize
def test_dequant_bf16_is_rne_of_fp32(orc):
    W = np.random.default_rng(12).standard_normal((64, 448)).astype(np.float32) * 0.02
    f32, b16 = orc.dequantize(orc.quantize(W))
    ref = torch.tensor(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, ref)


def test_dequant_value_is_level_times_block_scale(orc):
    """Every dequantized value divided by its block's value at a code-15
    element (the scale itself) is a codebook level, exactly for these
    power-of-two scales."""
    rng = np.random.default_rng(13)
    W = rng.standard_normal((16, 64)).astype(np.float32)
    W *= (2.0 ** rng.integers(-8, 3, size=(16, 1))).astype(np.float32)
    # a power-of-two absmax at element 0 (code 15) makes every product exact
    W[np.arange(16), 0] = 2.0 ** np.ceil(np.log2(np.abs(W).max(axis=1)))
    st = orc.quantize(W, double_quant=False)
    f32, _ = orc.dequantize(st)
    codes = orc.codes_of(st).reshape(16, 64)
    for i in range(16):
        assert codes[i, 0] == 15
        assert np.array_equal(f32[i] / f32[i, 0], LIT.astype(np.float32)[codes[i]])


def test_reconstruction_error_magnitude(orc):
    g = _golden.table("reconstruction_error.txt")
    W = np.random.default_rng(14).standard_normal((1024, 1024)).astype(np.float32) * 0.02
    for dq in (False, True):
        f32, _ = orc.dequantize(orc.quantize(W, double_quant=dq))
        rel = np.linalg.norm(f32 - W) / np.linalg.norm(W)
        assert g["rel_frobenius_min"] <= rel <= g["rel_frobenius_max"]
        assert abs(rel - 0.092) < 0.003  # N(0, s) NF4 at block 64


# --------------------------------------------------------------- QLoRA linear oracle
def _lin(M, N, K, r, seed, B_zero=False):
    import workloads as wl
    W = wl.weight(N, K, seed)
    x = wl.normal_bf16((M, K), seed + 1, 1.0)
    A = wl.normal_bf16((r, K), seed + 2, 0.05)
    B = wl.normal_bf16((N, r), seed + 3, 0.05)
    if B_zero:
        B[:] = 0
    G = wl.normal_bf16((M, N), seed + 4, 1.0)
    return W, x, A, B, G


def _f64(bits):
    import workloads as wl
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def test_linear_oracle_matches_numpy_matmul(orc):
    M, N, K, r, s = 7, 40, 128, 3, 1.75
    W, x, A, B, G = _lin(M, N, K, r, 100)
    Wd, _ = orc.dequantize(orc.quantize(W))
    Y, u = orc.qlora_fwd(Wd, x, A, B, s)
    X64, A64, B64, G64, W64 = _f64(x), _f64(A), _f64(B), _f64(G), Wd.astype(np.float64)
    np.testing.assert_allclose(u, X64 @ A64.T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Y, X64 @ W64.T + s * (X64 @ A64.T) @ B64.T, rtol=1e-12, atol=1e-12)
    dX, v = orc.qlora_dx(Wd, G, A, B, s)
    np.testing.assert_allclose(v, G64 @ B64, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dX, G64 @ W64 + s * (G64 @ B64) @ A64, rtol=1e-12, atol=1e-12)
    dA, dB = orc.adapter_grads(x, G, A, B, s)
    np.testing.assert_allclose(dB, s * G64.T @ (X64 @ A64.T), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, s * (G64 @ B64).T @ X64, rtol=1e-12, atol=1e-12)
    # row selection computes the same rows
    rows = np.array([6, 0, 3])
    Yr, _ = orc.qlora_fwd(Wd, x, A, B, s, rows=rows)
    assert np.array_equal(Yr, Y[rows])
    dXr, _ = orc.qlora_dx(Wd, G, A, B, s, rows=rows)
    assert np.array_equal(dXr, dX[rows])


def test_linear_oracle_gradients_match_autograd(orc):
    """L = sum(Y * G) so dL/dY = G; torch autograd in fp64 gives dX, dA, dB."""
    M, N, K, r, s = 5, 24, 64, 4, 0.5
    W, x, A, B, G = _lin(M, N, K, r, 200)
    Wd, _ = orc.dequantize(orc.quantize(W))
    Xt = torch.tensor(_f64(x), requires_grad=True)
    At = torch.tensor(_f64(A), requires_grad=True)
    Bt = torch.tensor(_f64(B), requires_grad=True)
    Wt = torch.tensor(Wd.astype(np.float64))
    Y = Xt @ Wt.T + s * (Xt @ At.T) @ Bt.T
    (Y * torch.tensor(_f64(G))).sum().backward()
    dX, _ = orc.qlora_dx(Wd, G, A, B, s)
    dA, dB = orc.adapter_grads(x, G, A, B, s)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dB, Bt.grad.numpy(), rtol=1e-11, atol=1e-11)


def test_linear_oracle_finite_differences(orc):
    """Central differences of the fp64 forward pin one entry of each gradient."""
    M, N, K, r, s = 3, 8, 64, 2, 2.0
    W, x, A, B, G = _lin(M, N, K, r, 300)
    Wd, _ = orc.dequantize(orc.quantize(W))
    X64, A64, B64, G64, W64 = _f64(x), _f64(A), _f64(B), _f64(G), Wd.astype(np.float64)

    def loss(X, A_, B_):
        return float(np.sum((X @ W64.T + s * (X @ A_.T) @ B_.T) * G64))

    h = 1e-6
    dX, _ = orc.qlora_dx(Wd, G, A, B, s)
    dA, dB = orc.adapter_grads(x, G, A, B, s)
    for (i, j) in [(0, 5), (2, 63)]:
        E = np.zeros_like(X64); E[i, j] = h
        fd = (loss(X64 + E, A64, B64) - loss(X64 - E, A64, B64)) / (2 * h)
        assert abs(fd - dX[i, j]) <= 1e-6 * max(1, abs(fd))
    E = np.zeros_like(A64); E[1, 7] = h
    fd = (loss(X64, A64 + E, B64) - loss(X64, A64 - E, B64)) / (2 * h)
    assert abs(fd - dA[1, 7]) <= 1e-6 * max(1, abs(fd))
    E = np.zeros_like(B64); E[5, 0] = h
    fd = (loss(X64, A64, B64 + E) - loss(X64, A64, B64 - E)) / (2 * h)
    assert abs(fd - dB[5, 0]) <= 1e-6 * max(1, abs(fd))


def test_lora_b_zero_special_case(orc):
    """B = 0: output equals the base exactly, dA is exactly zero, dB is not."""
    M, N, K, r, s = 6, 32, 128, 4, 2.0
    W, x, A, B, G = _lin(M, N, K, r, 400, B_zero=True)
    Wd, _ = orc.dequantize(orc.quantize(W))
    Y, _ = orc.qlora_fwd(Wd, x, A, B, s)
    Yb, _ = orc.qlora_fwd(Wd, x, A, B, 0.0)
    assert np.array_equal(Y, Yb)
    dA, dB = orc.adapter_grads(x, G, A, B, s)
    assert np.count_nonzero(dA) == 0 and np.abs(dB).sum() > 0


def test_merge_identity(orc):
    """X W'^T + s X A^T B^T equals X (W' + s B A)^T (the merged operator)."""
    g = _golden.table("reconstruction_error.txt")
    M, N, K, r, s = 9, 48, 192, 5, 2.0
    W, x, A, B, _ = _lin(M, N, K, r, 500)
    Wd, _ = orc.dequantize(orc.quantize(W))
    Y, _ = orc.qlora_fwd(Wd, x, A, B, s)
    merged = Wd.astype(np.float64) + s * _f64(B) @ _f64(A)
    Ym = _f64(x) @ merged.T
    gap = np.max(np.abs(Y - Ym))
    assert gap <= 1e-12 * np.max(np.abs(Y)) and gap < g["merge_gap_fp32"] * 1e-3


# --------------------------------------------------------------- merge and requantize
# Page "QLoRA: NF4 storage, gradients and local integration", section "Merge
# changes the operator: test it explicitly", and the merge checks of the
# teaching listing: the adapter merged into Qhat(W) gives the operator used in
# training, merged into W it does not, and requantizing the merged weight
# changes the operator again.
def _merge_case(rows, cols, r, seed):
    import workloads as wl
    W = wl.weight(rows, cols, seed)
    A = wl.normal_bf16((r, cols), seed + 1, 0.05)
    B = wl.normal_bf16((rows, r), seed + 2, 0.05)
    return W, A, B


def _bf64(bits):
    return ((np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)).astype(np.float64)


def test_merge_is_the_nearest_fp32_of_the_exact_sum(orc):
    """Every merged value lies within half an fp32 ulp (plus the fp64 steps'
    slack) of the exact rational Qhat(W) + s B A; non-square shapes and
    several ranks, so a transposed operand or a dropped term fails."""
    for rows, cols, r, alpha in [(5, 7, 3, 6.0), (3, 64, 8, 16.0), (16, 9, 1, 1.0)]:
        W, A, B = _merge_case(rows, cols, r, seed=rows * 100 + cols)
        Wd, _ = orc.dequantize(orc.quantize(W), want_bf16=False)
        s = np.float32(alpha) / np.float32(r)
        got = orc.merge(Wd, A, B, s)
        Af, Bf = _bf64(A), _bf64(B)
        for n in range(rows):
            for k in range(cols):
                exact = Fraction(float(Wd[n, k])) + Fraction(float(s)) * sum(
                    Fraction(float(Bf[n, j])) * Fraction(float(Af[j, k])) for j in range(r))
                g = np.float32(got[n, k])
                ulp = float(np.spacing(np.float32(abs(float(exact)) or 1e-38)))
                assert abs(Fraction(float(g)) - exact) <= Fraction(ulp) / 2 * Fraction(1 + 2 ** -20)


def test_merge_with_zero_adapter_is_the_dequantized_weight(orc):
    W, A, B = _merge_case(24, 128, 4, seed=31)
    B[:] = 0
    Wd, _ = orc.dequantize(orc.quantize(W), want_bf16=False)
    assert np.array_equal(orc.merge(Wd, A, B, np.float32(8.0)), Wd)


def test_merge_distinguishes_the_three_operators(orc):
    """y of the separate adapter path = y of the merged weight (up to the fp32
    rounding of the merged weight), but not y of W + s B A (the original
    weight merged) and not y of the requantized merged weight."""
    import workloads as wl
    rows, cols, r = 64, 256, 8
    W, A, B = _merge_case(rows, cols, r, seed=41)
    s = np.float32(2.0)
    Wd, _ = orc.dequantize(orc.quantize(W), want_bf16=False)
    x = _bf64(wl.normal_bf16((32, cols), 42, 1.0))
    Af, Bf = _bf64(A), _bf64(B)
    separate = x @ Wd.astype(np.float64).T + float(s) * (x @ Af.T) @ Bf.T
    merged = orc.merge(Wd, A, B, s)
    y_merged = x @ merged.astype(np.float64).T
    assert np.linalg.norm(y_merged - separate) / np.linalg.norm(separate) < 1e-6
    original = W.astype(np.float64) + float(s) * Bf @ Af
    assert not np.allclose(original, merged.astype(np.float64))
    requant, _ = orc.dequantize(orc.quantize(merged), want_bf16=False)
    y_requant = x @ requant.astype(np.float64).T
    err = np.linalg.norm(y_requant - separate) / np.linalg.norm(separate)
    assert not np.allclose(y_requant, separate) and err > 1e-3


# --------------------------------------------------------------- adapter variants
# Course notebook FT-02: "Exercise 4: alpha/r vs alpha/sqrt(r) scaling
# (rsLoRA)", and the LoraConfig of the QLoRA setup (lora_dropout=0.05).
def test_rslora_scale(orc):
    # alpha fixed at 16, the exercise's ranks: alpha/sqrt(r) = 8, 4, 2 exactly
    assert [orc.lora_scale(16.0, r, rslora=True) for r in (4, 16, 64)] == [8.0, 4.0, 2.0]
    assert [orc.lora_scale(16.0, r) for r in (4, 16, 64)] == [4.0, 1.0, 0.25]
    # doubling the rank halves alpha/r but divides alpha/sqrt(r) by sqrt(2)
    for r in (4, 16):
        a, b = orc.lora_scale(16.0, r), orc.lora_scale(16.0, 2 * r)
        ra, rb = orc.lora_scale(16.0, r, True), orc.lora_scale(16.0, 2 * r, True)
        assert a / b == 2.0 and abs(ra / rb - math.sqrt(2)) < 1e-6
    # inverted dropout folds 1/(1-p) into the scale
    assert orc.lora_scale(32.0, 16, dropout_p=0.5) == 4.0


def _packed_mask(M, K, keep, seed):
    bits = np.random.default_rng(seed).random(M * K) < keep
    return np.packbits(bits, bitorder="little"), bits.reshape(M, K)


def test_dropout_gradients_match_autograd(orc):
    """The dropout variant against torch autograd in fp64 on
    y = x W'^T + s ((m (.) x) A^T) B^T with L = sum(y * G)."""
    import workloads as wl
    M, N, K, r = 6, 24, 64, 4
    W = wl.weight(N, K, 71)
    x, A, B, G = (wl.normal_bf16(sh, 72 + i, sd) for i, (sh, sd) in
                  enumerate([((M, K), 1.0), ((r, K), 0.1), ((N, r), 0.1), ((M, N), 1.0)]))
    mask, bits = _packed_mask(M, K, 0.7, 73)
    s = orc.lora_scale(8.0, r, dropout_p=0.3)
    Wd, _ = orc.dequantize(orc.quantize(W), want_bf16=False)
    y, _ = orc.qlora_fwd_dropout(Wd, x, A, B, s, mask)
    dX, _ = orc.qlora_dx_dropout(Wd, G, A, B, s, mask)
    dA, dB = orc.adapter_grads_dropout(x, G, A, B, s, mask)
    t = lambda a: torch.tensor(_bf64(a), dtype=torch.float64)
    xt = t(x).requires_grad_(True)
    At, Bt = t(A).requires_grad_(True), t(B).requires_grad_(True)
    mt = torch.tensor(bits, dtype=torch.float64)
    yt = xt @ torch.tensor(Wd, dtype=torch.float64).T + s * ((mt * xt) @ At.T) @ Bt.T
    (yt * t(G)).sum().backward()
    assert np.allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dX, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_dropout_special_masks(orc):
    """All kept: the plain linear at the same scale.  All dropped: the base
    product alone, zero adapter gradients, dX = G W'."""
    import workloads as wl
    M, N, K, r = 5, 16, 128, 3
    W, x, A, B, G = (wl.weight(N, K, 81), wl.normal_bf16((M, K), 82, 1.0),
                     wl.normal_bf16((r, K), 83, 0.1), wl.normal_bf16((N, r), 84, 0.1),
                     wl.normal_bf16((M, N), 85, 1.0))
    Wd, _ = orc.dequantize(orc.quantize(W), want_bf16=False)
    s = 2.0
    ones = np.full(M * K // 8, 0xFF, np.uint8)
    zeros = np.zeros(M * K // 8, np.uint8)
    y1, _ = orc.qlora_fwd_dropout(Wd, x, A, B, s, ones)
    y_ref, _ = orc.qlora_fwd(Wd, x, A, B, s)
    assert np.allclose(y1, y_ref, rtol=1e-13, atol=1e-13)
    dX1, _ = orc.qlora_dx_dropout(Wd, G, A, B, s, ones)
    assert np.array_equal(dX1, orc.qlora_dx(Wd, G, A, B, s)[0])
    y0, _ = orc.qlora_fwd_dropout(Wd, x, A, B, s, zeros)
    assert np.allclose(y0, orc.qlora_fwd(Wd, x, A, B, 0.0)[0], rtol=1e-13, atol=1e-13)
    dX0, _ = orc.qlora_dx_dropout(Wd, G, A, B, s, zeros)
    assert np.array_equal(dX0, orc.qlora_dx(Wd, G, A, B, 0.0)[0])
    dA0, dB0 = orc.adapter_grads_dropout(x, G, A, B, s, zeros)
    assert not dA0.any() and not dB0.any()


# --------------------------------------------------------------- FP4 codes and DQ off
# Course notebook FT-02: "Exercise 3: NF4 vs FP4 at equal memory" (FP4
# levels) and "Guided example 3: double quantization" (DQ on/off, 4.5 vs
# 4.127 bits per weight).
def test_fp4_levels_round_to_the_printed_table(orc):
    printed = np.array(_golden.values("fp4_levels_page1.txt"))
    cb = orc.fp4_codebook().astype(np.float64)
    assert np.array_equal(np.round(cb[:8], 4), printed)
    assert np.array_equal(cb[8:], -cb[:8])
    assert np.signbit(cb[8]) and cb[8] == 0.0 and cb[0] == 0.0 and not np.signbit(cb[0])
    # E2M1: sign, two exponent bits, one mantissa bit; with the subnormal
    # level 0.0625 (bitsandbytes' table), over the largest value 12
    e2m1 = np.array([0, 0.0625, 2, 3, 4, 6, 8, 12]) / 12
    assert np.array_equal(cb[:8], e2m1.astype(np.float32).astype(np.float64))
    assert np.all(np.diff(cb[:8]) > 0)


def _fp4_exact(n):
    """Sign of n and the nearest magnitude by exact rational distances,
    ties to the lower magnitude."""
    mags = [Fraction(float(np.float32(v))) for v in np.array([0, 0.0625, 2, 3, 4, 6, 8, 12]) / 12]
    out = []
    for v in np.asarray(n, np.float32):
        a = Fraction(abs(float(v)))
        d = [abs(a - m) for m in mags]
        k = min(range(8), key=lambda i: (d[i], i))
        out.append((8 if np.signbit(v) else 0) | k)
    return np.array(out, np.uint8)


def test_fp4_codes_brute_force(orc):
    cb = orc.fp4_codebook()
    mids = [(float(cb[k]) + float(cb[k + 1])) / 2 for k in range(7)]
    vals = np.concatenate([fp32_window(m, 200) for m in mids] +
                          [-fp32_window(m, 200) for m in mids] +
                          [np.random.default_rng(3).uniform(-1, 1, 20000).astype(np.float32),
                           np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45], np.float32)])
    assert np.array_equal(orc.fp4_codes(vals), _fp4_exact(vals))


def test_fp4_quantize_against_brute_force(orc):
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((7, 100)) * 0.02).astype(np.float32)
    W[2, :64] = 0.0
    st = orc.quantize(W, codebook="fp4")
    flat = np.concatenate([W.ravel(), np.zeros((-W.size) % 64, np.float32)]).reshape(-1, 64)
    s = np.abs(flat).max(axis=1)
    n = np.where(s[:, None] > 0, flat / np.where(s > 0, s, 1)[:, None], flat).astype(np.float32)
    assert np.array_equal(orc.codes_of(st)[:flat.size], _fp4_exact(n.ravel()))
    # every nonzero block holds its absmax at magnitude index 7 (+-1)
    codes = orc.codes_of(st)[:flat.size].reshape(-1, 64)
    assert all(((codes[b] & 7) == 7).any() for b in range(codes.shape[0]) if s[b] > 0)
    # dequantization: level times the block scale
    f32, _ = orc.dequantize(st, want_bf16=False)
    cbv = orc.fp4_codebook()
    assert f32.shape == W.shape
    ref = (cbv[codes.ravel()].reshape(codes.shape) *
           np.array([orc.e4m3_decode(q) * st.scale2[b // 256] + st.offset
                     for b, q in enumerate(st.qscale)], np.float32)[:, None])
    assert np.allclose(f32.ravel(), ref.ravel()[:W.size], rtol=1e-6, atol=0)


def test_dq_off_state_and_storage(orc):
    """DQ off: the state keeps the fp32 block scales and dequantization uses
    them as they are; 4 + 32/64 = 4.5 bits per weight against 4.127 with DQ."""
    g = _golden.table("storage_bits.txt")
    W = np.random.default_rng(5).standard_normal((64, 1024)).astype(np.float32) * 0.02
    for cb in ("nf4", "fp4"):
        st = orc.quantize(W, double_quant=False, codebook=cb)
        f32, _ = orc.dequantize(st, want_bf16=False)
        levels = orc.codebook() if cb == "nf4" else orc.fp4_codebook()
        codes = orc.codes_of(st)[:W.size].reshape(-1, 64)
        ref = (levels[codes] * st.absmax[:, None]).astype(np.float32)
        assert np.array_equal(f32.ravel().view(np.uint32), ref.ravel().view(np.uint32))
        bits = 8 * st.packed.size + 32 * st.absmax.size
        assert bits / W.size == g["bits_no_dq"]


# --------------------------------------------------------------- 8-bit AdamW
# Course notebook FT-02: the training arguments' optim="paged_adamw_8bit"
# (the Adam states kept in 8 bits) and the memory table's "Optimizer states
# (AdamW) 8 bytes/param (m + v)".
def _torch_adamw(p0, grads, lr, b1, b2, eps, wd):
    pt = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float32))
    opt = torch.optim.AdamW([pt], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                            foreach=False)
    for g in grads:
        pt.grad = torch.tensor(g, dtype=torch.float32)
        opt.step()
    return pt.detach().numpy().astype(np.float64)


def test_adamw8_first_step_is_adamw(orc):
    """From zero states the first update uses the fp32 moments before they
    are stored, so it is AdamW's (torch.optim.AdamW), up to rounding order."""
    rng = np.random.default_rng(21)
    n = 1000
    p0 = rng.standard_normal(n).astype(np.float32) * 0.05
    g = rng.standard_normal(n).astype(np.float32) * 1e-3
    hp = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    p = p0.copy()
    orc.adamw8_step(p, g, orc.Adam8State.zeros(n), step=1, **hp)
    ref = _torch_adamw(p0, [g], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    # within two fp32 ulps of the parameter (the two round in another order)
    assert np.all(np.abs(p.astype(np.float64) - ref) <= 2 * np.spacing(np.abs(p)))
    assert np.abs(ref - p0).max() > 1e4 * np.spacing(np.float32(0.05))  # a real step


def test_adamw8_tracks_adamw_over_steps(orc):
    """Twenty steps on random gradients: the 8-bit states move the parameters
    as fp32 AdamW does, within the states' 3-bit-mantissa precision."""
    rng = np.random.default_rng(22)
    n = 4096
    p0 = rng.standard_normal(n).astype(np.float32) * 0.05
    grads = [(rng.standard_normal(n) * 1e-3 + 5e-4).astype(np.float32) for _ in range(20)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    p, st = p0.copy(), orc.Adam8State.zeros(n)
    for t, g in enumerate(grads, 1):
        orc.adamw8_step(p, g, st, step=t, **hp)
    ref = _torch_adamw(p0, grads, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], 0.0)
    d, dref = p.astype(np.float64) - p0, ref - p0
    rel = np.linalg.norm(d - dref) / np.linalg.norm(dref)
    assert rel < 0.03, rel


def test_adamw8_states_hold_the_moments(orc):
    """After a step each stored moment decodes to within half an E4M3 step
    (at its magnitude relative to the block scale) of the fp32 moment, and
    every nonzero block holds a code of magnitude 448."""
    rng = np.random.default_rng(23)
    n = 700  # a partial last block
    g = rng.standard_normal(n).astype(np.float32) * 1e-2
    p, st = np.zeros(n, np.float32), orc.Adam8State.zeros(n)
    orc.adamw8_step(p, g, st, lr=1e-3, step=1)
    m = (np.float32(0.1) * g).astype(np.float64)        # (1 - b1) g
    v = ((np.float32(0.001) * g) * g).astype(np.float64)  # (1 - b2) g g
    for q, sc, x in ((st.mq, st.ms, m), (st.vq, st.vs, v)):
        dec = np.array([orc.e4m3_decode(c) for c in q], np.float64) * np.repeat(sc, 256)[:n]
        s = np.repeat(sc.astype(np.float64), 256)[:n]
        xs = np.abs(x) / s
        e = np.maximum(np.floor(np.log2(np.maximum(xs, 2.0 ** -9))), -6)
        assert np.all(np.abs(dec - x) <= s * 2.0 ** (e - 3) / 2 * (1 + 1e-6) + 1e-30)
        for b in range(sc.size):
            blk = q[256 * b:256 * b + 256]
            assert (blk & 0x7F).max() == 0x7E  # 448
    assert np.all(st.vq < 0x80)  # the second moment is never negative


def test_adamw8_decay_and_state_bytes(orc):
    """No gradient: the decoupled decay alone, p (1 - lr wd); the states take
    2 (1 + 4/256) bytes per parameter against the table's 8 for fp32 m and v."""
    p = np.linspace(-1, 1, 512).astype(np.float32)
    p0 = p.copy()
    orc.adamw8_step(p, np.zeros(512, np.float32), orc.Adam8State.zeros(512), lr=0.1,
                    weight_decay=0.5, step=3)
    assert np.array_equal(p, p0 * np.float32(1 - 0.1 * 0.5))
    st = orc.Adam8State.zeros(256 * 1000)
    per_param = (st.mq.nbytes + st.vq.nbytes + st.ms.nbytes + st.vs.nbytes) / st.mq.size
    assert per_param == 2 * (1 + 4 / 256) and per_param < 8
