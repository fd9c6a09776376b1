"""Seeded synthetic inputs for the QLoRA NF4 hot path.

This module only draws data: it holds none of the method's arithmetic, so
both the HIP path and the CPU oracle can be fed from it.  Every array is
drawn with ``numpy.random.default_rng(seed)`` (PCG64) as fp64 standard
normals, scaled, rounded to fp32; bf16 operands are the round-to-nearest-even
bf16 of that fp32 value (returned as uint16 bit patterns).

Shapes follow the pages' 7B-class example layer (hidden 4096, FFN 14336,
32 query / 8 key-value heads of 128, rank-16 adapters on the seven projection
targets: page "QLoRA: NF4 storage, gradients and local integration", section
"Memory accounting before optimization"), weights N(0, 0.02), activations and
upstream gradients N(0, 1), adapters N(0, 0.01).
"""
from __future__ import annotations

import numpy as np

# Seed bases: weight, activation, A, B, upstream gradient.
SEED_W, SEED_X, SEED_A, SEED_B, SEED_DY = 1000, 2000, 3000, 3100, 4000

HIDDEN, FFN, N_HEADS, N_KV_HEADS, HEAD_DIM = 4096, 14336, 32, 8, 128

# The seven adapted projections of one decoder layer: name -> (d_out, d_in).
DECODER_LINEARS = [
    ("q_proj", N_HEADS * HEAD_DIM, HIDDEN),
    ("k_proj", N_KV_HEADS * HEAD_DIM, HIDDEN),
    ("v_proj", N_KV_HEADS * HEAD_DIM, HIDDEN),
    ("o_proj", HIDDEN, N_HEADS * HEAD_DIM),
    ("gate_proj", FFN, HIDDEN),
    ("up_proj", FFN, HIDDEN),
    ("down_proj", HIDDEN, FFN),
]

# The synthetic workloads, by name; ``seed`` offsets the input seeds.
TINY = dict(name="tiny", seed=1, rows=256, cols=256, M=8, r=8, alpha=16.0)
QUANT_OUTLIERS = dict(name="quant_roundtrip_4096x4096_outliers", seed=2, rows=4096, cols=4096)
DECODE = dict(name="decode_fwd_14336x4096", seed=3, rows=FFN, cols=HIDDEN, Ms=(1, 4, 16), r=16,
              alpha=32.0)
TRAIN = dict(name="train_fwd_bwd_4096x4096_M8192", seed=4, rows=4096, cols=4096, M=8192, r=16,
             alpha=32.0)
DECODER_LAYER = dict(name="decoder_layer_7_linears_M4096", seed=5, M=4096, r=16, alpha=32.0)
WORKLOADS = {w["name"]: w for w in (TINY, QUANT_OUTLIERS, DECODE, TRAIN, DECODER_LAYER)}


def normal_f32(shape, seed: int, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * std).astype(np.float32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns of an fp32 array (via torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, seed: int, std: float) -> np.ndarray:
    return to_bf16_bits(normal_f32(shape, seed, std))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def weight(rows: int, cols: int, seed: int, std: float = 0.02) -> np.ndarray:
    return normal_f32((rows, cols), seed, std)



def equal_absmax_weight(rows: int, cols: int, seed: int) -> np.ndarray:
    """Every 64-block holds one element of +-0.25 and the rest inside
    (-0.2, 0.2), so every block's largest magnitude is 0.25, a power of two
    (with double quantization the scales' mean is 0.25 and every group's
    spread is 0; without it the stored scale is 0.25)."""
    rng = np.random.default_rng(seed)
    W = rng.uniform(-0.2, 0.2, (rows, cols)).astype(np.float32)
    pos = rng.integers(0, 64, size=(rows, cols // 64))
    sign = np.where(rng.integers(0, 2, size=pos.shape) == 1, 1.0, -1.0).astype(np.float32)
    W.reshape(rows, cols // 64, 64)[np.arange(rows)[:, None], np.arange(cols // 64)[None, :],
                                    pos] = 0.25 * sign
    return W

def outlier_weight(rows: int = 4096, cols: int = 4096, seed: int = SEED_W + 2) -> np.ndarray:
    """The quantize/dequantize round-trip weight: N(0, 0.02), 1% of the
    columns scaled x20, plus four all-zero and four constant 64-blocks."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    n_out = int(round(0.01 * cols))
    cols_out = rng.choice(cols, n_out, replace=False)
    W[:, cols_out] *= np.float32(20.0)
    last_r, last_b = rows - 1, cols // 64 - 1
    mid_r, mid_b = rows // 2, cols // 128
    for (r, b) in [(0, 0), (1, 1), (mid_r, mid_b), (last_r, last_b)]:
        W[r, 64 * b:64 * b + 64] = 0.0
    for (r, b, v) in [(0, 1, 0.02), (1, 2, -0.02), (mid_r, mid_b + 1, 0.5),
                      (last_r, last_b - 1, -1e-3)]:
        W[r, 64 * b:64 * b + 64] = np.float32(v)
    return W


def linear_inputs(rows: int, cols: int, M: int, r: int, seed: int, index: int = 0,
                  with_grad: bool = True, adapter_std: float = 0.01):
    """W fp32 [rows, cols]; x [M, cols], A [r, cols], B [rows, r], dY [M, rows]
    as bf16 bit patterns.  ``seed`` (a workload's) and ``index`` offset the
    seeds."""
    off = seed + 10 * index
    W = weight(rows, cols, SEED_W + off)
    x = normal_bf16((M, cols), SEED_X + off, 1.0)
    A = normal_bf16((r, cols), SEED_A + off, adapter_std)
    B = normal_bf16((rows, r), SEED_B + off, adapter_std)
    dY = normal_bf16((M, rows), SEED_DY + off, 1.0) if with_grad else None
    return W, x, A, B, dY


def adapter_params(linears=DECODER_LINEARS, r: int = 16) -> int:
    """Logical adapter parameter count r*(d_in + d_out) summed over targets."""
    return sum(r * (d_in + d_out) for _, d_out, d_in in linears)
