"""GPU adapter merge (nf4_merge_lora) and requantization against the CPU
oracle: the merged fp32 weight Qhat(W) + s B A and the requantized state
bit-exact (page "QLoRA: NF4 storage, gradients and local integration",
section "Merge changes the operator: test it explicitly")."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import bf16_dev, f32_dev, needs_gpu, say, state_np

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def qn():
    import quantized_fine_tuning_nf4_amd as qn
    qn.load_library()
    return qn


@pytest.mark.parametrize("rows,cols,r", [
    (256, 256, 8),      # the tiny workload's shape
    (5, 77, 3),         # ragged: blocks span rows, odd columns, a partial workgroup
    (1000, 1000, 5),    # rank not a multiple of 16
    (520, 576, 64),     # four rank chunks
    (4096, 4096, 16),   # the quantize workload's shape
])
def test_merge_and_requantize_bit_exact(qn, rows, cols, r):
    say(f"[merge] rows={rows} cols={cols} r={r}")
    W = wl.weight(rows, cols, 500 + rows + r)
    A = wl.normal_bf16((r, cols), 600 + r, 0.05)
    B = wl.normal_bf16((rows, r), 700 + r, 0.05)
    alpha = 2.0 * r
    st = qn.nf4_quantize_dq(f32_dev(W))
    merged = qn.nf4_merge_lora(st, bf16_dev(A), bf16_dev(B), alpha)
    st2 = qn.nf4_quantize_dq(merged)
    torch.cuda.synchronize()
    ref_state = oracle.quantize(W)
    Wd, _ = oracle.dequantize(ref_state, want_bf16=False)
    s = np.float32(alpha) / np.float32(r)
    ref = oracle.merge(Wd, A, B, s)
    got = merged.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    ref2 = oracle.quantize(ref)
    g2 = state_np(st2)
    assert np.array_equal(g2["packed"], ref2.packed)
    assert np.array_equal(g2["qscale"], ref2.qscale)
    assert np.array_equal(g2["scale2"].view(np.uint32), ref2.scale2.view(np.uint32))
    assert g2["offset"] == ref2.offset


def test_merge_with_zero_adapter_is_dequantize(qn):
    W = wl.weight(300, 448, 77)
    st = qn.nf4_quantize_dq(f32_dev(W))
    A = torch.randn(4, 448, device="cuda").to(torch.bfloat16)
    B = torch.zeros(300, 4, dtype=torch.bfloat16, device="cuda")
    merged = qn.nf4_merge_lora(st, A, B, 8.0)
    deq = qn.nf4_dequantize(st, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(merged, deq)
