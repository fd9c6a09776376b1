"""qlora_linear_fwd_noalloc (the forward for callers that cannot allocate:
its scratch is a static device array inside the library) against
qlora_linear_fwd through the C ABI: bit-identical outputs on two calls in a
row, the second with a smaller input, on each route whose scratch fits, and
the size error past the array."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from tests._gpu import bf16_dev, f32_dev, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def qn():
    import quantized_fine_tuning_nf4_amd as qn
    qn.load_library()
    return qn


def _case(qn, rows, cols, M, r, seed):
    W = wl.weight(rows, cols, seed)
    st = qn.nf4_quantize_dq(f32_dev(W))
    x = bf16_dev(wl.normal_bf16((M, cols), seed + 1, 1.0))
    A = bf16_dev(wl.normal_bf16((r, cols), seed + 2, 0.01))
    B = bf16_dev(wl.normal_bf16((rows, r), seed + 3, 0.01))
    return st, x, A, B


def _noalloc(qn, st, x, A, B, alpha, with_u=True):
    L = qn.load_library()
    M, r = x.shape[0], A.shape[0]
    y = torch.full((M, st.rows), 7.0, dtype=torch.bfloat16, device="cuda")
    u = torch.full((M, r), 7.0, dtype=torch.float32, device="cuda") if with_u else None
    s = st.c_struct()
    rc = L.qlora_linear_fwd_noalloc(ctypes.byref(s), x.data_ptr(), M, A.data_ptr(), B.data_ptr(),
                                    r, float(alpha), y.data_ptr(),
                                    None if u is None else u.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    return rc, y, u


@pytest.mark.parametrize("rows,cols,big,small,r", [
    (4096, 4096, 16, 3, 16),     # decode over column slices (counters and partial sums)
    (14336, 4096, 16, 1, 16),    # decode over whole rows
    (2048, 2048, 16, 5, 32),     # decode in two kernels (rank 32)
    (520, 576, 300, 37, 16),     # dequantization inside the GEMM tiles
    (4096, 14336, 16, 2, 16),    # decode over 14 column slices
])
def test_noalloc_matches_workspace_forward(qn, rows, cols, big, small, r):
    for M in (big, small):
        say(f"[noalloc] rows={rows} cols={cols} M={M} r={r} route={qn.route(M, rows, cols, r)}")
        st, x, A, B = _case(qn, rows, cols, M, r, seed=rows + cols + M)
        y_ref, u_ref = qn.qlora_linear_fwd(st, x, A, B, 2.0 * r)
        rc, y, u = _noalloc(qn, st, x, A, B, 2.0 * r)
        torch.cuda.synchronize()
        assert rc == qn.QN_OK
        assert torch.equal(y, y_ref) and torch.equal(u, u_ref)
        rc, y2, _ = _noalloc(qn, st, x, A, B, 2.0 * r, with_u=False)
        torch.cuda.synchronize()
        assert rc == qn.QN_OK and torch.equal(y2, y_ref)


def test_noalloc_rejects_what_does_not_fit(qn):
    L = qn.load_library()
    # the large-batch route keeps a bf16 copy of the weight: 32 MB here
    assert qn.route(8192, 4096, 4096, 16) == "dense"
    assert L.qlora_linear_workspace(8192, 4096, 4096, 16, 0) > (16 << 20)
    st, x, A, B = _case(qn, 4096, 4096, 8, 16, seed=5)
    x = torch.zeros((8192, 4096), dtype=torch.bfloat16, device="cuda")
    rc, _, _ = _noalloc(qn, st, x, A, B, 32.0)
    assert rc == qn.QN_EWORKSPACE
    # invalid sizes are refused before anything else
    s = st.c_struct()
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(s), x.data_ptr(), -1, A.data_ptr(),
                                      B.data_ptr(), 16, 32.0, x.data_ptr(), None, None) == \
        qn.QN_EINVAL


def test_noalloc_in_a_graph(qn):
    """Captured in a HIP graph (nothing to allocate at capture), replayed with
    eager calls between replays: every replay equals the eager forward."""
    st, x, A, B = _case(qn, 4096, 4096, 4, 16, seed=77)
    y_ref, u_ref = qn.qlora_linear_fwd(st, x, A, B, 32.0)
    L = qn.load_library()
    y = torch.empty_like(y_ref)
    u = torch.empty_like(u_ref)
    s = st.c_struct()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert L.qlora_linear_fwd_noalloc(ctypes.byref(s), x.data_ptr(), 4, A.data_ptr(),
                                          B.data_ptr(), 16, 32.0, y.data_ptr(), u.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream) == 0
    for k in range(3):
        y.zero_()
        u.zero_()
        _noalloc(qn, st, x[:1].contiguous(), A, B, 8.0)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(u, u_ref), k
