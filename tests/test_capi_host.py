"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/qlora_nf4.h declares, and rejects bad arguments on the
host before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from tests import _golden

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def qn():
    import quantized_fine_tuning_nf4_amd as qn
    qn.load_library()
    return qn


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qlora_nf4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for f in ["nf4_quantize_dq", "nf4_dequantize", "qlora_linear_fwd", "qlora_linear_bwd"]:
        assert f in names


def test_library_exports_every_declared_symbol(qn):
    names = declared_functions()
    L = qn.load_library()
    for f in names:
        assert hasattr(L, f), f
    assert sorted(qn.EXPORTS) == names


def test_abi_version_and_status_strings(qn):
    L = qn.load_library()
    assert L.qn_abi_version() == 4
    for s in range(6):
        assert len(L.qn_status_str(s)) > 0
    assert L.qn_status_str(0) == b"ok"


def test_library_codebook_equals_page_table(qn):
    lit = np.array(_golden.values("nf4_codebook_page2.txt"), np.float32)
    assert np.array_equal(np.array(qn.codebook(), np.float32), lit)


def test_library_fp4_table_equals_the_oracles(qn):
    import oracle
    lib_t = np.array(qn.codebook("fp4"), np.float32)
    assert np.array_equal(lib_t.view(np.uint32), oracle.fp4_codebook().view(np.uint32))
    printed = np.array(_golden.values("fp4_levels_page1.txt"))
    assert np.array_equal(np.round(lib_t[:8].astype(np.float64), 4), printed)


def test_workspace_sizes(qn):
    L = qn.load_library()
    # arrival-counter page (left alone by the quantizer) | absmax fp32 [nb] |
    # fp64 partials [pow2(ng)] | group flags int [ng] | flag | the unused
    # mean of a call without double quantization, 256-aligned pieces
    nb, ng = 262144, 1024
    want = 4096 + nb * 4 + ng * 8 + ng * 4 + 256 + 4
    assert L.nf4_quantize_dq_workspace(4096, 4096) == want
    assert L.nf4_quantize_dq_workspace(0, 5) == 0
    assert L.qlora_linear_workspace(8192, 4096, 4096, 16, 0) >= 4096 + 8192 * 16 * 4
    b = L.qlora_linear_workspace(8192, 4096, 4096, 16, 1)
    assert b >= 4096 + 8192 * 16 * 4 * 2 + 16 * 4096 * 2
    assert L.qlora_linear_workspace(1, 8, 64, 65, 0) == 0
    # an empty batch is legal: its workspace query must not fault on the host
    # (the counter page is always part of a linear workspace)
    assert L.qlora_linear_workspace(0, 4096, 4096, 16, 0) == 4096
    assert L.qlora_linear_workspace(0, 4096, 4096, 16, 1) >= 4096
    # the largest batch the calls accept still sizes on the host
    assert L.qlora_linear_workspace(1 << 23, 14336, 4096, 16, 1) > (1 << 23) * 16 * 4


FAKE = 1 << 20  # a non-null, 256-aligned address that is never dereferenced


def _state(rows, cols, packed=FAKE):
    from quantized_fine_tuning_nf4_amd import _NF4DQ
    return _NF4DQ(packed, FAKE, FAKE, FAKE, rows, cols)


def test_argument_errors_are_host_side(qn):
    L = qn.load_library()
    EINVAL, EALIGN, EWS = qn.QN_EINVAL, qn.QN_EALIGN, qn.QN_EWORKSPACE
    # quantize
    q = L.nf4_quantize_dq
    assert q(None, 4, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == EINVAL
    assert q(FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == EINVAL
    assert q(FAKE + 4, 4, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == EALIGN
    assert q(FAKE, 4, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE + 16, 1 << 20, None) == EALIGN
    assert q(FAKE, 4, 4, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, 1 << 20, None) == EALIGN
    assert q(FAKE, 4096, 4096, FAKE, FAKE, FAKE, FAKE, None, FAKE, 100, None) == EWS
    # dequantize
    s = _state(0, 64)
    assert L.nf4_dequantize(ctypes.byref(s), 1, FAKE, None) == EINVAL
    s = _state(8, 64, packed=FAKE + 2)
    assert L.nf4_dequantize(ctypes.byref(s), 1, FAKE, None) == EALIGN
    s = _state(8, 64)
    assert L.nf4_dequantize(ctypes.byref(s), 7, FAKE, None) == EINVAL
    assert L.nf4_dequantize(None, 1, FAKE, None) == EINVAL
    # linear: cols % 64, rows % 8, rank range, M < 0, nulls, alignment, workspace
    for rows, cols, r, M in [(8, 65, 4, 2), (12, 64, 4, 2), (8, 64, 0, 2), (8, 64, 65, 2),
                             (8, 64, 4, -1)]:
        s = _state(rows, cols)
        assert L.qlora_linear_fwd(ctypes.byref(s), FAKE, M, FAKE, FAKE, r, 8.0, FAKE, None, FAKE,
                                  1 << 20, None) == EINVAL
        assert L.qlora_linear_bwd(ctypes.byref(s), FAKE, FAKE, M, FAKE, FAKE, r, 8.0, None,
                                  FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == EINVAL
    s = _state(8, 64)
    assert L.qlora_linear_fwd(ctypes.byref(s), None, 2, FAKE, FAKE, 4, 8.0, FAKE, None, FAKE,
                              1 << 20, None) == EINVAL
    assert L.qlora_linear_fwd(ctypes.byref(s), FAKE + 8, 2, FAKE, FAKE, 4, 8.0, FAKE, None, FAKE,
                              1 << 20, None) == EALIGN
    assert L.qlora_linear_fwd(ctypes.byref(s), FAKE, 2, FAKE, FAKE, 4, 8.0, FAKE, None, FAKE,
                              10, None) == EWS
    assert L.qlora_linear_bwd(ctypes.byref(s), FAKE, FAKE, 2, FAKE, FAKE, 4, 8.0, None, FAKE,
                              FAKE, FAKE, FAKE, 10, None) == EWS
    assert L.qlora_linear_bwd(ctypes.byref(s), FAKE, FAKE, 2, FAKE, FAKE, 4, 8.0, None, FAKE,
                              None, FAKE, FAKE, 1 << 20, None) == EINVAL
    # sizes past what the kernels' 32-bit buffer offsets allow are refused
    for rows, cols, M in [(8, 64, (1 << 23) + 1), ((1 << 20) + 8, 64, 2), (8, (1 << 20) + 64, 2)]:
        s2 = _state(rows, cols)
        assert L.qlora_linear_fwd(ctypes.byref(s2), FAKE, M, FAKE, FAKE, 4, 8.0, FAKE, None, FAKE,
                                  1 << 40, None) == EINVAL
        assert L.qlora_linear_bwd(ctypes.byref(s2), FAKE, FAKE, M, FAKE, FAKE, 4, 8.0, None,
                                  FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == EINVAL
    # M == 0 forward is a no-op that touches nothing
    assert L.qlora_linear_fwd(ctypes.byref(s), None, 0, None, None, 4, 8.0, None, None, None, 0,
                              None) == qn.QN_OK
    # dense LoRA linear on a bf16 weight: same shape rules, alignment, nulls
    for rows, cols, r, M in [(8, 65, 4, 2), (12, 64, 4, 2), (8, 64, 0, 2), (8, 64, 65, 2),
                             (8, 64, 4, -1), (0, 64, 4, 2)]:
        assert L.lora_linear_bf16(FAKE, M, FAKE, rows, cols, FAKE, FAKE, r, 8.0, FAKE,
                                  None) == EINVAL
    assert L.lora_linear_bf16(FAKE, 2, None, 8, 64, FAKE, FAKE, 4, 8.0, FAKE, None) == EINVAL
    assert L.lora_linear_bf16(FAKE, 2, FAKE, 8, 64, FAKE + 4, FAKE, 4, 8.0, FAKE, None) == EALIGN
    assert L.lora_linear_bf16(None, 0, None, 8, 64, None, None, 4, 8.0, None, None) == qn.QN_OK


def test_binding_rejects_cpu_tensors(qn):
    import torch
    with pytest.raises(ValueError):
        qn.nf4_quantize_dq(torch.zeros(4, 64))


def test_bench_refuses_more_than_one_gpu():
    # the measured path runs on one GPU; asking for more ends with a message
    # and a usage error before anything touches a device
    import json
    import subprocess
    import sys
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
