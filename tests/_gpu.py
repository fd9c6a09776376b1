"""Helpers for GPU parity tests: move seeded numpy inputs to the device and
device results back.  Every expected value comes from the CPU oracle."""
import sys

import numpy as np
import pytest
import torch

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

# Relative Frobenius bound for GEMM outputs and gradients against fp64.
REL_TOL = 5e-3


def say(*a):
    """Print and flush: names the case before each GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits, np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def state_np(st):
    torch.cuda.synchronize()
    return dict(packed=st.packed.cpu().numpy(), qscale=st.qscale.cpu().numpy(),
                scale2=st.scale2.cpu().numpy(), offset=st.offset.cpu().numpy()[0])


def rel_err(out, ref) -> float:
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(out - ref) / np.linalg.norm(ref))
