"""GPU 8-bit AdamW step (adamw8_step) against the CPU oracle, bit for bit:
parameters, their bf16 copy, the moments' E4M3 codes and block scales, over
several steps (course notebook FT-02, the training arguments'
optim="paged_adamw_8bit")."""
import numpy as np
import pytest
import torch

import oracle
from tests._gpu import f32_dev, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def qn():
    import quantized_fine_tuning_nf4_amd as qn
    qn.load_library()
    return qn


# 1310720: the decoder layer's adapter parameters (r = 16), as the benchmark times it
@pytest.mark.parametrize("n", [1, 255, 256, 1000, 65543, 131072, 1310720])
@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_adamw8_bit_exact(qn, n, wd):
    say(f"[adamw8] n={n} wd={wd}")
    rng = np.random.default_rng(n)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    pd = f32_dev(p0)
    opt = qn.Adam8(pd, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                   weight_decay=wd)
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    p, st = p0.copy(), oracle.Adam8State.zeros(n)
    for t in range(1, 6):
        g = (rng.standard_normal(n) * 1e-2 * t + (1e-3 if t % 2 else -2e-3)).astype(np.float32)
        if t == 3:
            g[: min(n, 300)] = 0.0  # a block whose moments decay
        opt.step(f32_dev(g), pb)
        ref_b = oracle.adamw8_step(p, g, st, step=t, want_bf16=True, **hp)
    torch.cuda.synchronize()
    assert np.array_equal(pd.cpu().numpy().view(np.uint32), p.view(np.uint32))
    assert np.array_equal(pb.cpu().view(torch.int16).numpy().view(np.uint16), ref_b)
    assert np.array_equal(opt.mq.cpu().numpy()[:n], st.mq)
    assert np.array_equal(opt.vq.cpu().numpy()[:n], st.vq)
    nb = st.ms.size
    assert np.array_equal(opt.ms.cpu().numpy()[:nb].view(np.uint32), st.ms.view(np.uint32))
    assert np.array_equal(opt.vs.cpu().numpy()[:nb].view(np.uint32), st.vs.view(np.uint32))


def test_adamw8_rejects_bad_hparams(qn):
    import ctypes
    L = qn.load_library()
    p = torch.zeros(256, device="cuda")
    mq = torch.zeros(256, dtype=torch.uint8, device="cuda")
    ms = torch.zeros(4, device="cuda")
    for h in [qn._AdamHP(1e-3, 0.9, 0.999, 1e-8, 0.0, 0), qn._AdamHP(1e-3, 1.0, 0.999, 1e-8, 0.0, 1)]:
        assert L.adamw8_step(p.data_ptr(), p.data_ptr(), 256, mq.data_ptr(), ms.data_ptr(),
                             mq.data_ptr(), ms.data_ptr(), None, ctypes.byref(h),
                             None) == qn.QN_EINVAL
