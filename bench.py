"""Benchmark of the QLoRA NF4 hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic batch of the
training-shaped workload (W 4096x4096 fp32 ~ N(0, 0.02), x and dY bf16
[8192, 4096] ~ N(0, 1), rank-16 bf16 adapters ~ N(0, 0.01), alpha 32):
    nf4_quantize_dq -> nf4_dequantize (bf16) -> qlora_linear_fwd -> qlora_linear_bwd
The headline value is the fwd+bwd algorithmic FLOPs of the step divided by
the wall time of the whole step (quantize and dequantize included).
Also printed in the same JSON line: the roofline of the dominant kernel,
the CPU oracle on a bounded sample, and per-kernel-group rates for the other
workloads (dequantize/quantize 4096x4096, decode forward, one decoder layer).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
M_TRAIN = 8192                 # rows of the training-shaped workload
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


# ----------------------------------------------------------------- accounting
def fwd_flops(M, N, K, r):
    """Algorithmic FLOPs of y = x W'^T + s (x A^T) B^T (dequant not counted)."""
    return 2 * M * N * K + 2 * M * r * (K + N)


def measured_traffic(profile, source):
    """HBM bytes per launch recorded in a committed rocprofv3 summary, or None
    when the kernel source has changed since the counters were taken."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
        sha = hashlib.sha256(open(os.path.join(ROOT, source), "rb").read()).hexdigest()
    except OSError:
        return None
    vals = dict(line.split(": ", 1) for line in text.splitlines()
                if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
    if vals.get("source_sha256", "").strip() != sha:
        return None
    return int(vals["traffic_bytes_per_launch"])


def gemm_flops(M, N, K, r):
    """Algorithmic FLOPs of one dense GEMM launch: x W'^T plus the fused
    LoRA-up term s u B^T (its bf16 high/low split is an implementation detail
    and not counted)."""
    return 2 * M * N * K + 2 * M * r * N


def bwd_flops(M, N, K, r):
    """dX = G W' + s (G B) A, dB = s G^T u, dA = s v^T x (u saved by fwd)."""
    return 2 * M * N * K + 2 * M * r * (N + K) + 2 * M * N * r + 2 * M * K * r


def state_bytes(rows, cols):
    n = rows * cols
    nb = (n + 63) // 64
    ng = (nb + 255) // 256
    return 32 * nb + nb + 4 * ng + 4


def dequant_bytes(rows, cols, out_bytes=2):
    return state_bytes(rows, cols) + out_bytes * rows * cols


def quant_bytes(rows, cols):
    return 4 * rows * cols + state_bytes(rows, cols)


def decode_bytes(rows, cols, M, r):
    """Algorithmic HBM bytes of one decode forward: the NF4 state, x, A, B, y."""
    return state_bytes(rows, cols) + 2 * M * cols + 2 * r * cols + 2 * rows * r + 2 * M * rows


def throughput(work, seconds):
    if not (math.isfinite(seconds) and seconds > 0):
        raise ValueError("invalid elapsed time")
    return work / seconds


def measure(step, batches, tokens, clock, sync, warmup):
    """Warmup excluded, synchronize, clock, run the measured batches,
    synchronize, clock; returns (seconds, work units).  (The measurement
    order of the page-2 measurement reference, without its allocator
    counters.)"""
    if type(warmup) is not int or warmup < 0 or len(batches) <= warmup:
        raise ValueError("warmup and a non-empty measured suffix are required")
    for b in batches[:warmup]:
        step(b)
    sync()
    t0 = clock()
    for b in batches[warmup:]:
        step(b)
    sync()
    elapsed = clock() - t0
    if not (math.isfinite(elapsed) and elapsed > 0):
        raise ValueError("invalid elapsed time")
    return elapsed, sum(tokens(b) for b in batches[warmup:])


# ----------------------------------------------------------------- GPU helpers
def _bf16(torch, a):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _event_time_ms(torch, fn, iters):
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(iters):
        fn(i)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def _median_min(xs):
    s = sorted(xs)
    return s[len(s) // 2], s[0]


def bench_train(torch, qn, wl, steps, warmup):
    cfg = wl.TRAIN
    N, K, M, r, alpha = cfg["rows"], cfg["cols"], cfg["M"], cfg["r"], cfg["alpha"]
    W, x, A, B, dY = wl.linear_inputs(N, K, M, r, seed=cfg["seed"])
    Wd = torch.from_numpy(W).cuda()
    xd, Ad, Bd, Gd = (_bf16(torch, a) for a in (x, A, B, dY))
    st = qn.empty_state(N, K, "cuda")
    L = qn.load_library()
    qws = torch.empty(L.nf4_quantize_dq_workspace(N, K), dtype=torch.uint8, device="cuda")
    fws = torch.empty(L.qlora_linear_workspace(M, N, K, r, 0), dtype=torch.uint8, device="cuda")
    bws = torch.empty(L.qlora_linear_workspace(M, N, K, r, 1), dtype=torch.uint8, device="cuda")
    wbf = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    flag = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(_):
        # asynchronous non-finite report: no host round trip inside the step
        qn.nf4_quantize_dq(Wd, out=st, workspace=qws, nonfinite=flag)
        qn.nf4_dequantize(st, torch.bfloat16, out=wbf)
        _, u = qn.qlora_linear_fwd(st, xd, Ad, Bd, alpha, y=y, workspace=fws)
        qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, alpha, u, workspace=bws)

    batches = list(range(warmup + steps))
    secs, nsteps = measure(step, batches, lambda b: 1, time.perf_counter,
                           torch.cuda.synchronize, warmup)
    if int(flag.item()) != 0:
        raise RuntimeError("quantizer reported non-finite input")
    flops = fwd_flops(M, N, K, r) + bwd_flops(M, N, K, r)
    res = dict(seconds=secs, steps=nsteps, ms_per_step=1e3 * secs / nsteps,
               tflops=flops * nsteps / secs / 1e12, flops_per_step=flops)

    # dominant kernels: time the forward and backward calls with HIP events on
    # the stream the library launches on (torch's current stream)
    u = torch.empty((M, r), dtype=torch.float32, device="cuda")

    def fwd(_):
        L.qlora_linear_fwd(qn.ctypes.byref(st.c_struct()), xd.data_ptr(), M, Ad.data_ptr(),
                           Bd.data_ptr(), r, float(alpha), y.data_ptr(), u.data_ptr(),
                           fws.data_ptr(), fws.numel(), torch.cuda.current_stream().cuda_stream)

    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((N, r), dtype=torch.float32, device="cuda")

    def bwd(_):
        L.qlora_linear_bwd(qn.ctypes.byref(st.c_struct()), xd.data_ptr(), Gd.data_ptr(), M,
                           Ad.data_ptr(), Bd.data_ptr(), r, float(alpha), u.data_ptr(),
                           dX.data_ptr(), dA.data_ptr(), dB.data_ptr(), bws.data_ptr(),
                           bws.numel(), torch.cuda.current_stream().cuda_stream)

    # the dominant kernel alone: the dense bf16 GEMM with the fused LoRA-up
    # term, which the forward runs after dequantizing (and dX on the
    # transposed copy); lora_linear_bf16 launches exactly that kernel
    wbf_fixed = qn.nf4_dequantize(st, torch.bfloat16)
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def gemm(_):
        L.lora_linear_bf16(xd.data_ptr(), M, wbf_fixed.data_ptr(), N, K, u.data_ptr(),
                           Bd.data_ptr(), r, float(alpha), y2.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)

    for f in (fwd, bwd, gemm):
        f(0)
    torch.cuda.synchronize()
    fwd_ms = [_event_time_ms(torch, fwd, 20) for _ in range(5)]
    bwd_ms = [_event_time_ms(torch, bwd, 20) for _ in range(5)]
    gemm_ms = [_event_time_ms(torch, gemm, 20) for _ in range(5)]
    res["fwd_call_ms"] = _median_min(fwd_ms)
    res["bwd_call_ms"] = _median_min(bwd_ms)
    res["gemm_ms"] = _median_min(gemm_ms)
    res["fwd_flops"] = fwd_flops(M, N, K, r)
    res["bwd_flops"] = bwd_flops(M, N, K, r)
    res["gemm_flops"] = gemm_flops(M, N, K, r)
    return res


def bench_extras(torch, qn, wl):
    import numpy as np
    L = qn.load_library()
    out = {}
    # quantize + dequantize of the 4096x4096 outlier weight, rotated copies
    W2 = torch.from_numpy(wl.outlier_weight()).cuda()
    R = 12
    states = [qn.nf4_quantize_dq(W2) for _ in range(R)]
    outs = [torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    torch.cuda.synchronize()
    ms = [_event_time_ms(torch, lambda i: qn.nf4_dequantize(states[i % R], torch.bfloat16,
                                                             out=outs[i % R]), 48)
          for _ in range(5)]
    med, mn = _median_min(ms)
    nbytes = dequant_bytes(4096, 4096, 2)
    out["dequant_bf16_4096x4096"] = dict(ms=med, ms_min=mn, bytes=nbytes,
                                         GBs=nbytes / med / 1e6,
                                         hbm_frac=nbytes / med / 1e6 / HBM_PEAK_GBS)
    outs32 = [torch.empty((4096, 4096), dtype=torch.float32, device="cuda") for _ in range(6)]
    ms = [_event_time_ms(torch, lambda i: qn.nf4_dequantize(states[i % 6], torch.float32,
                                                             out=outs32[i % 6]), 24)
          for _ in range(5)]
    med, mn = _median_min(ms)
    nbytes = dequant_bytes(4096, 4096, 4)
    out["dequant_f32_4096x4096"] = dict(ms=med, ms_min=mn, bytes=nbytes,
                                        GBs=nbytes / med / 1e6,
                                        hbm_frac=nbytes / med / 1e6 / HBM_PEAK_GBS)
    del outs, outs32
    # quantize with the device-side non-finite flag (no host round trip):
    # GPU time per call over 6 rotated fp32 inputs (6 x 67 MB, past the
    # 256 MB memory-side cache); the wall time of the synchronizing call is
    # reported beside it
    Ws = [torch.from_numpy(wl.weight(4096, 4096, 90 + i)).cuda() for i in range(6)]
    qws = torch.empty(L.nf4_quantize_dq_workspace(4096, 4096), dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(3):
        qn.nf4_quantize_dq(Ws[i % 6], out=states[i % R], workspace=qws, nonfinite=flag)
    torch.cuda.synchronize()
    ms = [_event_time_ms(torch, lambda i: qn.nf4_quantize_dq(Ws[i % 6], out=states[i % R],
                                                             workspace=qws, nonfinite=flag), 24)
          for _ in range(5)]
    med, mn = _median_min(ms)
    assert int(flag.item()) == 0
    t0 = time.perf_counter()
    n_q = 20
    for i in range(n_q):
        qn.nf4_quantize_dq(Ws[i % 6], out=states[i % R], workspace=qws)
    q_wall = (time.perf_counter() - t0) * 1e3 / n_q
    nbytes = quant_bytes(4096, 4096)
    out["quantize_dq_4096x4096"] = dict(ms=med, ms_min=mn, bytes=nbytes, GBs=nbytes / med / 1e6,
                                        hbm_frac=nbytes / med / 1e6 / HBM_PEAK_GBS,
                                        sync_call_wall_ms=q_wall)
    del Ws, states, W2
    torch.cuda.empty_cache()

    # decode forward 14336x4096, M = 1, 4, 16, rotated weight copies
    cfg = wl.DECODE
    N, K, r, alpha = cfg["rows"], cfg["cols"], cfg["r"], cfg["alpha"]
    Wq = torch.from_numpy(wl.weight(N, K, wl.SEED_W + 3)).cuda()
    base = qn.nf4_quantize_dq(Wq)
    R = 20
    copies = [qn.NF4State(base.packed.clone(), base.qscale.clone(), base.scale2.clone(),
                          base.offset.clone(), N, K) for _ in range(R)]
    del Wq
    A = _bf16(torch, wl.normal_bf16((r, K), wl.SEED_A + 3, 0.01))
    B = _bf16(torch, wl.normal_bf16((N, r), wl.SEED_B + 3, 0.01))
    dec = {}
    for M in cfg["Ms"]:
        x = _bf16(torch, wl.normal_bf16((M, K), wl.SEED_X + 3, 1.0))
        ws = torch.empty(L.qlora_linear_workspace(M, N, K, r, 0), dtype=torch.uint8, device="cuda")
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        us = [torch.empty((M, r), dtype=torch.float32, device="cuda") for _ in range(R)]
        stream = torch.cuda.current_stream().cuda_stream
        structs = [c.c_struct() for c in copies]

        def call(i):
            L.qlora_linear_fwd(qn.ctypes.byref(structs[i % R]), x.data_ptr(), M, A.data_ptr(),
                               B.data_ptr(), r, float(alpha), ys[i % R].data_ptr(),
                               us[i % R].data_ptr(), ws.data_ptr(), ws.numel(), stream)
        call(0)
        torch.cuda.synchronize()
        ms = [_event_time_ms(torch, call, 100) for _ in range(5)]
        med, mn = _median_min(ms)
        # the same R calls captured in one HIP graph: the GPU time of a decode
        # forward without the host's per-launch cost
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                L.qlora_linear_fwd(qn.ctypes.byref(structs[i]), x.data_ptr(), M, A.data_ptr(),
                                   B.data_ptr(), r, float(alpha), ys[i].data_ptr(),
                                   us[i].data_ptr(), ws.data_ptr(), ws.numel(),
                                   torch.cuda.current_stream().cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        gms = [_event_time_ms(torch, lambda _: g.replay(), 10) / R for _ in range(5)]
        gmed, gmn = _median_min(gms)
        nbytes = decode_bytes(N, K, M, r)
        dec[f"M{M}"] = dict(ms=med, ms_min=mn, graph_ms=gmed, graph_ms_min=gmn, bytes=nbytes,
                            GBs=nbytes / gmed / 1e6, hbm_frac=nbytes / gmed / 1e6 / HBM_PEAK_GBS,
                            eager_GBs=nbytes / med / 1e6)
        del g
    out["decode_fwd_14336x4096"] = dec
    del copies, base
    torch.cuda.empty_cache()

    # one decoder layer's seven linears, M = 4096, fwd + bwd
    cfg = wl.DECODER_LAYER
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    layers = []
    for idx, (name, N, K) in enumerate(wl.DECODER_LINEARS):
        W, x, A, B, G = wl.linear_inputs(N, K, M, r, seed=cfg["seed"], index=idx)
        st = qn.nf4_quantize_dq(torch.from_numpy(W).cuda())
        layers.append(dict(st=st, x=_bf16(torch, x), A=_bf16(torch, A), B=_bf16(torch, B),
                           G=_bf16(torch, G), N=N, K=K,
                           fws=torch.empty(L.qlora_linear_workspace(M, N, K, r, 0),
                                           dtype=torch.uint8, device="cuda"),
                           bws=torch.empty(L.qlora_linear_workspace(M, N, K, r, 1),
                                           dtype=torch.uint8, device="cuda"),
                           y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))

    def layer_step(_):
        for d in layers:
            _, u = qn.qlora_linear_fwd(d["st"], d["x"], d["A"], d["B"], alpha, y=d["y"],
                                       workspace=d["fws"])
            qn.qlora_linear_bwd(d["st"], d["x"], d["G"], d["A"], d["B"], alpha, u,
                                workspace=d["bws"])
    layer_step(0)
    torch.cuda.synchronize()
    ms = [_event_time_ms(torch, layer_step, 3) for _ in range(5)]
    med, mn = _median_min(ms)
    flops = sum(fwd_flops(M, d["N"], d["K"], r) + bwd_flops(M, d["N"], d["K"], r) for d in layers)
    out["decoder_layer_7_linears_M4096"] = dict(ms=med, ms_min=mn, flops=flops,
                                                TFLOPs=flops / med / 1e9,
                                                mfma_frac=flops / med / 1e9 / BF16_PEAK_TFLOPS,
                                                adapter_params=wl.adapter_params(r=r))
    del layers
    torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, target_s=15.0):
    """The oracle, untuned, on a bounded sample of the training workload:
    forward and input-gradient rows for a row sample, adapter gradients over
    a row block; reported as sampled FLOPs per second.  A 16-row probe sets
    the sample size so that the timed part takes about target_s seconds."""
    import numpy as np
    import oracle
    cfg = wl.TRAIN
    N, K, M, r, alpha = cfg["rows"], cfg["cols"], cfg["M"], cfg["r"], cfg["alpha"]
    W, x, A, B, dY = wl.linear_inputs(N, K, M, r, seed=cfg["seed"])
    s = alpha / r
    t0 = time.perf_counter()
    st = oracle.quantize(W)
    Wd, _ = oracle.dequantize(st, want_bf16=False)
    t_q = time.perf_counter() - t0

    def sample_flops(nr, mb):
        return (fwd_flops(nr, N, K, r) + 2 * nr * N * K + 2 * nr * r * (N + K)
                + 2 * mb * r * (K + N) + 2 * mb * N * r + 2 * mb * K * r)

    def run(nr, mb):
        rows = np.linspace(0, M - 1, nr).astype(np.int64)
        t1 = time.perf_counter()
        oracle.qlora_fwd(Wd, x, A, B, s, rows=rows)
        oracle.qlora_dx(Wd, dY, A, B, s, rows=rows)
        oracle.adapter_grads(x[:mb], dY[:mb], A, B, s)
        return time.perf_counter() - t1

    t_probe = run(16, 256)
    rate = sample_flops(16, 256) / max(t_probe, 1e-6)
    nr = int(min(M, max(16, target_s * rate / sample_flops(1, 16))))
    mb = min(M, 16 * nr)
    t_lin = run(nr, mb)
    flops = sample_flops(nr, mb)
    return dict(value=flops / t_lin / 1e12, unit="TFLOP/s", cores=oracle.num_threads(),
                kind="oracle",
                sample=(f"fp64 oracle: y and dX rows for {nr} of {M} rows, dA/dB over {mb} "
                        f"rows, at 4096x4096 r=16 ({flops / 1e9:.1f} GFLOP in {t_lin:.1f} s); "
                        f"quantize+dequantize 4096x4096 took {t_q:.2f} s"),
                seconds=t_lin)


def kernels_workload(torch, qn, wl, launches=5):
    """Fixed launches for rocprofv3 runs (--kernels): a plain 256 MiB device
    copy (the byte-counter calibration), then the dominant GEMM, the bf16
    dequantization, the decode forward and the quantizer, each `launches`
    times, synchronizing between groups."""
    import numpy as np
    L = qn.load_library()
    n_copy = 256 * 2 ** 20 // 4
    src = torch.ones(n_copy, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[kernels] copy {n_copy * 4} bytes x {launches}", file=sys.stderr, flush=True)
    cfg = wl.TRAIN
    N, K, M, r, alpha = cfg["rows"], cfg["cols"], cfg["M"], cfg["r"], cfg["alpha"]
    W, x, A, B, _ = wl.linear_inputs(N, K, M, r, seed=cfg["seed"])
    st = qn.nf4_quantize_dq(torch.from_numpy(W).cuda())
    xd, Bd = _bf16(torch, x), _bf16(torch, B)
    u = torch.randn(M, r, device="cuda", dtype=torch.float32) * 0.01
    wbf = qn.nf4_dequantize(st, torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    # bring the clocks up with other kernels (about 50 ms of bf16 matmuls),
    # so that the first of the GEMM launches below is not a cold one
    wa = torch.randn(4096, 4096, device="cuda").to(torch.bfloat16)
    for _ in range(40):
        wa = torch.mm(wa, wa.t().contiguous()) * 1e-3
    torch.cuda.synchronize()
    for _ in range(launches):
        qn.lora_linear_bf16(xd, wbf, u, Bd, alpha, y=y)
    torch.cuda.synchronize()
    print(f"[kernels] k_gemm_nt {M}x{N}x{K} x {launches}", file=sys.stderr, flush=True)
    for _ in range(launches):
        qn.nf4_dequantize(st, torch.bfloat16, out=wbf)
    torch.cuda.synchronize()
    print(f"[kernels] dequant bf16 {N}x{K} x {launches}", file=sys.stderr, flush=True)
    dcfg = wl.DECODE
    Nd, Kd = dcfg["rows"], dcfg["cols"]
    std = qn.nf4_quantize_dq(torch.from_numpy(wl.weight(Nd, Kd, wl.SEED_W + 3)).cuda())
    Ad = _bf16(torch, wl.normal_bf16((r, Kd), wl.SEED_A + 3, 0.01))
    Bdd = _bf16(torch, wl.normal_bf16((Nd, r), wl.SEED_B + 3, 0.01))
    xdec = _bf16(torch, wl.normal_bf16((16, Kd), wl.SEED_X + 3, 1.0))
    for _ in range(launches):
        qn.qlora_linear_fwd(std, xdec, Ad, Bdd, alpha)
    torch.cuda.synchronize()
    print(f"[kernels] decode forward M=16 {Nd}x{Kd} x {launches}", file=sys.stderr, flush=True)
    Wq = torch.from_numpy(wl.weight(N, K, wl.SEED_W + 90)).cuda()
    for _ in range(launches):
        qn.nf4_quantize_dq(Wq, out=st)
    torch.cuda.synchronize()
    print(f"[kernels] quantize {N}x{K} x {launches}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kernels", action="store_true",
                    help="only the fixed kernel launches used by the rocprofv3 summaries")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only: the hot path is measured "
                                   "on one MI355X; sharding across GPUs is described in the "
                                   "design notes, not implemented", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import quantized_fine_tuning_nf4_amd as qn
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qn.load_library()
    if args.kernels:
        kernels_workload(torch, qn, wl)
        return
    print(f"[bench] training step: {args.warmup} warmup + {args.steps} timed", file=sys.stderr,
          flush=True)
    tr = bench_train(torch, qn, wl, args.steps, args.warmup)
    fwd_med = tr["fwd_call_ms"][0]
    bwd_med = tr["bwd_call_ms"][0]
    g_med = tr["gemm_ms"][0]
    g_tf = tr["gemm_flops"] / g_med / 1e9
    roof = dict(bound="mfma", kernel="k_gemm_nt (dense bf16 GEMM + fused LoRA-up, 8192x4096x4096)",
                achieved=g_tf, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                frac=g_tf / BF16_PEAK_TFLOPS,
                traffic=measured_traffic("k_gemm_nt_8192x4096x4096.md",
                                         "quantized_fine_tuning_nf4_amd/csrc/gemm_bf16.hip"),
                traffic_unit="bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE, copy-calibrated)",
                algorithmic_bytes=2 * M_TRAIN * 4096 * 2 + 4096 * 4096 * 2,
                launch_ms=g_med, flops_per_launch=tr["gemm_flops"],
                fwd_call=dict(ms=fwd_med, TFLOPs=tr["fwd_flops"] / fwd_med / 1e9,
                              frac=tr["fwd_flops"] / fwd_med / 1e9 / BF16_PEAK_TFLOPS),
                bwd_call=dict(ms=bwd_med, TFLOPs=tr["bwd_flops"] / bwd_med / 1e9,
                              frac=tr["bwd_flops"] / bwd_med / 1e9 / BF16_PEAK_TFLOPS))
    extras = {}
    if not args.no_extras:
        print("[bench] extras", file=sys.stderr, flush=True)
        extras = bench_extras(torch, qn, wl)
    cpu = None
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)
    line = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s and NF4 dequant GB/s, % of MI355X roofline",
        "value": tr["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": tr["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "train_fwd_bwd_4096x4096_M8192", "rows": 4096, "cols": 4096,
                   "M": 8192, "r": 16, "alpha": 32,
                   "step": "nf4_quantize_dq (device non-finite flag) + nf4_dequantize(bf16) + "
                           "qlora_linear_fwd + qlora_linear_bwd", "flops_per_step": tr["flops_per_step"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
