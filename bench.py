"""Benchmark of the QLoRA NF4 hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic batch of the
training-shaped workload (W 4096x4096 fp32 ~ N(0, 0.02), x and dY bf16
[8192, 4096] ~ N(0, 1), rank-16 bf16 adapters ~ N(0, 0.01), alpha 32):
    nf4_quantize_dq -> nf4_dequantize (bf16) -> qlora_linear_fwd -> qlora_linear_bwd
captured once in a HIP graph and replayed once per timed step (the same step
issued call by call from Python is timed too and reported beside it).
The headline value is the fwd+bwd algorithmic FLOPs of the step divided by
the wall time of the whole step (quantize and dequantize included).
Also printed in the same JSON line: the roofline of the dominant kernel,
the CPU oracle on a bounded sample, and per-kernel-group rates for the other
workloads (dequantize/quantize 4096x4096, decode forward, one decoder layer).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]
"""
from __future__ import annotations

import argparse
import dataclasses
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


def merge_bytes(rows, cols, r):
    """Algorithmic HBM bytes of one merge: the NF4 state, A, B and the fp32 output."""
    return state_bytes(rows, cols) + 2 * r * (rows + cols) + 4 * rows * cols


def decode_bytes(rows, cols, M, r):
    """Algorithmic HBM bytes of one decode forward: the NF4 state, x, A, B, y."""
    return state_bytes(rows, cols) + 2 * M * cols + 2 * r * cols + 2 * rows * r + 2 * M * rows


class Window:
    """What one timed window of repeated steps measured: its length in
    seconds, the steps and work units inside it, and the memory gauge at the
    window's start and its highest value during the window (bytes; None when
    the probe has no gauge)."""

    def __init__(self, seconds, steps, units, start_bytes=None, peak_bytes=None):
        if not (isinstance(seconds, (int, float)) and math.isfinite(seconds) and seconds > 0):
            raise ValueError(f"a timed window must last a positive finite time, got {seconds!r}")
        self.seconds, self.steps, self.units = float(seconds), steps, units
        self.start_bytes, self.peak_bytes = start_bytes, peak_bytes

    @property
    def rate(self):
        return self.units / self.seconds

    @property
    def peak_above_start(self):
        if self.start_bytes is None or self.peak_bytes is None:
            return None
        return self.peak_bytes - self.start_bytes


def time_window(run, items, units_of, untimed, probe):
    """Runs run(item) for every item; the first `untimed` items are warmup
    (outside the window and its work count), the rest are timed as one
    window.  probe.begin() is called once the warmup has been issued and
    must wait for it to finish before it stamps the start (and resets its
    peak gauge); probe.end() must wait for the timed steps before it stamps
    the stop; probe.seconds(start, stop) converts the two stamps.  A probe
    may also offer memory() -> (bytes at the start, peak bytes since).
    Returns a Window."""
    if isinstance(untimed, bool) or not isinstance(untimed, int) or untimed < 0:
        raise ValueError(f"the number of untimed steps must be an int >= 0, got {untimed!r}")
    items = list(items)
    if len(items) <= untimed:
        raise ValueError(f"{len(items)} steps leave none to time after {untimed} untimed ones")
    for item in items[:untimed]:
        run(item)
    start = probe.begin()
    units = 0
    for item in items[untimed:]:
        run(item)
        units += units_of(item)
    stop = probe.end()
    gauge = probe.memory() if hasattr(probe, "memory") else (None, None)
    return Window(probe.seconds(start, stop), len(items) - untimed, units, *gauge)


class DeviceProbe:
    """Window probe for the GPU: synchronizes the device at both ends and
    stamps the host clock there (the step's wall time, launches included);
    HIP events recorded on torch's current stream at the same two points
    give the device's own view of the window (device_seconds).  The memory
    gauge is torch's allocator (allocated bytes at the start, peak since)."""

    def __init__(self, torch):
        self.torch = torch
        self.device_seconds = None

    def begin(self):
        t = self.torch
        t.cuda.synchronize()
        t.cuda.reset_peak_memory_stats()
        self._start_bytes = t.cuda.memory_allocated()
        self._e0 = t.cuda.Event(enable_timing=True)
        self._e1 = t.cuda.Event(enable_timing=True)
        self._e0.record(t.cuda.current_stream())
        return time.perf_counter()

    def end(self):
        t = self.torch
        self._e1.record(t.cuda.current_stream())
        t.cuda.synchronize()
        stamp = time.perf_counter()
        self.device_seconds = self._e0.elapsed_time(self._e1) / 1e3
        return stamp

    def seconds(self, start, stop):
        return stop - start

    def memory(self):
        return self._start_bytes, self.torch.cuda.max_memory_allocated()


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


def _settled_times(torch, fn, iters, reps):
    """`reps` event timings of `iters` calls of fn each (ms per call), after
    running fn untimed for SETTLE_S / 2 so that the clocks have settled."""
    settle(torch, fn, SETTLE_S / 2)
    return [_event_time_ms(torch, fn, iters) for _ in range(reps)]


def _median_min(xs):
    s = sorted(xs)
    return s[len(s) // 2], s[0]


SETTLE_S = 0.05


def settle(torch, fn, seconds):
    """Run fn untimed until `seconds` of wall time have passed (at least
    once), synchronizing at the end; returns how many calls ran."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break
    torch.cuda.synchronize()
    return n


def bench_train(torch, qn, wl, steps, warmup):
    cfg = wl.TRAIN
    N, K, M, r, alpha = cfg["rows"], cfg["cols"], cfg["M"], cfg["r"], cfg["alpha"]
    W, x, A, B, dY = wl.linear_inputs(N, K, M, r, seed=cfg["seed"])
    Wd = torch.from_numpy(W).cuda()
    xd, Ad, Bd, Gd = (_bf16(torch, a) for a in (x, A, B, dY))
    st = qn.empty_state(N, K, "cuda")
    L = qn.load_library()
    qws = torch.empty(L.nf4_quantize_dq_workspace(N, K), dtype=torch.uint8, device="cuda")
    fws = qn.linear_workspace(L.qlora_linear_workspace(M, N, K, r, 0))
    bws = qn.linear_workspace(L.qlora_linear_workspace(M, N, K, r, 1))
    wbf = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    flag = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(_):
        # asynchronous non-finite report: no host round trip inside the step
        qn.nf4_quantize_dq(Wd, out=st, workspace=qws, nonfinite=flag)
        qn.nf4_dequantize(st, torch.bfloat16, out=wbf)
        _, u = qn.qlora_linear_fwd(st, xd, Ad, Bd, alpha, y=y, workspace=fws)
        return (u,) + qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, alpha, u, workspace=bws)

    # clocks settle first: the chip reaches its sustained clock only after
    # tens of milliseconds of this load (measured: 0.525-0.534 ms per step
    # after 3 warm-up steps, 0.486-0.487 after 50, on one box), so the step
    # runs untimed for at least SETTLE_S before the warm-up steps proper
    settle_steps = settle(torch, step, SETTLE_S)
    # the step as issued from Python, call by call
    probe = DeviceProbe(torch)
    eager = time_window(step, range(warmup + steps), lambda _: 1, warmup, probe)
    eager_device_s = probe.device_seconds
    # the same step captured once in a HIP graph and replayed: one replay is
    # one step (every kernel of the eager step, no host work between them)
    ref = [t.clone() for t in step(0)] + [y.clone()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(0)
    # (building the graph leaves the chip idle long enough for its clocks to
    # drop again: the replays settle the same way)
    settle_steps += settle(torch, lambda _: graph.replay(), SETTLE_S)
    probe = DeviceProbe(torch)
    win = time_window(lambda _: graph.replay(), range(warmup + steps), lambda _: 1, warmup, probe)
    if int(flag.item()) != 0:
        raise RuntimeError("quantizer reported non-finite input")
    # the replays computed what the eager step computes, bit for bit
    if not all(torch.equal(a, b) for a, b in zip(list(outs) + [y], ref)):
        raise RuntimeError("graph replay of the step differs from the eager step")
    flops = fwd_flops(M, N, K, r) + bwd_flops(M, N, K, r)
    secs, nsteps = win.seconds, win.steps
    res = dict(seconds=secs, steps=nsteps, ms_per_step=1e3 * secs / nsteps,
               settle_steps=settle_steps, settle_s=SETTLE_S,
               tflops=flops * nsteps / secs / 1e12, flops_per_step=flops,
               device_ms_per_step=1e3 * probe.device_seconds / nsteps,
               eager_ms_per_step=1e3 * eager.seconds / eager.steps,
               eager_device_ms_per_step=1e3 * eager_device_s / eager.steps,
               peak_bytes_above_start=win.peak_above_start)
    del graph

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
    settle(torch, lambda i: (fwd(i), bwd(i)), SETTLE_S)
    fwd_ms = [_event_time_ms(torch, fwd, 20) for _ in range(5)]
    bwd_ms = [_event_time_ms(torch, bwd, 20) for _ in range(5)]
    gemm_ms = [_event_time_ms(torch, gemm, 20) for _ in range(5)]
    res["fwd_call_ms"] = _median_min(fwd_ms)
    res["bwd_call_ms"] = _median_min(bwd_ms)
    res["gemm_ms"] = _median_min(gemm_ms)
    # the adapter-branch variants on the same workload: rsLoRA's scale (no
    # extra work) and dropout p = 0.05 on the branch's input (a keep mask in,
    # the u and dA products mask x as they load it, the branch's dX share is
    # added after the base product)
    mask = qn.dropout_mask(M, K, 0.05, generator=torch.Generator(device="cuda").manual_seed(7))
    dws = qn.linear_workspace(max(L.qlora_linear_workspace_ex(M, N, K, r, 1, None),
                                  L.qlora_linear_workspace_ex(
                                      M, N, K, r, 1, qn.ctypes.byref(qn._LoraOpts(0, 1, 0.05)))))

    def fwd_bwd_dropout(_):
        _, ud = qn.qlora_linear_fwd(st, xd, Ad, Bd, alpha, y=y, workspace=dws, dropout_mask=mask,
                                    dropout_p=0.05)
        qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, alpha, ud, workspace=dws, dropout_mask=mask,
                            dropout_p=0.05)

    fwd_bwd_dropout(0)
    torch.cuda.synchronize()
    res["fwd_bwd_dropout_ms"] = _median_min(_settled_times(torch, fwd_bwd_dropout, 10, 5))
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
    ms = _settled_times(torch, lambda i: qn.nf4_dequantize(states[i % R], torch.bfloat16,
                                                             out=outs[i % R]), 48, 5)
    med, mn = _median_min(ms)
    nbytes = dequant_bytes(4096, 4096, 2)
    out["dequant_bf16_4096x4096"] = dict(ms=med, ms_min=mn, bytes=nbytes,
                                         GBs=nbytes / med / 1e6,
                                         hbm_frac=nbytes / med / 1e6 / HBM_PEAK_GBS)
    outs32 = [torch.empty((4096, 4096), dtype=torch.float32, device="cuda") for _ in range(6)]
    ms = _settled_times(torch, lambda i: qn.nf4_dequantize(states[i % 6], torch.float32,
                                                             out=outs32[i % 6]), 24, 5)
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
    ms = _settled_times(torch, lambda i: qn.nf4_quantize_dq(Ws[i % 6], out=states[i % R],
                                                             workspace=qws, nonfinite=flag), 24, 5)
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
    # the format variants on the same weight: FP4 codes, double quantization
    # off (fp32 block scales): quantize and dequantize to bf16
    fmt = {}
    for cb, dq in (("fp4", True), ("nf4", False), ("fp4", False)):
        # 12 rotated states and outputs (> 2x the 256 MB memory-side cache),
        # as for the NF4 figures above
        sts = [qn.qn_quantize(Ws[i % 6], codebook=cb, double_quant=dq) for i in range(12)]
        torch.cuda.synchronize()
        qms = _settled_times(torch, lambda i: qn.qn_quantize(
            Ws[i % 6], codebook=cb, double_quant=dq, workspace=qws, nonfinite=flag), 24, 5)
        outs_fmt = [torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda")
                    for _ in range(12)]
        dms = _settled_times(torch, lambda i: qn.nf4_dequantize(sts[i % 12], torch.bfloat16,
                                                                  out=outs_fmt[i % 12]), 48, 5)
        sb = sts[0].nbytes()
        qb, db = 4 * 4096 * 4096 + sb, sb + 2 * 4096 * 4096
        qmed, dmed = _median_min(qms)[0], _median_min(dms)[0]
        fmt[f"{cb}_{'dq' if dq else 'nodq'}"] = dict(
            quantize_ms=qmed, quantize_hbm_frac=qb / qmed / 1e6 / HBM_PEAK_GBS,
            dequant_bf16_ms=dmed, dequant_hbm_frac=db / dmed / 1e6 / HBM_PEAK_GBS,
            state_bytes=sb, bits_per_weight=8 * sb / (4096 * 4096))
        del sts, outs_fmt
    out["formats_4096x4096"] = fmt

    # adapter merge Qhat(W) + s B A into fp32 (rank 16), rotated states
    Am = _bf16(torch, wl.normal_bf16((16, 4096), wl.SEED_A + 2, 0.01))
    Bm = _bf16(torch, wl.normal_bf16((4096, 16), wl.SEED_B + 2, 0.01))
    outs_m = [torch.empty((4096, 4096), dtype=torch.float32, device="cuda") for _ in range(6)]
    qn.nf4_merge_lora(states[0], Am, Bm, 32.0, out=outs_m[0])
    torch.cuda.synchronize()
    ms = _settled_times(torch, lambda i: qn.nf4_merge_lora(states[i % R], Am, Bm, 32.0,
                                                             out=outs_m[i % 6]), 24, 5)
    med, mn = _median_min(ms)
    nbytes = merge_bytes(4096, 4096, 16)
    out["merge_lora_4096x4096_r16"] = dict(ms=med, ms_min=mn, bytes=nbytes, GBs=nbytes / med / 1e6,
                                           hbm_frac=nbytes / med / 1e6 / HBM_PEAK_GBS)
    del Ws, states, W2, outs_m
    torch.cuda.empty_cache()

    # decode forward 14336x4096, M = 1, 4, 16, rotated weight copies
    cfg = wl.DECODE
    N, K, r, alpha = cfg["rows"], cfg["cols"], cfg["r"], cfg["alpha"]
    Wq = torch.from_numpy(wl.weight(N, K, wl.SEED_W + 3)).cuda()
    base = qn.nf4_quantize_dq(Wq)
    R = 20
    copies = [qn.NF4State(base.packed.clone(), base.qscale.clone(), base.scale2.clone(),
                          base.offset.clone(), N, K) for _ in range(R)]
    # the same weight in the other formats (FP4 codes, double quantization off)
    fmt_states = {f"{cb}_{'dq' if dq else 'nodq'}": qn.qn_quantize(Wq, codebook=cb, double_quant=dq)
                  for cb, dq in (("fp4", True), ("nf4", False), ("fp4", False))}
    del Wq
    A = _bf16(torch, wl.normal_bf16((r, K), wl.SEED_A + 3, 0.01))
    B = _bf16(torch, wl.normal_bf16((N, r), wl.SEED_B + 3, 0.01))
    dec = {}
    for M in cfg["Ms"]:
        x = _bf16(torch, wl.normal_bf16((M, K), wl.SEED_X + 3, 1.0))
        ws = qn.linear_workspace(L.qlora_linear_workspace(M, N, K, r, 0))
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
        ms = _settled_times(torch, call, 100, 5)
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
        gms = [t / R for t in _settled_times(torch, lambda _: g.replay(), 10, 5)]
        gmed, gmn = _median_min(gms)
        nbytes = decode_bytes(N, K, M, r)
        dec[f"M{M}"] = dict(ms=med, ms_min=mn, graph_ms=gmed, graph_ms_min=gmn, bytes=nbytes,
                            GBs=nbytes / gmed / 1e6, hbm_frac=nbytes / gmed / 1e6 / HBM_PEAK_GBS,
                            eager_GBs=nbytes / med / 1e6)
        del g
    # M = 1 in the other formats: the same kernels with their level table and
    # block-scale source (graph of R rotated copies)
    M = 1
    x = _bf16(torch, wl.normal_bf16((M, K), wl.SEED_X + 3, 1.0))
    for name, st0 in fmt_states.items():
        fc = [dataclasses.replace(st0, **{f: (None if getattr(st0, f) is None
                                              else getattr(st0, f).clone())
                                          for f in ("packed", "qscale", "scale2", "offset",
                                                    "absmax")}) for _ in range(R)]
        fs = [c.c_struct() for c in fc]
        ws = qn.linear_workspace(L.qlora_linear_workspace_state(qn.ctypes.byref(fs[0]), M, r, 0,
                                                                None))
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        us = [torch.empty((M, r), dtype=torch.float32, device="cuda") for _ in range(R)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                L.qlora_linear_fwd(qn.ctypes.byref(fs[i]), x.data_ptr(), M, A.data_ptr(),
                                   B.data_ptr(), r, float(alpha), ys[i].data_ptr(),
                                   us[i].data_ptr(), ws.data_ptr(), ws.numel(),
                                   torch.cuda.current_stream().cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        gmed, gmn = _median_min([t / R for t in _settled_times(torch, lambda _: g.replay(), 10, 5)])
        nbytes = decode_bytes(N, K, M, r) - state_bytes(N, K) + st0.nbytes()
        dec[f"M1_{name}"] = dict(graph_ms=gmed, graph_ms_min=gmn, bytes=nbytes,
                                 GBs=nbytes / gmed / 1e6,
                                 hbm_frac=nbytes / gmed / 1e6 / HBM_PEAK_GBS)
        del g, fc, fs
    out["decode_fwd_14336x4096"] = dec
    del copies, base, fmt_states
    torch.cuda.empty_cache()

    # 8-bit AdamW step over the decoder layer's adapters (1,310,720
    # parameters: A and B of the seven rank-16 targets), fp32 gradients
    n_ad = wl.adapter_params(r=16)
    pa = torch.randn(n_ad, device="cuda") * 0.01
    ga = torch.randn(n_ad, device="cuda") * 1e-3
    pab = torch.empty(n_ad, dtype=torch.bfloat16, device="cuda")
    opt = qn.Adam8(pa, lr=2e-4)
    opt.step(ga, pab)
    torch.cuda.synchronize()
    ms = _settled_times(torch, lambda i: opt.step(ga, pab), 50, 5)
    med, mn = _median_min(ms)
    nbytes = n_ad * (4 + 4 + 4 + 2 + 2 + 2) + 4 * 4 * ((n_ad + 255) // 256)
    out["adamw8_step_decoder_layer_adapters"] = dict(
        ms=med, ms_min=mn, params=n_ad, bytes=nbytes, GBs=nbytes / med / 1e6,
        hbm_frac=nbytes / med / 1e6 / HBM_PEAK_GBS)
    del pa, ga, pab, opt

    # one decoder layer's seven linears, M = 4096, fwd + bwd
    cfg = wl.DECODER_LAYER
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    layers = []
    for idx, (name, N, K) in enumerate(wl.DECODER_LINEARS):
        W, x, A, B, G = wl.linear_inputs(N, K, M, r, seed=cfg["seed"], index=idx)
        st = qn.nf4_quantize_dq(torch.from_numpy(W).cuda())
        layers.append(dict(st=st, x=_bf16(torch, x), A=_bf16(torch, A), B=_bf16(torch, B),
                           G=_bf16(torch, G), N=N, K=K,
                           fws=qn.linear_workspace(L.qlora_linear_workspace(M, N, K, r, 0)),
                           bws=qn.linear_workspace(L.qlora_linear_workspace(M, N, K, r, 1)),
                           y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))

    def layer_step(_):
        outs = []
        for d in layers:
            _, u = qn.qlora_linear_fwd(d["st"], d["x"], d["A"], d["B"], alpha, y=d["y"],
                                       workspace=d["fws"])
            outs += [u] + list(qn.qlora_linear_bwd(d["st"], d["x"], d["G"], d["A"], d["B"],
                                                   alpha, u, workspace=d["bws"]))
        return outs
    ref = [t.clone() for t in layer_step(0)] + [d["y"].clone() for d in layers]
    torch.cuda.synchronize()
    # as issued from Python, call by call
    eager_med, eager_mn = _median_min(_settled_times(torch, layer_step, 3, 5))
    # the fourteen calls captured once in a HIP graph and replayed (no host
    # work between the kernels), as the training step is timed
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gouts = layer_step(0)
    ms = _settled_times(torch, lambda _: graph.replay(), 3, 5)
    if not all(torch.equal(a, b) for a, b in zip(gouts + [d["y"] for d in layers], ref)):
        raise RuntimeError("graph replay of the decoder layer differs from the eager calls")
    del graph, gouts, ref
    med, mn = _median_min(ms)
    flops = sum(fwd_flops(M, d["N"], d["K"], r) + bwd_flops(M, d["N"], d["K"], r) for d in layers)
    # each linear's forward and backward on its own (same inputs, eager calls)
    per = {}
    for (name, N, K), d in zip(wl.DECODER_LINEARS, layers):
        def f_call(_, d=d):
            qn.qlora_linear_fwd(d["st"], d["x"], d["A"], d["B"], alpha, y=d["y"],
                                workspace=d["fws"])
        _, u = qn.qlora_linear_fwd(d["st"], d["x"], d["A"], d["B"], alpha, y=d["y"],
                                   workspace=d["fws"])

        def b_call(_, d=d, u=u):
            qn.qlora_linear_bwd(d["st"], d["x"], d["G"], d["A"], d["B"], alpha, u,
                                workspace=d["bws"])
        b_call(0)
        torch.cuda.synchronize()
        fm, _ = _median_min(_settled_times(torch, f_call, 5, 3))
        bm, _ = _median_min(_settled_times(torch, b_call, 5, 3))
        ff, bf = fwd_flops(M, N, K, r), bwd_flops(M, N, K, r)
        per[name] = dict(rows=N, cols=K, fwd_route=qn.route(M, N, K, r, False),
                         bwd_route=qn.route(M, N, K, r, True), fwd_ms=fm, bwd_ms=bm,
                         fwd_mfma_frac=ff / fm / 1e9 / BF16_PEAK_TFLOPS,
                         bwd_mfma_frac=bf / bm / 1e9 / BF16_PEAK_TFLOPS)
    out["decoder_layer_7_linears_M4096"] = dict(ms=med, ms_min=mn, eager_ms=eager_med,
                                                eager_ms_min=eager_mn, flops=flops,
                                                TFLOPs=flops / med / 1e9,
                                                mfma_frac=flops / med / 1e9 / BF16_PEAK_TFLOPS,
                                                adapter_params=wl.adapter_params(r=r),
                                                per_linear=per)
    del layers
    torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, target_s=15.0):
    """The oracle, untuned, on the host.  Headline: a bounded sample of the
    training workload (forward and input-gradient rows for a row sample,
    adapter gradients over a row block) as sampled FLOPs per second; a
    16-row probe sizes the sample to about target_s seconds.  Beside it, the
    other workloads' legs (each a few seconds at most): the tiny workload and
    the 4096x4096 quantize on one thread, the full quantize / dequantize /
    decode forward on every thread, and a row sample of the decoder layer."""
    import numpy as np
    import oracle
    threads = oracle.num_threads()
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
    legs = _cpu_legs(wl, oracle, np)
    return dict(value=flops / t_lin / 1e12, unit="TFLOP/s", cores=threads,
                kind="oracle", cpu_model=_cpu_model(),
                sample=(f"fp64 oracle: y and dX rows for {nr} of {M} rows, dA/dB over {mb} "
                        f"rows, at 4096x4096 r=16 ({flops / 1e9:.1f} GFLOP in {t_lin:.1f} s); "
                        f"quantize+dequantize 4096x4096 took {t_q:.2f} s"),
                seconds=t_lin, legs=legs)


def _cpu_legs(wl, oracle, np):
    """Oracle timings of the other workloads (see cpu_baseline)."""
    legs = {}
    threads = oracle.num_threads()

    def timed(f):
        t = time.perf_counter()
        out = f()
        return time.perf_counter() - t, out

    # tiny workload, one thread: quantize, dequantize, forward, backward
    oracle.set_num_threads(1)
    try:
        c = wl.TINY
        W, x, A, B, G = wl.linear_inputs(c["rows"], c["cols"], c["M"], c["r"], seed=c["seed"])
        sc = c["alpha"] / c["r"]

        def tiny():
            st = oracle.quantize(W)
            Wd, _ = oracle.dequantize(st)
            oracle.qlora_fwd(Wd, x, A, B, sc)
            oracle.qlora_dx(Wd, G, A, B, sc)
            oracle.adapter_grads(x, G, A, B, sc)
        sec, _ = timed(tiny)
        legs["tiny_1thread"] = dict(seconds=sec, threads=1)
        W2 = wl.outlier_weight()
        sec, _ = timed(lambda: oracle.quantize(W2))
        nbytes = quant_bytes(4096, 4096)
        legs["quantize_dq_4096x4096_1thread"] = dict(seconds=sec, threads=1, GBs=nbytes / sec / 1e9)
    finally:
        oracle.set_num_threads(threads)
    sec, st2 = timed(lambda: oracle.quantize(W2))
    legs["quantize_dq_4096x4096"] = dict(seconds=sec, threads=threads,
                                         GBs=quant_bytes(4096, 4096) / sec / 1e9)
    sec, _ = timed(lambda: oracle.dequantize(st2, want_f32=False))
    legs["dequant_bf16_4096x4096"] = dict(seconds=sec, threads=threads,
                                          GBs=dequant_bytes(4096, 4096, 2) / sec / 1e9)
    # decode forward 14336x4096, M = 1 and 16 (all rows)
    d = wl.DECODE
    Nd, Kd, rd = d["rows"], d["cols"], d["r"]
    Wq = wl.weight(Nd, Kd, wl.SEED_W + d["seed"])
    Wdd, _ = oracle.dequantize(oracle.quantize(Wq), want_bf16=False)
    Ad = wl.normal_bf16((rd, Kd), wl.SEED_A + d["seed"], 0.01)
    Bd = wl.normal_bf16((Nd, rd), wl.SEED_B + d["seed"], 0.01)
    for Mx in (1, 16):
        xd = wl.normal_bf16((Mx, Kd), wl.SEED_X + d["seed"], 1.0)
        sec, _ = timed(lambda: oracle.qlora_fwd(Wdd, xd, Ad, Bd, d["alpha"] / rd))
        nbytes = decode_bytes(Nd, Kd, Mx, rd)
        legs[f"decode_fwd_14336x4096_M{Mx}"] = dict(seconds=sec, threads=threads,
                                                    GBs=nbytes / sec / 1e9)
    del Wq, Wdd
    # decoder layer: every linear quantized and dequantized, y and dX for 8
    # sampled rows, dA and dB over the first 256 rows
    c5 = wl.DECODER_LAYER
    M5, r5 = c5["M"], c5["r"]
    s5 = c5["alpha"] / r5
    rows = np.linspace(0, M5 - 1, 8).astype(np.int64)
    flops, secs = 0, 0.0
    for idx, (_, N5, K5) in enumerate(wl.DECODER_LINEARS):
        W5, x5, A5, B5, G5 = wl.linear_inputs(N5, K5, M5, r5, seed=c5["seed"], index=idx)

        def layer():
            Wd5, _ = oracle.dequantize(oracle.quantize(W5), want_bf16=False)
            oracle.qlora_fwd(Wd5, x5, A5, B5, s5, rows=rows)
            oracle.qlora_dx(Wd5, G5, A5, B5, s5, rows=rows)
            oracle.adapter_grads(x5[:256], G5[:256], A5, B5, s5)
        sec, _ = timed(layer)
        secs += sec
        flops += (fwd_flops(8, N5, K5, r5) + 2 * 8 * N5 * K5 + 2 * 8 * r5 * (N5 + K5)
                  + 2 * 256 * r5 * (K5 + N5) + 2 * 256 * N5 * r5 + 2 * 256 * K5 * r5)
    legs["decoder_layer_7_linears_M4096_sample"] = dict(
        seconds=secs, threads=threads, TFLOPs=flops / secs / 1e12,
        sample="each linear: quantize + dequantize, y and dX for 8 of 4096 rows, "
               "dA and dB over 256 rows")
    return legs


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
    x1 = xdec[:1].contiguous()
    for _ in range(launches):
        qn.qlora_linear_fwd(std, x1, Ad, Bdd, alpha)
    torch.cuda.synchronize()
    print(f"[kernels] decode forward M=1 {Nd}x{Kd} x {launches}", file=sys.stderr, flush=True)
    # the decoder layer's k_proj shape (1024 x 4096, M = 4096): the forward
    # with the dequantization inside 128 x 128 GEMM tiles
    lc = wl.DECODER_LAYER
    Wk, xk, Ak, Bk, _ = wl.linear_inputs(1024, 4096, lc["M"], r, seed=lc["seed"], index=1)
    stk = qn.nf4_quantize_dq(torch.from_numpy(Wk).cuda())
    xk, Ak, Bk = _bf16(torch, xk), _bf16(torch, Ak), _bf16(torch, Bk)
    for _ in range(launches):
        qn.qlora_linear_fwd(stk, xk, Ak, Bk, alpha)
    torch.cuda.synchronize()
    print(f"[kernels] fused forward M={lc['M']} 1024x4096 ({qn.route(lc['M'], 1024, 4096, r)}) "
          f"x {launches}", file=sys.stderr, flush=True)
    Wq = torch.from_numpy(wl.weight(N, K, wl.SEED_W + 90)).cuda()
    for _ in range(launches):
        qn.nf4_quantize_dq(Wq, out=st)
    torch.cuda.synchronize()
    print(f"[kernels] quantize {N}x{K} x {launches}", file=sys.stderr, flush=True)


def layer_workload(torch, qn, wl, reps=3):
    """The decoder layer's seven linears (M = 4096, r = 16), forward then
    backward of each in turn, `reps` times after one untimed pass, with a
    synchronization and a stderr line per linear so that a kernel trace can
    be cut into linears."""
    L = qn.load_library()
    cfg = wl.DECODER_LAYER
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    layers = []
    for idx, (name, N, K) in enumerate(wl.DECODER_LINEARS):
        W, x, A, B, G = wl.linear_inputs(N, K, M, r, seed=cfg["seed"], index=idx)
        st = qn.nf4_quantize_dq(torch.from_numpy(W).cuda())
        layers.append(dict(name=name, st=st, x=_bf16(torch, x), A=_bf16(torch, A),
                           B=_bf16(torch, B), G=_bf16(torch, G),
                           fws=qn.linear_workspace(L.qlora_linear_workspace(M, N, K, r, 0)),
                           bws=qn.linear_workspace(L.qlora_linear_workspace(M, N, K, r, 1)),
                           y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
    for rep in range(reps + 1):
        for d in layers:
            _, u = qn.qlora_linear_fwd(d["st"], d["x"], d["A"], d["B"], alpha, y=d["y"],
                                       workspace=d["fws"])
            qn.qlora_linear_bwd(d["st"], d["x"], d["G"], d["A"], d["B"], alpha, u,
                                workspace=d["bws"])
            torch.cuda.synchronize()
            print(f"[layer] pass {rep} {d['name']}", file=sys.stderr, flush=True)


def adapter_workload(torch, qn, wl, reps=5):
    """The adapter rows' kernels for a kernel trace: the merge W' + s B A of a
    4096x4096 weight (r = 16) `reps` times, then the training shape's forward
    and backward (8192x4096x4096, r = 16) with dropout p = 0.05 on the
    adapter branch `reps` times, then once more without dropout; a
    synchronization and a stderr line after each call so that the trace can be
    cut into calls."""
    L = qn.load_library()
    cfg = wl.TRAIN
    N, K, M, r, alpha = cfg["rows"], cfg["cols"], cfg["M"], cfg["r"], cfg["alpha"]
    st = qn.nf4_quantize_dq(torch.from_numpy(wl.weight(N, K, wl.SEED_W)).cuda())
    Am = _bf16(torch, wl.normal_bf16((16, K), wl.SEED_A + 2, 0.01))
    Bm = _bf16(torch, wl.normal_bf16((N, 16), wl.SEED_B + 2, 0.01))
    merged = torch.empty((N, K), dtype=torch.float32, device="cuda")
    for rep in range(reps):
        qn.nf4_merge_lora(st, Am, Bm, 32.0, out=merged)
        torch.cuda.synchronize()
        print(f"[adapter] merge {rep}", file=sys.stderr, flush=True)
    xd = _bf16(torch, wl.normal_bf16((M, K), wl.SEED_X, 1.0))
    Gd = _bf16(torch, wl.normal_bf16((M, N), wl.SEED_DY, 1.0))
    Ad = _bf16(torch, wl.normal_bf16((r, K), wl.SEED_A, 0.01))
    Bd = _bf16(torch, wl.normal_bf16((N, r), wl.SEED_B, 0.01))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mask = qn.dropout_mask(M, K, 0.05, generator=torch.Generator(device="cuda").manual_seed(7))
    dws = qn.linear_workspace(max(L.qlora_linear_workspace_ex(M, N, K, r, 1, None),
                                  L.qlora_linear_workspace_ex(
                                      M, N, K, r, 1, qn.ctypes.byref(qn._LoraOpts(0, 1, 0.05)))))
    for rep in range(reps + 1):
        drop = rep < reps
        kw = dict(dropout_mask=mask, dropout_p=0.05) if drop else {}
        _, u = qn.qlora_linear_fwd(st, xd, Ad, Bd, alpha, y=y, workspace=dws, **kw)
        torch.cuda.synchronize()
        print(f"[adapter] forward {'dropout' if drop else 'plain'} {rep}", file=sys.stderr,
              flush=True)
        qn.qlora_linear_bwd(st, xd, Gd, Ad, Bd, alpha, u, workspace=dws, **kw)
        torch.cuda.synchronize()
        print(f"[adapter] backward {'dropout' if drop else 'plain'} {rep}", file=sys.stderr,
              flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kernels", action="store_true",
                    help="only the fixed kernel launches used by the rocprofv3 summaries")
    ap.add_argument("--layer", action="store_true",
                    help="only the decoder layer's seven linears, forward and backward, "
                         "three times (for a rocprofv3 kernel trace)")
    ap.add_argument("--adapter", action="store_true",
                    help="only the adapter merge and the dropout training step, five times "
                         "each (for a rocprofv3 kernel trace)")
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
    if args.layer:
        layer_workload(torch, qn, wl)
        return
    if args.adapter:
        adapter_workload(torch, qn, wl)
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
    dms = tr["fwd_bwd_dropout_ms"][0]
    extras["train_fwd_bwd_dropout_p0.05_4096x4096_M8192"] = dict(
        ms=dms, ms_min=tr["fwd_bwd_dropout_ms"][1], TFLOPs=(tr["fwd_flops"] + tr["bwd_flops"]) / dms / 1e9,
        mfma_frac=(tr["fwd_flops"] + tr["bwd_flops"]) / dms / 1e9 / BF16_PEAK_TFLOPS,
        without_dropout_ms=fwd_med + bwd_med)
    if not args.no_extras:
        print("[bench] extras", file=sys.stderr, flush=True)
        extras.update(bench_extras(torch, qn, wl))
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
                           "qlora_linear_fwd + qlora_linear_bwd, captured once in a HIP graph "
                           "and replayed once per step", "flops_per_step": tr["flops_per_step"],
                   "eager_ms_per_step": tr["eager_ms_per_step"],
                   "settle": f"{tr['settle_steps']} untimed steps ({tr['settle_s']} s before "
                             f"the eager and again before the graph-replay timing) ahead of "
                             f"the {args.warmup} warm-up steps, for sustained clocks"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
