"""Host-side checks of the benchmark's accounting (no GPU).

The timed-window logic is checked on a fake probe against the worked
example the pages give for a measurement state machine (tests/golden/
fake_meter.txt), and the adapter parameter count of the synthetic decoder
layer against the counts the pages print (tests/golden/adapter_counts.txt).
"""
import math

import pytest

import bench
import workloads as wl
from tests import _golden


class FakeProbe:
    """A clock that reads `elapsed` seconds later at end() than at begin(),
    and an allocator gauge fixed at (baseline, peak); records the order of
    the calls it sees."""

    def __init__(self, log, elapsed, baseline, peak):
        self.log, self.elapsed, self.baseline, self.peak = log, elapsed, baseline, peak

    def begin(self):
        self.log.append("begin")
        return 10.0

    def end(self):
        self.log.append("end")
        return 10.0 + self.elapsed

    def seconds(self, start, stop):
        return stop - start

    def memory(self):
        return self.baseline, self.peak


def test_window_on_the_pages_fake_meter():
    g = _golden.table("fake_meter.txt")
    tokens = [int(t) for t in g["tokens"]]
    log = []
    probe = FakeProbe(log, g["elapsed"], g["baseline_alloc"], g["peak_alloc"])
    win = bench.time_window(lambda i: log.append(("step", i)), range(len(tokens)),
                            lambda i: tokens[i], g["warmup"], probe)
    assert win.rate == g["tokens_per_second"]
    assert win.units == sum(tokens[g["warmup"]:])
    assert win.steps == len(tokens) - g["warmup"]
    assert win.peak_above_start == g["peak_above_baseline"]
    # warmup steps run before the window opens, every timed one inside it
    w = g["warmup"]
    assert log == ([("step", i) for i in range(w)] + ["begin"] +
                   [("step", i) for i in range(w, len(tokens))] + ["end"])


@pytest.mark.parametrize("untimed", [-1, 1.0, True, "2", None])
def test_window_rejects_bad_warmup(untimed):
    with pytest.raises(ValueError):
        bench.time_window(lambda i: None, range(4), lambda i: 1, untimed,
                          FakeProbe([], 1.0, 0, 0))


def test_window_needs_a_timed_step():
    for n, w in [(0, 0), (2, 2), (2, 3)]:
        with pytest.raises(ValueError):
            bench.time_window(lambda i: None, range(n), lambda i: 1, w, FakeProbe([], 1.0, 0, 0))


@pytest.mark.parametrize("elapsed", [0.0, -1.0, math.nan, math.inf])
def test_window_rejects_bad_elapsed(elapsed):
    with pytest.raises(ValueError):
        bench.time_window(lambda i: None, range(3), lambda i: 1, 1, FakeProbe([], elapsed, 0, 0))


def test_window_without_gauge():
    class Clock:
        def begin(self):
            return 1.0

        def end(self):
            return 4.0

        def seconds(self, a, b):
            return b - a
    win = bench.time_window(lambda i: None, range(5), lambda i: 2, 2, Clock())
    assert (win.seconds, win.units, win.rate, win.peak_above_start) == (3.0, 6, 2.0, None)


def test_adapter_counts_of_the_pages():
    g = _golden.table("adapter_counts.txt")
    # seven rank-16 targets per 7B-class layer, 32 layers
    assert wl.adapter_params(r=16) * g["layers_7b"] == g["adapters_7b_rank16"]
    assert wl.adapter_params(r=16) == g["adapters_7b_rank16"] // g["layers_7b"] == 1310720
    # OPT-1.3B in the course notebook: d_model 2048, q and v targets, 24 layers
    opt = [("q_proj", 2048, 2048), ("v_proj", 2048, 2048)]
    for r in (4, 16, 64):
        assert 24 * wl.adapter_params(opt, r=r) == g[f"opt_rank{r}"]


def test_flop_accounting_closed_forms():
    # training workload: 556.20 GFLOP of fwd + bwd at 4096x4096, M=8192, r=16
    M, N, K, r = 8192, 4096, 4096, 16
    total = bench.fwd_flops(M, N, K, r) + bench.bwd_flops(M, N, K, r)
    # two base products (forward, dX) of 2MNK each; three rank-r products of
    # 2Mr(N+K) each in total (u and s u B^T; v and s v A; dA and dB)
    assert total == 4 * M * N * K + 6 * M * r * (N + K)
    assert round(total / 1e9, 2) == 556.2
    # state bytes: 0.5 + 1/64 + 1/4096 B per weight plus the 4-byte offset
    assert bench.state_bytes(4096, 4096) == 4096 * 4096 // 2 + 4096 * 4096 // 64 + 4096 * 4096 // 4096 + 4
    assert bench.quant_bytes(4096, 4096) == 75763716
    assert bench.dequant_bytes(4096, 4096, 2) == 42209284
    assert bench.decode_bytes(14336, 4096, 16, 16) == 31471620
    # merge: the state, A and B (bf16, rank 16), the fp32 merged weight
    assert bench.merge_bytes(4096, 4096, 16) == bench.state_bytes(4096, 4096) + 2 * 16 * 8192 + 4 * 4096 * 4096
