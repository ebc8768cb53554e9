"""bench.py's host-side pieces without a GPU: the CPU-baseline leg on every
matmul workload (including the transposed-operand ones), the description of
each workload's data, and the table of the oracle's full-output digests."""
from __future__ import annotations

import importlib.util
import os

import numpy as np
import pytest

from bit_reproducible_fp32_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_cpu_baseline_runs_on_every_workload(bench, name):
    w = inputs.WORKLOADS[name]
    # Zero operands of the stored shapes: only the slicing and the shapes the
    # oracle sees are under test here (pages of zeros are never written).
    A = np.zeros(w.a_shape, dtype=np.float32)
    B = np.zeros(w.b_shape, dtype=np.float32)
    r = bench.cpu_baseline(A, B, w, target_s=0.0, rows=2, threads=2)
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["value"] > 0
    assert "rows 0..1 of C (all %d columns, K=%d)" % (w.N, w.K) in r["sample"]


def test_op_a_rows_are_rows_of_the_logical_operand(bench):
    w = inputs.WORKLOADS["llama1b_mlp_dW"]        # A stored K x M, trans_a
    A = np.arange(6 * 5, dtype=np.float32).reshape(6, 5)   # K=6, M=5
    rows = bench.op_a_rows(A, w, 3)
    assert rows.shape == (6, 3)                   # still stored K x rows
    assert np.array_equal(rows.T, A.T[:3])        # = the first 3 rows of op(A)


def test_cpu_threads_within_the_declared_share(bench, monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.cpu_threads() == 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.cpu_threads() == bench.affinity_cores()


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_data_text_names_each_operand_distribution(bench, name):
    w = inputs.WORKLOADS[name]
    text = bench.data_text(w)
    assert "seed %d" % w.seed_a in text and "seed %d" % w.seed_b in text
    assert bench.dist_text(w.a_dist) in text and bench.dist_text(w.b_dist) in text


def test_full_output_digests_cover_every_workload(bench):
    for name in inputs.WORKLOADS:
        g = bench.golden_output_sha(name)
        assert g is not None, name
        assert all(len(g[k]) == 64 for k in "ABC")


def test_gfx_clock_parsing(bench):
    # The shape `amd-smi metric --clock --json` prints: one entry per GPU, a
    # gfx_<n> block per XCD with the current clock under "clk".
    text = ('{"gpu_data": [{"gpu": 0, "clock": {'
            '"gfx_0": {"clk": {"value": 2343, "unit": "MHz"}, "max_clk": {"value": 2400}},'
            '"gfx_1": {"clk": {"value": 2351, "unit": "MHz"}},'
            '"mem_0": {"clk": {"value": 1300, "unit": "MHz"}}}}]}')
    assert bench.parse_gfx_clocks(text) == [2343, 2351]
    assert bench.parse_gfx_clocks("not json") is None
    assert bench.parse_gfx_clocks('{"gpu_data": []}') is None


def test_other_workloads_name_known_workloads(bench):
    """The default run's list of other operators' workloads names only
    workloads that have a bench mode of their own."""
    for name in bench.OTHER_WORKLOADS:
        assert bench.other_bench(name, inputs) is not None, name
    assert bench.other_bench("llama8b_mlp_up", inputs) is None


class _FakeEvent:
    def record(self, stream):
        pass

    def synchronize(self):
        pass


class _FakeCuda:
    Event = _FakeEvent

    @staticmethod
    def synchronize():
        pass


class _FakeTorch:
    cuda = _FakeCuda


class _FakeClocks:
    """Answers a request after `delay_polls` polls."""

    def __init__(self, delay_polls, ok=True):
        self.delay, self.ok, self.requested, self.polls = delay_polls, ok, None, 0

    def request(self):
        self.requested = self.polls
        return self.ok

    def poll(self, timeout_s=0.0):
        self.polls += 1
        if self.requested is not None and self.polls - self.requested > self.delay:
            return [2300, 2310]
        return None


def test_clock_under_load_keeps_launching_until_the_reading(bench):
    launches = []
    clocks = _FakeClocks(delay_polls=5)
    reading, n = bench.clock_under_load(_FakeTorch, None, lambda: launches.append(1), 10.0,
                                        clocks, busy_before_s=0.0)
    assert reading == [2300, 2310]
    assert n == len(launches)
    # batches of 20 ms / 10 ms per step = 2 launches, one per poll, until the
    # sixth poll answers (no busy time asked for before the request)
    assert n == 2 * 6


def test_clock_under_load_busy_before_the_request(bench):
    import time as _time
    clocks = _FakeClocks(delay_polls=0)
    t0 = _time.perf_counter()
    reading, n = bench.clock_under_load(_FakeTorch, None, lambda: None, 10.0, clocks,
                                        busy_before_s=0.05)
    assert reading is not None and _time.perf_counter() - t0 >= 0.05
    assert clocks.requested == 0      # nothing was polled before the request


def test_clock_under_load_without_a_helper(bench):
    clocks = _FakeClocks(delay_polls=0, ok=False)
    reading, n = bench.clock_under_load(_FakeTorch, None, lambda: None, 10.0, clocks,
                                        busy_before_s=0.0)
    assert reading is None and n == 0
