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
