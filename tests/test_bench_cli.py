"""bench.py's command line without a GPU: the workload list in --help, the
refusal of unknown workloads and of more than one GPU (all before any device
work)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from bit_reproducible_fp32_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    # A child process is started only from a process that has not touched the
    # GPU (its state must not be carried into another program).
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_initialized():
        pytest.skip("the GPU is initialised in this process")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_help_lists_every_workload():
    r = run("--help")
    assert r.returncode == 0
    text = " ".join(r.stdout.split())
    for family in (inputs.WORKLOADS, inputs.FOLD_WORKLOADS, inputs.BATCHED_WORKLOADS,
                   inputs.HASH_WORKLOADS, inputs.OPS_WORKLOADS):
        for name in family:
            assert name in text, name


def test_unknown_workload_is_refused():
    r = run("--workload", "no_such_workload")
    assert r.returncode == 2
    assert "unknown workload" in r.stderr


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""        # no JSON line

