"""GPU: calls from several host threads at once, each thread on its own stream.

The library keeps no mutable state between calls: every call reads only its
arguments, and the tensor hash writes only the workspace it is given. So
calls from different host threads on different streams may overlap, on the
host and on the GPU.

Four threads each repeat, on their own stream:
- a ragged matmul under every kernel variant;
- the tensor hash of one of those outputs, with the thread's own workspace;
- a LayerNorm.

The threads' shapes and inputs all differ. Every result must equal the
oracle's for that thread's inputs, bit for bit."""
from __future__ import annotations

import threading

import numpy as np
import pytest

import oracle
from oracle import merkle
from bit_reproducible_fp32_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_reproducible_fp32_amd as rp  # noqa: E402

DEV = "cuda:0"
LEAF = 256
THREADS = 4
ROUNDS = 3


def say(msg):
    print("[gpu-threads] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def same_bits(got, want, what):
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, what
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    w = want.view(np.uint32) if want.dtype == np.float32 else want
    bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
    assert bad.size == 0, "%s: %d elements differ, first at %d" % (what, bad.size, bad[0])


class Job:
    def __init__(self, t, n_variants):
        M, N, K = 150 + 37 * t, 130 + 29 * t, 61 + 13 * t
        A = inputs.random_matrix((M, K), 8100 + 10 * t)
        B = inputs.random_matrix((K, N), 8101 + 10 * t, "normal0.02")
        X = inputs.random_matrix((19 + 5 * t, 500 + 211 * t), 8102 + 10 * t)
        self.want_C = oracle.matmul_f32(A, B)
        self.want_root = np.frombuffer(merkle.tensor_root(self.want_C, LEAF), np.uint8)
        self.want_y = oracle.layernorm_f32(X)[0]
        self.A = torch.from_numpy(A).to(DEV)
        self.B = torch.from_numpy(B).to(DEV)
        self.X = torch.from_numpy(X).to(DEV)
        self.C = [torch.full((M, N), float("nan"), device=DEV) for _ in range(n_variants)]
        self.y = torch.full(X.shape, float("nan"), device=DEV)
        self.root = torch.zeros(32, dtype=torch.uint8, device=DEV)
        self.ws = torch.empty(rp.repops_merkle_workspace_bytes(M * N * 4, LEAF),
                              dtype=torch.uint8, device=DEV)
        self.error = None

    def run(self):
        try:
            s = torch.cuda.Stream()
            for _ in range(ROUNDS):
                for v, out in enumerate(self.C):
                    rp.matmul(self.A, self.B, out=out, variant=v, stream=s)
                rp.merkle_root(self.C[-1], leaf_bytes=LEAF, out=self.root, workspace=self.ws,
                               stream=s)
                rp.layernorm(self.X, out=self.y, stream=s)
            s.synchronize()
        except BaseException as e:  # reported by the main thread
            self.error = e


def test_threads_on_their_own_streams():
    n_var = rp.repops_variant_count()
    jobs = [Job(t, n_var) for t in range(THREADS)]
    torch.cuda.synchronize()
    say("%d threads x %d rounds x (%d variants + hash + LayerNorm)" % (THREADS, ROUNDS, n_var))
    threads = [threading.Thread(target=j.run) for j in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=90)
        assert not th.is_alive(), "a thread did not finish"
    torch.cuda.synchronize()
    for t, j in enumerate(jobs):
        assert j.error is None, "thread %d: %r" % (t, j.error)
        for v, out in enumerate(j.C):
            same_bits(out.cpu().numpy(), j.want_C, "thread %d variant %s" % (t, rp.repops_variant_name(v)))
        same_bits(j.root.cpu().numpy(), j.want_root, "thread %d root" % t)
        same_bits(j.y.cpu().numpy(), j.want_y, "thread %d LayerNorm" % t)
