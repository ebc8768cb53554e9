"""Seeded synthetic inputs for the reproducible FP32 matmul workloads.

This module generates operand bytes only and holds none of the matmul's
arithmetic; the GPU path and the CPU oracle both consume what it returns.
It imports nothing else from this package.

Recipe (numpy PCG64; seeds A = 1000*c + 1, B = 1000*c + 2 for workload c):

* ``uniform``: ``(integers(0, 2**24) - 2**23) * 2**-23`` -- exact U[-1, 1) on
  the 2^-23 grid, never subnormal;
* ``int8grid``: integers uniform in {-8, ..., 8} (every product and partial
  sum up to K = 2^18 is an integer below 2^24, so the result is exact);
* ``normal(std)``: float32 ``standard_normal`` times float32 ``std``, then any
  nonzero |x| < 2^-126 replaced by copysign(2^-126, x) so no input is
  subnormal (at these sizes it never triggers);

The transformer-shaped workloads are synthetic stand-ins for the
Llama-3.1-1B and -8B MLP products that the Verde and RepOps article measures
(section 4.3): random data with the activation (std 1) and weight (std 0.02)
scales of those layers, since no weights or datasets are used here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TINY = np.float32(2.0 ** -126)


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    trans_a: bool
    trans_b: bool
    a_dist: str
    b_dist: str
    seed_a: int
    seed_b: int
    description: str

    @property
    def a_shape(self):
        """Shape of A as stored (row-major)."""
        return (self.K, self.M) if self.trans_a else (self.M, self.K)

    @property
    def b_shape(self):
        """Shape of B as stored (row-major)."""
        return (self.N, self.K) if self.trans_b else (self.K, self.N)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    w.name: w
    for w in [
        Workload("square256_uniform", 256, 256, 256, False, False, "uniform", "uniform",
                 1001, 1002, "M=N=K=256, A,B ~ U[-1,1) on the 2^-23 grid"),
        Workload("square256_int", 256, 256, 256, False, False, "int8grid", "int8grid",
                 1011, 1012, "M=N=K=256, integer entries in [-8, 8]: exact result"),
        Workload("square1024_normal", 1024, 1024, 1024, False, False, "normal1", "normal1",
                 2001, 2002, "M=N=K=1024, A,B ~ N(0,1) float32, no subnormals"),
        Workload("llama1b_mlp_up", 4096, 8192, 2048, False, False, "normal1", "normal0.02",
                 3001, 3002, "Llama-3.1-1B-shaped MLP up-projection X W: M=4096 tokens, "
                 "K=2048, N=8192; X ~ N(0,1), W ~ N(0,0.02)"),
        Workload("llama8b_mlp_up", 4096, 14336, 4096, False, False, "normal1", "normal0.02",
                 4001, 4002, "Llama-3.1-8B-shaped MLP up-projection X W: M=4096 tokens, "
                 "K=4096, N=14336; X ~ N(0,1), W ~ N(0,0.02)"),
        Workload("llama1b_mlp_dW", 2048, 8192, 4096, True, False, "normal1", "normal1",
                 5001, 5002, "Llama-3.1-1B MLP weight gradient dW = X^T dY: X stored "
                 "4096x2048 (transposed operand), dY 4096x8192; K=4096 tokens"),
        Workload("llama1b_mlp_dX", 4096, 2048, 8192, False, True, "normal1", "normal1",
                 5002, 5003, "Llama-3.1-1B MLP input gradient dX = dY W^T: dY 4096x8192, "
                 "W stored 2048x8192 (transposed operand); K=8192"),
    ]
}


def _draw(dist: str, shape, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    if dist == "uniform":
        v = rng.integers(0, 2 ** 24, size=shape, dtype=np.int64) - 2 ** 23
        return (v.astype(np.float32) * np.float32(2.0 ** -23)).astype(np.float32)
    if dist == "int8grid":
        return rng.integers(-8, 9, size=shape, dtype=np.int64).astype(np.float32)
    if dist.startswith("normal"):
        std = np.float32(float(dist[len("normal"):]))
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if std != np.float32(1.0):
            x = x * std
        tiny = (x != 0) & (np.abs(x) < TINY)
        if tiny.any():
            x[tiny] = np.copysign(TINY, x[tiny])
        return x.astype(np.float32, copy=False)
    raise ValueError("unknown distribution %r" % dist)


def make_operands(name: str):
    """(A, B) as stored, C-contiguous float32, for the named workload."""
    w = WORKLOADS[name]
    return _draw(w.a_dist, w.a_shape, w.seed_a), _draw(w.b_dist, w.b_shape, w.seed_b)


def random_matrix(shape, seed: int, dist: str = "normal1") -> np.ndarray:
    """A seeded float32 matrix of any shape with one of the distributions above."""
    return _draw(dist, shape, seed)


def sample_entries(M: int, N: int, count: int, seed: int):
    """Output coordinates to check at full size: the four corners, the last
    row and column (ragged tiles), and ``count`` uniform random (i, j)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ii = [0, 0, M - 1, M - 1]
    jj = [0, N - 1, 0, N - 1]
    edge = min(64, N)
    ii += [M - 1] * edge
    jj += list(rng.integers(0, N, size=edge))
    edge = min(64, M)
    ii += list(rng.integers(0, M, size=edge))
    jj += [N - 1] * edge
    ii += list(rng.integers(0, M, size=count))
    jj += list(rng.integers(0, N, size=count))
    return np.asarray(ii, dtype=np.int64), np.asarray(jj, dtype=np.int64)


@dataclass(frozen=True)
class FoldWorkload:
    """Fixed-order gradient average + SGD step over d parameters from k
    contributors (the chain-soundness spec's aggregation, synthetic data)."""
    name: str
    k: int
    d: int
    grad_std: str
    theta_std: str
    eta: float
    seed: int
    description: str

    @property
    def algorithmic_bytes(self) -> int:
        """k gradients and theta read, theta written (gbar not written)."""
        return 4 * self.d * (self.k + 2)


FOLD_WORKLOADS = {
    w.name: w
    for w in [
        FoldWorkload("fold_k8_d64M", 8, 1 << 26, "normal0.001", "normal0.02", 1e-3, 6001,
                     "k=8 contributors, d=2^26 parameters (67M, a 268 MB gradient each), "
                     "gradients ~ N(0, 0.001), theta ~ N(0, 0.02), eta = 1e-3"),
        FoldWorkload("fold_k3_d1M", 3, (1 << 20) + 7, "normal0.001", "normal0.02", 1e-3, 6101,
                     "k=3 (1/k inexact), d=2^20+7 (ragged tail)"),
    ]
}


def make_fold_operands(name: str):
    """(list of k gradient arrays, theta) as float32, in contributor order
    c = 0..k-1 (seeds seed+1+c for the gradients, seed for theta)."""
    w = FOLD_WORKLOADS[name]
    grads = [_draw(w.grad_std, (w.d,), w.seed + 1 + c) for c in range(w.k)]
    theta = _draw(w.theta_std, (w.d,), w.seed)
    return grads, theta


def fold_sample_indices(d: int, count: int, seed: int):
    """Parameters to check at full size: both ends, a window around every
    multiple of 4 boundary class, and count uniform random indices."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = list(range(min(d, 64))) + list(range(max(0, d - 64), d))
    idx += list(rng.integers(0, d, size=count))
    return np.unique(np.asarray(idx, dtype=np.int64))


@dataclass(frozen=True)
class BatchedWorkload:
    """A batch of independent fixed-order products (batch is a free
    dimension), as in multi-head attention."""
    name: str
    batch: int
    M: int
    N: int
    K: int
    trans_a: bool
    trans_b: bool
    a_dist: str
    b_dist: str
    seed: int
    description: str

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K


BATCHED_WORKLOADS = {
    w.name: w
    for w in [
        BatchedWorkload("llama8b_attn_scores", 32, 2048, 2048, 128, False, True, "normal1",
                        "normal1", 7001, "Llama-3.1-8B-shaped attention scores Q K^T: 32 "
                        "heads, S=2048, head dim 128; Q and K stored (32, 2048, 128)"),
        BatchedWorkload("llama8b_attn_pv", 32, 2048, 128, 2048, False, False, "normal0.02",
                        "normal1", 7101, "Llama-3.1-8B-shaped P V: 32 heads, P (2048 x 2048), "
                        "V (2048 x 128)"),
    ]
}


def make_batched_operands(name: str):
    """(A, B) as stored 3-D float32 arrays for a batched workload."""
    w = BATCHED_WORKLOADS[name]
    a_shape = (w.batch, w.K, w.M) if w.trans_a else (w.batch, w.M, w.K)
    b_shape = (w.batch, w.N, w.K) if w.trans_b else (w.batch, w.K, w.N)
    return _draw(w.a_dist, a_shape, w.seed + 1), _draw(w.b_dist, b_shape, w.seed + 2)


@dataclass(frozen=True)
class HashWorkload:
    """Hashing one operator output: the tensor hash a trainer attaches to a
    graph node and the referee recomputes in a dispute.  The hashed tensor
    is the output C of the named matmul workload."""
    name: str
    source: str
    leaf_bytes: int
    description: str


HASH_WORKLOADS = {
    w.name: w
    for w in [
        HashWorkload("merkle_llama8b_mlp_up_C", "llama8b_mlp_up", 1024,
                     "SHA-256 Merkle tree hash of the Llama-3.1-8B-shaped up-projection output "
                     "C (4096 x 14336 float32, 235 MB) in 1 KiB leaves"),
    ]
}


@dataclass(frozen=True)
class OpsWorkload:
    """An elementwise (erf, gelu) or row-wise (layernorm) operator over a
    DistilBERT-shaped activation: batch 32 x sequence 512 tokens, hidden 768,
    feed-forward 3072, LayerNorm epsilon 1e-12 (the model the Verde and RepOps
    article measures in section 4.3; synthetic data, no weights)."""
    name: str
    op: str
    rows: int
    H: int
    seed: int
    eps: float
    description: str

    @property
    def algorithmic_bytes(self) -> int:
        """x read and y written once; LayerNorm also reads gamma and beta."""
        n = self.rows * self.H
        return 8 * n + (8 * self.H if self.op == "layernorm" else 0)


OPS_WORKLOADS = {
    w.name: w
    for w in [
        OpsWorkload("distilbert_gelu", "gelu", 32 * 512, 3072, 8001, 0.0,
                    "GeLU over a DistilBERT feed-forward activation, 16384 tokens x 3072, "
                    "x ~ N(0,1)"),
        OpsWorkload("distilbert_erf", "erf", 32 * 512, 3072, 8101, 0.0,
                    "erf over 16384 x 3072 values ~ N(0, 1/2) (the GeLU argument x/sqrt 2)"),
        OpsWorkload("distilbert_layernorm", "layernorm", 32 * 512, 768, 8201, 1e-12,
                    "LayerNorm over DistilBERT hidden states, 16384 tokens x 768, x ~ N(0,1) "
                    "times 4 plus 0.5, gamma ~ 1 + N(0, 0.02), beta ~ N(0, 0.02), eps 1e-12"),
        OpsWorkload("layernorm_h4096", "layernorm", 32 * 512, 4096, 8301, 1e-5,
                    "LayerNorm over 16384 rows x 4096 (a 4096-wide hidden state, the width of "
                    "the 8B-shaped products), x ~ N(0,1) times 4 plus 0.5, gamma ~ 1 + N(0, 0.02), "
                    "beta ~ N(0, 0.02), eps 1e-5"),
    ]
}


def make_ops_operands(name: str):
    """(x, gamma, beta): x of shape (rows, H); gamma and beta (H,) for
    LayerNorm, else None."""
    w = OPS_WORKLOADS[name]
    if w.op == "erf":
        x = (_draw("normal1", (w.rows, w.H), w.seed) * np.float32(0.70710678)).astype(np.float32)
        return x, None, None
    if w.op == "gelu":
        return _draw("normal1", (w.rows, w.H), w.seed), None, None
    x = (_draw("normal1", (w.rows, w.H), w.seed) * np.float32(4) + np.float32(0.5))
    gamma = (np.float32(1) + _draw("normal0.02", (w.H,), w.seed + 1)).astype(np.float32)
    beta = _draw("normal0.02", (w.H,), w.seed + 2)
    return x.astype(np.float32), gamma, beta
