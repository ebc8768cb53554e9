"""GPU parity of the batched product with a bias epilogue
(repops_matmul_batched_f32 through the C ABI) against the CPU oracle, bit for
bit: every variant, head-interleaved and transposed attention-style layouts,
batch strides that break 16-byte alignment, shared and per-batch bias, -0
bias, K = 0 with bias, and more batches than one launch takes."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bit_reproducible_fp32_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_reproducible_fp32_amd as rp  # noqa: E402

DEV = "cuda:0"


def say(msg):
    print("[gpu-batched] " + msg, flush=True)


def same_bits(x, y, what=""):
    x = np.asarray(x, np.float32)
    y = np.asarray(y, np.float32)
    assert x.shape == y.shape, what
    nx, ny = np.isnan(x), np.isnan(y)
    assert np.array_equal(nx, ny), what
    xb = np.where(nx, 0, x).view(np.uint32)
    yb = np.where(ny, 0, y).view(np.uint32)
    bad = np.argwhere(xb != yb)
    assert bad.size == 0, "%s: %d differ, first %s: %08x vs %08x" % (
        what, bad.shape[0], tuple(bad[0]), xb[tuple(bad[0])], yb[tuple(bad[0])])


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def g(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def run(a, b, **kw):
    c = rp.matmul_batched(a, b, **kw)
    torch.cuda.synchronize()
    return c.cpu().numpy()


@pytest.mark.parametrize("M", [70, 300])
def test_every_variant_with_and_without_bias(M):
    """M = 70: only edge tiles for 128- and 256-row tiles; M = 300: whole
    tiles inside M and a ragged last tile, for every tile shape."""
    Bn, N, K = 3, 90, 37
    A = inputs.random_matrix((Bn * M, K), 401).reshape(Bn, M, K)
    B = inputs.random_matrix((Bn * K, N), 402, "normal0.02").reshape(Bn, K, N)
    bias = inputs.random_matrix((Bn, N), 403)
    bias[0, 5] = -0.0
    want_b = oracle.matmul_batched_f32(A, B, bias=bias)
    want_n = oracle.matmul_batched_f32(A, B)
    ga, gb, gbias = g(A), g(B), g(bias)
    for v in range(rp.repops_variant_count()):
        say("variant %s" % rp.repops_variant_name(v))
        same_bits(run(ga, gb, bias=gbias, variant=v), want_b, "bias v%d" % v)
        same_bits(run(ga, gb, variant=v), want_n, "no bias v%d" % v)


def test_attention_layouts():
    """Q K^T per head from head-interleaved [S, H*D] storage, and P V."""
    H, S, D = 8, 130, 64
    Qf = inputs.random_matrix((S, H * D), 411)
    Kf = inputs.random_matrix((S, H * D), 412)
    Vf = inputs.random_matrix((S, H * D), 413)
    Q = Qf.reshape(S, H, D).transpose(1, 0, 2)        # (H, S, D) view, strides (D, H*D, 1)
    Kt = Kf.reshape(S, H, D).transpose(1, 0, 2)       # K as (H, S, D): B stored N x K
    want = oracle.matmul_batched_f32(Q, Kt, trans_b=True)
    gQ = g(Qf).view(S, H, D).permute(1, 0, 2)
    gK = g(Kf).view(S, H, D).permute(1, 0, 2)
    for v in (None, 0, 3, 9, 13):
        say("QK^T variant %s" % v)
        same_bits(run(gQ, gK, trans_b=True, variant=v), want, "QK^T")
    P = inputs.random_matrix((H * S, S), 414, "normal0.02").reshape(H, S, S)
    V = Vf.reshape(S, H, D).transpose(1, 0, 2)        # (H, S, D)
    want = oracle.matmul_batched_f32(P, V)
    gV = g(Vf).view(S, H, D).permute(1, 0, 2)
    for v in (None, 1, 13):
        say("PV variant %s" % v)
        same_bits(run(g(P), gV, variant=v), want, "PV")


def test_misaligned_batch_strides_and_shared_bias():
    """Batch stride M*K+1 (not a multiple of 4): later batches start at
    unaligned addresses, so the operand takes the element-wise loader."""
    Bn, M, N, K = 5, 33, 47, 28
    A = inputs.random_matrix((Bn * M, K), 421).reshape(Bn, M, K)
    B = inputs.random_matrix((Bn * K, N), 422).reshape(Bn, K, N)
    bias = inputs.random_matrix((1, N), 423)[0]
    want = oracle.matmul_batched_f32(A, B, bias=bias)
    store = torch.zeros(Bn * (M * K + 1), device=DEV)
    va = torch.as_strided(store, (Bn, M, K), (M * K + 1, K, 1))
    va.copy_(g(A))
    for v in (None, 1, 13):
        same_bits(run(va, g(B), bias=g(bias), variant=v), want, "misaligned batches v%s" % v)


def test_k_zero_with_bias_and_negative_zero():
    Bn, M, N = 2, 5, 7
    bias = inputs.random_matrix((Bn, N), 431)
    bias[1, 3] = -0.0
    bias[0, 2] = np.inf
    out = run(torch.empty(Bn, M, 0, device=DEV), torch.empty(Bn, 0, N, device=DEV),
              bias=g(bias))
    want = np.broadcast_to((np.float32(0.0) + bias)[:, None, :], (Bn, M, N))
    same_bits(out, want, "K=0")
    assert not np.any(out.view(np.uint32) == 0x80000000)


def test_more_batches_than_one_launch():
    Bn, M, N, K = 70000, 2, 3, 5
    A = inputs.random_matrix((Bn * M, K), 441).reshape(Bn, M, K)
    B = inputs.random_matrix((Bn * K, N), 442).reshape(Bn, K, N)
    bias = inputs.random_matrix((Bn, N), 443)
    want = oracle.matmul_batched_f32(A, B, bias=bias)
    same_bits(run(g(A), g(B), bias=g(bias)), want, "70000 batches")


def test_full_size_attention_scores_sampled():
    """Llama-3.1-8B-shaped attention scores: 32 heads, S=2048, D=128, in the
    benchmark's configuration; sampled outputs of every head against the
    oracle's entries routine on that head."""
    w = inputs.BATCHED_WORKLOADS["llama8b_attn_scores"]
    A, B = inputs.make_batched_operands(w.name)
    out = run(g(A), g(B), trans_a=w.trans_a, trans_b=w.trans_b)
    for h in range(0, w.batch, 7):
        ii, jj = inputs.sample_entries(w.M, w.N, 256, 900 + h)
        want = oracle.entries_f32(A[h], B[h], ii, jj, w.trans_a, w.trans_b)
        same_bits(out[h][ii, jj], want, "head %d" % h)
