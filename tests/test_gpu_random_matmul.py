"""GPU parity on seeded random configurations of the fixed-order matmul.

Each case draws sizes (a quarter of them 1 to 16, the rest log-uniform from
16 to about 700, so most span several tiles with ragged tails), a value distribution per operand, a
storage for each operand and for C (contiguous, transposed, padded leading
dimension, column-major view, misaligned base, every other element), and a
kernel variant (or the automatic choice), then compares every output with
the CPU oracle bit for bit.  A second set does the same for the batched entry
point with a random batch stride layout and an optional bias.  The cases are
reproducible from their index; a failure names the case and its draw.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from bit_reproducible_fp32_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_reproducible_fp32_amd as rp  # noqa: E402

DEV = "cuda:0"
N_CASES = 64
N_BATCHED = 16
DISTS = ("normal1", "normal0.02", "uniform", "int8grid")
STORAGES = ("contiguous", "padded", "colmajor", "offset", "every_other")


def say(msg):
    print("[gpu-random] " + msg, flush=True)
    sys.stdout.flush()


def bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def stored_on_gpu(x, storage, rng):
    """The 2-D array x (values as stored) placed on the GPU in one of several
    layouts; the returned tensor holds exactly x's values."""
    r, c = x.shape
    if storage == "contiguous":
        return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if storage == "padded":
        pad = int(rng.integers(1, 9))
        big = torch.full((r, c + pad), float("nan"), device=DEV)
        big[:, :c] = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        return big[:, :c]
    if storage == "colmajor":
        return torch.from_numpy(np.ascontiguousarray(x.T)).to(DEV).t()
    if storage == "offset":
        off = int(rng.integers(1, 4))       # a base that is not 16-byte aligned
        flat = torch.full((off + r * c,), float("nan"), device=DEV)
        flat[off:] = torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).to(DEV)
        return flat[off:].view(r, c)
    # every other element along both dimensions
    big = torch.full((2 * r, 2 * c), float("nan"), device=DEV)
    big[::2, ::2] = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return big[::2, ::2]


def out_on_gpu(M, N, storage, rng):
    if storage in ("contiguous", "offset", "every_other"):
        return torch.full((M, N), 7.0, device=DEV)
    if storage == "padded":
        return torch.full((M, N + int(rng.integers(1, 9))), 7.0, device=DEV)[:, :N]
    return torch.full((N, M), 7.0, device=DEV).t()


def draw_case(idx):
    rng = np.random.Generator(np.random.PCG64(20261202 + idx))

    def size(hi):
        # a quarter tiny (1..16), the rest log-uniform over 16..hi
        if rng.uniform() < 0.25:
            return int(rng.integers(1, 17))
        return int(np.exp(rng.uniform(np.log(16), np.log(hi))))

    M, N, K = size(700), size(700), size(900)
    ta, tb = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    da, db = DISTS[int(rng.integers(0, len(DISTS)))], DISTS[int(rng.integers(0, len(DISTS)))]
    sa, sb = STORAGES[int(rng.integers(0, 5))], STORAGES[int(rng.integers(0, 5))]
    sc = STORAGES[int(rng.integers(0, 3))]
    nvar = rp.repops_variant_count()
    v = int(rng.integers(-1, nvar))        # -1: the automatic choice
    return rng, dict(M=M, N=N, K=K, trans_a=ta, trans_b=tb, dist_a=da, dist_b=db,
                     store_a=sa, store_b=sb, store_c=sc, variant=v)


@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_matmul(idx):
    rng, d = draw_case(idx)
    M, N, K = d["M"], d["N"], d["K"]
    a_shape = (K, M) if d["trans_a"] else (M, K)
    b_shape = (N, K) if d["trans_b"] else (K, N)
    A = inputs.random_matrix(a_shape, 31000 + idx, d["dist_a"])
    B = inputs.random_matrix(b_shape, 32000 + idx, d["dist_b"])
    vname = "auto" if d["variant"] < 0 else rp.repops_variant_name(d["variant"])
    say("case %d: %s variant %s" % (idx, d, vname))
    want = oracle.matmul_f32(A, B, d["trans_a"], d["trans_b"])
    ga = stored_on_gpu(A, d["store_a"], rng)
    gb = stored_on_gpu(B, d["store_b"], rng)
    out = out_on_gpu(M, N, d["store_c"], rng)
    rp.matmul(ga, gb, trans_a=d["trans_a"], trans_b=d["trans_b"], out=out,
              variant=None if d["variant"] < 0 else d["variant"])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = np.argwhere(bits(got) != bits(want))
    assert bad.size == 0, "case %d %s: %d outputs differ, first at %s" % (
        idx, d, bad.shape[0], tuple(bad[0]))


@pytest.mark.parametrize("idx", range(N_BATCHED))
def test_random_batched(idx):
    rng, d = draw_case(1000 + idx)
    M, N, K = min(d["M"], 300), min(d["N"], 300), min(d["K"], 300)
    batch = int(rng.integers(1, 6))
    a_shape = (batch, K, M) if d["trans_a"] else (batch, M, K)
    b_shape = (batch, N, K) if d["trans_b"] else (batch, K, N)
    A = inputs.random_matrix(a_shape, 33000 + idx, d["dist_a"])
    B = inputs.random_matrix(b_shape, 34000 + idx, d["dist_b"])
    bias = inputs.random_matrix((N,), 35000 + idx) if rng.integers(0, 2) else None
    vname = "auto" if d["variant"] < 0 else rp.repops_variant_name(d["variant"])
    say("batched case %d: batch %d %dx%dx%d trans %s/%s bias %s variant %s"
        % (idx, batch, M, N, K, d["trans_a"], d["trans_b"], bias is not None, vname))
    want = oracle.matmul_batched_f32(A, B, d["trans_a"], d["trans_b"], bias)
    # A with heads interleaved (batch as the middle dimension of the storage)
    ga = torch.from_numpy(np.ascontiguousarray(A.transpose(1, 0, 2))).to(DEV).transpose(0, 1)
    gb = torch.from_numpy(np.ascontiguousarray(B)).to(DEV)
    gbias = torch.from_numpy(bias).to(DEV) if bias is not None else None
    out = rp.matmul_batched(ga, gb, trans_a=d["trans_a"], trans_b=d["trans_b"], bias=gbias,
                            variant=None if d["variant"] < 0 else d["variant"])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = np.argwhere(bits(got) != bits(want))
    assert bad.size == 0, "batched case %d: %d outputs differ, first at %s" % (
        idx, bad.shape[0], tuple(bad[0]))
