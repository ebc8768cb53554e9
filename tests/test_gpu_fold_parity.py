"""GPU parity of the fixed-order gradient average and SGD step
(repops_fold_mean_sgd_f32 through the C ABI) against the CPU oracle, bit for
bit (NaN as a class).  Covered: the hand-derived cases, random contributor
counts 1..130 (single and multi-pass folds), ragged lengths (vector and
scalar paths), misaligned pointers, with and without the gbar output,
canonical DID order through the wrapper, special values, and the full-size
workload in the benchmark's configuration on sampled parameters."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

import oracle
from bit_reproducible_fp32_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_reproducible_fp32_amd as rp  # noqa: E402

DEV = "cuda:0"
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from test_oracle_fold_pins import CASES, matches  # noqa: E402


def say(msg):
    print("[gpu-fold] " + msg, flush=True)


def same_bits(x, y, what=""):
    x = np.asarray(x, np.float32)
    y = np.asarray(y, np.float32)
    assert x.shape == y.shape, what
    nx, ny = np.isnan(x), np.isnan(y)
    assert np.array_equal(nx, ny), "%s: NaN positions differ" % what
    xb = np.where(nx, 0, x).view(np.uint32)
    yb = np.where(ny, 0, y).view(np.uint32)
    bad = np.flatnonzero(xb != yb)
    assert bad.size == 0, "%s: %d differ, first at %d: %08x vs %08x" % (
        what, bad.size, bad[0], xb[bad[0]], yb[bad[0]])


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def gpu_fold(grads, theta, eta, with_gbar=True, offset=0):
    """Run the library on copies of grads/theta placed `offset` floats into
    fresh buffers (offset 1 gives 4-byte-aligned, not 16-byte-aligned data)."""
    d = theta.size

    def place(x):
        buf = torch.zeros(d + offset, device=DEV)
        buf[offset:] = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        return buf[offset:]

    gg = [place(g) for g in grads]
    th = place(theta)
    gb = place(np.zeros(d, np.float32)) if with_gbar else None
    out = rp.fold_mean_sgd(gg, th, eta, gbar=gb)
    torch.cuda.synchronize()
    return th.cpu().numpy(), (out.cpu().numpy() if out is not None else None)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_cases(case):
    k = len(case["g"])
    rng = np.random.Generator(np.random.PCG64(3))
    for d, pos in ((1, 0), (37, 17), (64, 63)):
        grads = [rng.standard_normal(d).astype(np.float32) for _ in range(k)]
        theta = rng.standard_normal(d).astype(np.float32)
        for c in range(k):
            grads[c][pos] = case["g"][c]
        theta[pos] = case["theta"]
        with np.errstate(all="ignore"):
            want = oracle.fold_mean_sgd_f32(grads, case["eta"], theta)
        for offset in (0, 1):
            say("golden %s d=%d offset=%d" % (case["name"], d, offset))
            th, gb = gpu_fold(grads, theta, case["eta"], offset=offset)
            assert matches(gb[pos], case["gbar"]) and matches(th[pos], case["theta1"]), case["name"]
            same_bits(th, want[0], case["name"])
            same_bits(gb, want[1], case["name"])


SHAPES = [(1, 1), (2, 5), (3, 4), (3, 1023), (7, 4099), (8, 65536 + 3), (64, 1000),
          (65, 777), (130, 4096 + 1), (5, 1 << 20)]


@pytest.mark.parametrize("k,d", SHAPES, ids=["k%d_d%d" % s for s in SHAPES])
def test_random_shapes(k, d):
    grads = [inputs.random_matrix((1, d), 500 + c, "normal0.001")[0] for c in range(k)]
    theta = inputs.random_matrix((1, d), 499, "normal0.02")[0]
    eta = np.float32(3e-4)
    want = oracle.fold_mean_sgd_f32(grads, eta, theta)
    for offset in (0, 1):
        for with_gbar in ((True,) if k > rp.REPOPS_FOLD_MAX_PER_PASS else (True, False)):
            say("k=%d d=%d offset=%d gbar=%s" % (k, d, offset, with_gbar))
            th, gb = gpu_fold(grads, theta, eta, with_gbar=with_gbar, offset=offset)
            same_bits(th, want[0], "theta k=%d d=%d" % (k, d))
            if with_gbar:
                same_bits(gb, want[1], "gbar k=%d d=%d" % (k, d))


def test_special_values():
    rng = np.random.Generator(np.random.PCG64(8))
    k, d = 5, 3001
    grads = [inputs.random_matrix((1, d), 700 + c)[0] for c in range(k)]
    for g in grads:
        g[rng.integers(0, d, 40)] = np.float32(-0.0)
        g[rng.integers(0, d, 5)] = np.inf
        g[rng.integers(0, d, 5)] = -np.inf
        g[rng.integers(0, d, 3)] = np.nan
        g[rng.integers(0, d, 50)] *= np.float32(2.0 ** -130)   # subnormal
        g[rng.integers(0, d, 20)] = np.float32(3.4e38)        # overflow in the fold
    theta = inputs.random_matrix((1, d), 699)[0]
    with np.errstate(all="ignore"):
        want = oracle.fold_mean_sgd_f32(grads, np.float32(0.25), theta)
    for offset in (0, 1):
        th, gb = gpu_fold(grads, theta, np.float32(0.25), offset=offset)
        same_bits(th, want[0], "special theta")
        same_bits(gb, want[1], "special gbar")


def test_canonical_order_through_the_wrapper():
    k, d = 11, 2049
    rng = np.random.Generator(np.random.PCG64(9))
    dids = ["did:zoo:%06x" % int(x) for x in rng.permutation(1 << 20)[:k]]
    grads = [inputs.random_matrix((1, d), 800 + c, "normal0.001")[0] for c in range(k)]
    theta = inputs.random_matrix((1, d), 799, "normal0.02")[0]
    order = oracle.canonical_order([x.encode() for x in dids])
    want = oracle.fold_mean_sgd_f32([grads[c] for c in order], np.float32(1e-3), theta)
    gg = [torch.from_numpy(g).to(DEV) for g in grads]
    th = torch.from_numpy(theta).to(DEV)
    gb = rp.fold_mean_sgd(gg, th, np.float32(1e-3), dids=dids, gbar=torch.empty_like(th))
    torch.cuda.synchronize()
    same_bits(th.cpu().numpy(), want[0], "canonical theta")
    same_bits(gb.cpu().numpy(), want[1], "canonical gbar")


def test_errors_surface():
    a = torch.zeros(16, device=DEV)
    with pytest.raises(rp.RepopsError) as e:
        rp.fold_mean_sgd([a], a, 0.1)  # theta is the gradient
    assert e.value.status == rp.REPOPS_ERR_ALIAS
    with pytest.raises(rp.RepopsError) as e:
        rp.fold_mean_sgd([a, torch.zeros(16, device=DEV)], torch.zeros(16, device=DEV), 0.1,
                         dids=["x", "x"])
    assert e.value.status == rp.REPOPS_ERR_DUPLICATE


@pytest.mark.parametrize("name", sorted(inputs.FOLD_WORKLOADS))
def test_full_size_workload_sampled(name):
    """The benchmark's configuration (16-byte-aligned tensors, no gbar
    output) at full size; every sampled parameter checked against the oracle
    run on the same gathered elements (parameters are independent)."""
    w = inputs.FOLD_WORKLOADS[name]
    grads, theta = inputs.make_fold_operands(name)
    idx = inputs.fold_sample_indices(w.d, 20000, 4243)
    want = oracle.fold_mean_sgd_f32([g[idx] for g in grads], np.float32(w.eta), theta[idx])
    say("%s: k=%d d=%d" % (name, w.k, w.d))
    gg = [torch.from_numpy(g).to(DEV) for g in grads]
    th = torch.from_numpy(theta).to(DEV)
    rp.fold_mean_sgd(gg, th, np.float32(w.eta))
    torch.cuda.synchronize()
    same_bits(th.cpu().numpy()[idx], want[0], name)
    # once more with the gbar output: the same theta bits from the same start
    th2 = torch.from_numpy(theta).to(DEV)
    gb = rp.fold_mean_sgd(gg, th2, np.float32(w.eta), gbar=torch.empty_like(th2))
    torch.cuda.synchronize()
    assert torch.equal(th.view(torch.int32), th2.view(torch.int32))
    same_bits(gb.cpu().numpy()[idx], want[1], name + " gbar")
