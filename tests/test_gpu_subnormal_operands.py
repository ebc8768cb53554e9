"""GPU parity with subnormal operands, on every kernel variant.

IEEE-754 binary32 with gradual underflow is the arithmetic the RepOps article
requires (Verde and RepOps article, section 3.3, the IEEE-754 compliance
limitation), and the matmul's definition (section 3.2, item 2) has exactly one
correct bit pattern per finite output.  An input below 2^-126 must therefore
enter every multiply as its true value: a kernel, or a multiplier, that
treats denormal inputs as zero changes the result.

The product kernels form their products on the matrix core
(v_mfma_f32_32x32x1_2b_f32 and 16x16x1_4b with a zero addend, one product per
output), so these sweeps are also the committed check that the matrix core
keeps denormal inputs and rounds each product exactly as a binary32 multiply
does (an exact -0 product may come back as +0, which the +0 start of the sum
absorbs).

* K = 1: C(i, j) = RN(+0 + RN(a_i * b_j)) over a 2560 x 2560 grid of operands
  that step through every exponent field (0 = zero and subnormal, 255 = inf and
  NaN), with fractions 0, 1, 2^22, 2^23-1 and a random one, and both signs.
* K = 2: RN(RN(a0 b0) + RN(a1 b1)) over random bit patterns whose exponent
  fields are uniform over 0..254, so products and sums land in every binade,
  including the subnormal range, the underflow ties and overflow.
* A random 200 x 150 x 300 product whose first 40 rows of A and first 20
  columns of B are scaled into the subnormal range.

Bar: bitwise equality with the oracle (NaNs as a class).
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


def say(msg):
    print("[gpu-subnormal] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def assert_same_bits(got, want, what):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape
    ng, nw = np.isnan(got), np.isnan(want)
    assert np.array_equal(ng, nw), "%s: NaN positions differ" % what
    gb = np.where(ng, 0, got).view(np.uint32)
    wb = np.where(nw, 0, want).view(np.uint32)
    bad = np.argwhere(gb != wb)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d outputs differ; first at %s: got %08x want %08x"
                             % (what, bad.shape[0], gb.size, i, gb[i], wb[i]))


def exponent_sweep(seed):
    """2560 binary32 values: every exponent field 0..255 with fractions
    0, 1, 2^22, 2^23 - 1 and one random fraction, both signs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    vals = []
    for e in range(256):
        for f in (0, 1, 1 << 22, (1 << 23) - 1, int(rng.integers(1, 1 << 23))):
            for s in (0, 1):
                vals.append((s << 31) | (e << 23) | f)
    return np.asarray(vals, dtype=np.uint32).view(np.float32)


def random_patterns(shape, seed):
    """Random sign, exponent field uniform in 0..254 (finite only) and random
    fraction."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = rng.integers(0, 2, size=shape, dtype=np.uint32)
    e = rng.integers(0, 255, size=shape, dtype=np.uint32)
    f = rng.integers(0, 1 << 23, size=shape, dtype=np.uint32)
    return ((s << 31) | (e << 23) | f).astype(np.uint32).view(np.float32)


def every_variant():
    return [None] + list(range(rp.repops_variant_count()))


def vname(v):
    return "auto" if v is None else rp.repops_variant_name(v)


def test_k1_exponent_sweep_every_variant():
    a = exponent_sweep(9101).reshape(-1, 1)          # A: 2560 x 1
    b = exponent_sweep(9102).reshape(1, -1)          # B: 1 x 2560
    with np.errstate(all="ignore"):
        want = oracle.matmul_f32(a, b)
    n_sub = int(np.count_nonzero((a.view(np.uint32) & 0x7f800000) == 0))
    say("K=1 sweep: %d x %d products, %d subnormal-or-zero operands per side"
        % (a.shape[0], b.shape[1], n_sub))
    ga = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    gb = torch.from_numpy(np.ascontiguousarray(b)).to(DEV)
    for v in every_variant():
        say("K=1 sweep variant %s" % vname(v))
        c = rp.matmul(ga, gb, variant=v)
        torch.cuda.synchronize()
        assert_same_bits(c.cpu().numpy(), want, "K=1 sweep/%s" % vname(v))
    # The sweep has teeth: many outputs whose A operand is a nonzero
    # subnormal are nonzero finite values, which a denormal-input flush would
    # have turned into +0.
    au = a.view(np.uint32)[:, 0]
    sub_rows = ((au & 0x7f800000) == 0) & ((au & 0x7fffff) != 0)
    w = want[sub_rows]
    assert np.count_nonzero(np.isfinite(w) & (w != 0)) > 10000


def test_k1_sweep_transposed_operands():
    """The same products with both operands stored transposed (the gather and
    along-x loaders feed the multiplier instead of the along-k ones)."""
    a = exponent_sweep(9103).reshape(-1, 1)
    b = exponent_sweep(9104).reshape(1, -1)
    with np.errstate(all="ignore"):
        want = oracle.matmul_f32(a, b)
    ga = torch.from_numpy(np.ascontiguousarray(a.T)).to(DEV)   # stored 1 x M
    gb = torch.from_numpy(np.ascontiguousarray(b.T)).to(DEV)   # stored N x 1
    for v in every_variant():
        say("K=1 transposed sweep variant %s" % vname(v))
        c = rp.matmul(ga, gb, trans_a=True, trans_b=True, variant=v)
        torch.cuda.synchronize()
        assert_same_bits(c.cpu().numpy(), want, "K=1 transposed/%s" % vname(v))


def test_k2_random_patterns_every_variant():
    a = random_patterns((1031, 2), 9201)
    b = random_patterns((2, 1029), 9202)
    with np.errstate(all="ignore"):
        want = oracle.matmul_f32(a, b)
    sub_out = int(np.count_nonzero(((want.view(np.uint32) & 0x7f800000) == 0)
                                   & ((want.view(np.uint32) & 0x7fffff) != 0)))
    say("K=2 random patterns: %d subnormal outputs of %d" % (sub_out, want.size))
    assert sub_out > 1000
    ga = torch.from_numpy(a).to(DEV)
    gb = torch.from_numpy(b).to(DEV)
    for v in every_variant():
        say("K=2 random patterns variant %s" % vname(v))
        c = rp.matmul(ga, gb, variant=v)
        torch.cuda.synchronize()
        assert_same_bits(c.cpu().numpy(), want, "K=2/%s" % vname(v))


def test_subnormal_rows_and_columns_every_variant():
    M, N, K = 200, 150, 300
    A = inputs.random_matrix((M, K), 9301)
    B = inputs.random_matrix((K, N), 9302)
    scale = np.float32(2.0 ** -130)
    A[:40] *= scale                      # rows 0..39 of A: subnormal inputs
    B[:, :20] *= scale                   # columns 0..19 of B: subnormal inputs
    A[40:44, :5] = np.float32(2.0 ** -149)   # the smallest subnormal
    assert np.count_nonzero((A.view(np.uint32) & 0x7f800000) == 0) > 40 * K // 2
    with np.errstate(all="ignore"):
        want = oracle.matmul_f32(A, B)
    assert np.count_nonzero(want[:40, 20:]) > 0
    ga = torch.from_numpy(A).to(DEV)
    gb = torch.from_numpy(B).to(DEV)
    for v in every_variant():
        say("subnormal rows/columns variant %s" % vname(v))
        c = rp.matmul(ga, gb, variant=v)
        torch.cuda.synchronize()
        assert_same_bits(c.cpu().numpy(), want, "subnormal rows/%s" % vname(v))
