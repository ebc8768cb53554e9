"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for bit.

Every finite output of the fixed-order matmul has exactly one correct bit
pattern, so the bar is bitwise equality (NaNs compared as a class: their
payload is not specified).  Covered: hand-derived adversarial dot products
inside larger matrices, whole small workloads on every kernel variant, every
operand layout (transposes, padded leading dimensions, column-major views,
misaligned bases, zero strides), ragged shapes spanning several tiles with
tails in M, N and K, the empty and K = 0 cases, special values (subnormal
products, infinities, NaN), and the transformer-shaped workloads at full size
in the launch configuration the benchmark times, checked on sampled outputs
plus whole rows and columns, and across variants on every output.
"""
from __future__ import annotations

import hashlib
import sys

import numpy as np
import pytest

import oracle
from bit_reproducible_fp32_amd import inputs
from golden_cases import load_cases, matches

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_reproducible_fp32_amd as rp  # noqa: E402

DEV = "cuda:0"


def say(msg):
    print("[gpu-parity] " + msg, flush=True)
    sys.stdout.flush()


def bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def assert_same_bits(got, want, what=""):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    ng, nw = np.isnan(got), np.isnan(want)
    assert np.array_equal(ng, nw), "%s: NaN positions differ" % what
    gb = bits(np.where(ng, 0, got))
    wb = bits(np.where(nw, 0, want))
    bad = np.argwhere(gb != wb)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d outputs differ; first at %s: got %08x want %08x"
                             % (what, bad.shape[0], gb.size, i, gb[i], wb[i]))


def digest(t):
    return hashlib.sha256(t.detach().cpu().numpy().tobytes()).hexdigest()


def gpu(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def run(a, b, trans_a=False, trans_b=False, variant=None, out=None):
    c = rp.matmul(a, b, trans_a=trans_a, trans_b=trans_b, variant=variant, out=out)
    torch.cuda.synchronize()
    return c


VARIANTS = None


def variants():
    global VARIANTS
    if VARIANTS is None:
        VARIANTS = list(range(rp.repops_variant_count()))
    return VARIANTS


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    say("library: %s" % rp.repops_build_manifest())
    yield


_ORACLE_CACHE = {}


def oracle_full(name):
    if name not in _ORACLE_CACHE:
        w = inputs.WORKLOADS[name]
        A, B = inputs.make_operands(name)
        say("oracle %s (%dx%dx%d)" % (name, w.M, w.N, w.K))
        _ORACLE_CACHE[name] = (A, B, oracle.matmul_f32(A, B, w.trans_a, w.trans_b))
    return _ORACLE_CACHE[name]


# ---------------------------------------------------------------- adversarial cases
CASES = load_cases()


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_golden_dot_inside_a_matrix(case):
    """The hand-derived dot product sits at (37, 45) of a 70 x 90 product;
    every variant must give the derived bits there and the oracle's bits
    everywhere."""
    K = case.a.size
    A = inputs.random_matrix((70, K), 7001)
    B = inputs.random_matrix((K, 90), 7002)
    A[37, :] = case.a
    B[:, 45] = case.b
    with np.errstate(all="ignore"):
        want = oracle.matmul_f32(A, B)
    ga, gb = gpu(A), gpu(B)
    for v in variants():
        say("golden %s variant %s" % (case.name, rp.repops_variant_name(v)))
        c = run(ga, gb, variant=v).cpu().numpy()
        assert matches(c[37, 45], case), (case.name, rp.repops_variant_name(v), case.why)
        assert_same_bits(c, want, "%s/%s" % (case.name, rp.repops_variant_name(v)))


# ---------------------------------------------------------------- whole workloads
@pytest.mark.parametrize("name", ["square256_uniform", "square256_int", "square1024_normal"])
def test_small_workload_every_variant(name):
    A, B, want = oracle_full(name)
    ga, gb = gpu(A), gpu(B)
    if name == "square256_int":
        assert np.array_equal(want.astype(np.int64), A.astype(np.int64) @ B.astype(np.int64))
    for v in variants():
        say("%s variant %s" % (name, rp.repops_variant_name(v)))
        assert_same_bits(run(ga, gb, variant=v).cpu().numpy(), want,
                         "%s/%s" % (name, rp.repops_variant_name(v)))


def _layouts(X):
    """The same logical matrix X (float32, on the GPU) in several stored
    forms: (stored tensor, trans flag, label)."""
    M, K = X.shape
    yield X, False, "row-major"
    yield X.t().contiguous(), True, "transposed storage"
    pad = torch.zeros(M, K + 3, device=DEV)
    pad[:, :K] = X
    yield pad[:, :K], False, "padded ld (+3)"
    yield X.t().contiguous().t(), False, "column-major view"
    buf = torch.zeros(M * K + 1, device=DEV)
    buf[1:] = X.reshape(-1)
    yield buf[1:].view(M, K), False, "misaligned base"
    big = torch.zeros(2 * M, 3 * K, device=DEV)
    big[::2, ::3] = X
    yield big[::2, ::3], False, "strided both ways"


def test_layout_invariance_square1024():
    A, B, want = oracle_full("square1024_normal")
    ga, gb = gpu(A), gpu(B)
    chosen = [None] + variants()
    for sa, ta, la in _layouts(ga):
        for sb, tb, lb in _layouts(gb):
            for v in chosen:
                vn = "auto" if v is None else rp.repops_variant_name(v)
                say("square1024 A:%s B:%s variant %s" % (la, lb, vn))
                c = run(sa, sb, trans_a=ta, trans_b=tb, variant=v)
                assert_same_bits(c.cpu().numpy(), want, "A:%s B:%s %s" % (la, lb, vn))


def test_output_layouts():
    A, B, want = oracle_full("square256_uniform")
    ga, gb = gpu(A), gpu(B)
    outT = torch.empty(256, 256, device=DEV).t()          # column-major output
    outP = torch.empty(256, 300, device=DEV)[:, 7:263]     # padded, offset output
    for out, label in ((outT, "column-major"), (outP, "padded offset")):
        for v in variants():
            say("output %s variant %s" % (label, rp.repops_variant_name(v)))
            run(ga, gb, variant=v, out=out)
            assert_same_bits(out.cpu().numpy(), want, label)


def test_broadcast_zero_strides():
    a_row = inputs.random_matrix((1, 96), 7101)
    B = inputs.random_matrix((96, 80), 7102)
    A = np.repeat(a_row, 50, axis=0)
    want = oracle.matmul_f32(A, B)
    ga = gpu(a_row).expand(50, 96)  # stride (0, 1)
    assert ga.stride(0) == 0
    for v in variants():
        say("broadcast variant %s" % rp.repops_variant_name(v))
        assert_same_bits(run(ga, gpu(B), variant=v).cpu().numpy(), want, "broadcast")


RAGGED = [(1, 1, 1), (1, 7, 3), (5, 1, 9), (3, 5, 2), (17, 33, 15), (65, 63, 17),
          (129, 127, 33), (128, 128, 16), (255, 257, 31), (300, 200, 1), (64, 130, 100),
          (3, 300, 1000), (513, 67, 19), (130, 518, 47)]


@pytest.mark.parametrize("shape", RAGGED, ids=["%dx%dx%d" % s for s in RAGGED])
def test_ragged_shapes(shape):
    M, N, K = shape
    A = inputs.random_matrix((M, K), 8000 + M)
    B = inputs.random_matrix((K, N), 9000 + N, "normal0.02")
    want = oracle.matmul_f32(A, B)
    ga, gb = gpu(A), gpu(B)
    gaT, gbT = gpu(A.T), gpu(B.T)
    for v in variants():
        say("ragged %s variant %s" % (shape, rp.repops_variant_name(v)))
        assert_same_bits(run(ga, gb, variant=v).cpu().numpy(), want, "NN %s" % (shape,))
        assert_same_bits(run(gaT, gbT, True, True, variant=v).cpu().numpy(), want,
                         "TT %s" % (shape,))


def test_k_zero_and_empty():
    for v in [None] + variants():
        out = torch.full((33, 65), 7.0, device=DEV)
        a = torch.empty(33, 0, device=DEV)
        b = torch.empty(0, 65, device=DEV)
        say("K=0 variant %s" % v)
        run(a, b, variant=v, out=out)
        assert np.all(bits(out.cpu().numpy()) == 0)
    c = run(torch.empty(0, 5, device=DEV), torch.ones(5, 4, device=DEV))
    assert tuple(c.shape) == (0, 4)
    c = run(torch.ones(4, 5, device=DEV), torch.ones(5, 0, device=DEV))
    assert tuple(c.shape) == (4, 0)


def test_special_values():
    """Subnormal products, infinities and NaNs spread through a 130x70x200
    product, against the oracle (NaN as a class)."""
    rng = np.random.Generator(np.random.PCG64(4242))
    A = inputs.random_matrix((130, 200), 7201)
    B = inputs.random_matrix((200, 70), 7202)
    A[:40] *= np.float32(2.0 ** -70)   # products near 2^-140: subnormal
    B[:, :20] *= np.float32(2.0 ** -70)
    A[50, 3] = np.inf
    A[51, 5] = -np.inf
    B[7, 60] = np.nan
    B[9, 61] = 0.0
    A[52, 9] = np.inf                   # inf * 0 at (52, 61)
    A[60:64] = -A[60:64]
    idx = rng.integers(0, A.size, size=50)
    A.reshape(-1)[idx] = np.float32(-0.0)
    with np.errstate(all="ignore"):
        want = oracle.matmul_f32(A, B)
    assert np.any((bits(want) & 0x7F800000) == 0) and np.any(np.isnan(want))
    ga, gb = gpu(A), gpu(B)
    for v in variants():
        say("special values variant %s" % rp.repops_variant_name(v))
        assert_same_bits(run(ga, gb, variant=v).cpu().numpy(), want, "special")


def test_errors_surface_as_exceptions():
    a = torch.ones(16, 16, device=DEV)
    with pytest.raises(rp.RepopsError) as e:
        rp.matmul(a, a, out=a)  # output aliases an input
    assert e.value.status == rp.REPOPS_ERR_ALIAS
    with pytest.raises(ValueError):
        rp.matmul(a, torch.ones(8, 16, device=DEV))
    with pytest.raises(ValueError):
        rp.matmul(a, a, variant="no-such-variant")


# ---------------------------------------------------------------- full-size workloads
LARGE = ["llama1b_mlp_up", "llama8b_mlp_up", "llama1b_mlp_dW", "llama1b_mlp_dX"]


@pytest.mark.parametrize("name", LARGE)
def test_large_workload_sampled_against_oracle(name):
    """At full size, in the benchmark's launch configuration (automatic
    variant, row-major stored operands): 4096 random outputs, the corners,
    the last row and column, and one whole row and one whole column are
    checked against the oracle."""
    w = inputs.WORKLOADS[name]
    A, B = inputs.make_operands(name)
    ga, gb = gpu(A), gpu(B)
    say("%s auto variant %s" % (name, rp.repops_variant_name(rp.repops_pick_variant_f32(
        ga.data_ptr(), ga.stride(0), ga.stride(1), gb.data_ptr(), gb.stride(0), gb.stride(1),
        w.M, w.N, w.K, w.trans_a, w.trans_b))))
    c = run(ga, gb, w.trans_a, w.trans_b).cpu().numpy()
    ii, jj = inputs.sample_entries(w.M, w.N, 4096, 31337)
    row, col = w.M // 3, w.N - 5
    ii = np.concatenate([ii, np.full(w.N, row), np.arange(w.M)])
    jj = np.concatenate([jj, np.arange(w.N), np.full(w.M, col)])
    say("%s oracle on %d entries" % (name, ii.size))
    want = oracle.entries_f32(A, B, ii, jj, w.trans_a, w.trans_b)
    assert_same_bits(c[ii, jj], want, name)


@pytest.mark.parametrize("name", LARGE)
def test_large_workload_variants_and_layouts_agree(name):
    """Every output at full size: other variants, the naive one-lane-per-output
    kernel and a re-stored operand layout all reproduce the automatic
    variant's bytes, and repeated runs are identical."""
    w = inputs.WORKLOADS[name]
    A, B = inputs.make_operands(name)
    ga, gb = gpu(A), gpu(B)
    ref = run(ga, gb, w.trans_a, w.trans_b)
    h = digest(ref)
    for v in variants():
        say("%s variant %s" % (name, rp.repops_variant_name(v)))
        c = run(ga, gb, w.trans_a, w.trans_b, variant=v)
        assert torch.equal(c.view(torch.int32), ref.view(torch.int32)), rp.repops_variant_name(v)
    say("%s re-stored operands" % name)
    gaT = ga.t().contiguous()
    gbT = gb.t().contiguous()
    c = run(gaT, gbT, not w.trans_a, not w.trans_b)
    assert torch.equal(c.view(torch.int32), ref.view(torch.int32))
    for _ in range(2):
        assert digest(run(ga, gb, w.trans_a, w.trans_b)) == h
