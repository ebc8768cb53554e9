"""Pins for the CPU oracle: it is checked against things other than itself.

* hand-derived adversarial dot products (tests/golden/adversarial_dots.txt):
  order, fused-multiply-add, cancellation, signed-zero, subnormal, overflow,
  NaN and rounding-tie detectors;
* closed forms: K = 0 gives +0; K = 1 and K = 2 reduce to numpy's binary32
  multiply and add (a library routine);
* an integer workload whose exact result numpy's int64 matmul gives;
* an exact-rational brute force with its own rounder (no hardware FP), on
  hypothesis-generated tiny cases;
* a binary64 emulation vectorised over (i, j) (a different route to the same
  bits);
* the Higham recursive-summation error bound;
* invariants: layouts, transposes, strides, thread counts, row/column
  permutations, power-of-two scaling, negation;
* mutation controls: each plausible mistake planted in a copy of the C
  oracle is caught by at least one of the pins above.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from bit_reproducible_fp32_amd import inputs
from golden_cases import load_cases, matches

CASES = load_cases()


def bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def bits1(x) -> int:
    return int(bits(x).reshape(-1)[0])


def same_bits(x, y):
    """Bitwise equality, with all NaNs in one class."""
    x = np.asarray(x, dtype=np.float32)
    y = np.asarray(y, dtype=np.float32)
    if x.shape != y.shape:
        return False
    nx, ny = np.isnan(x), np.isnan(y)
    if not np.array_equal(nx, ny):
        return False
    return np.array_equal(bits(np.where(nx, 0, x)), bits(np.where(ny, 0, y)))


def test_environment_is_rne_without_ftz_daz():
    assert oracle.env_status() == 0


# ---------------------------------------------------------------- golden cases
@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_golden_dot_c_oracle(case):
    A = case.a.reshape(1, -1)
    B = case.b.reshape(-1, 1)
    with np.errstate(all="ignore"):
        c = oracle.matmul_f32(A, B)[0, 0]
    assert matches(c, case), "%s: got %08x (%s)" % (case.name, bits1(c), case.why)


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_golden_dot_exact_and_emulation(case):
    A = case.a.reshape(1, -1)
    B = case.b.reshape(-1, 1)
    assert matches(oracle.exact_matmul(A, B)[0, 0], case)
    with np.errstate(all="ignore"):
        assert matches(oracle.emulate_f64(A, B)[0, 0], case)


def test_golden_order_negative_control():
    """Reversing k on the order detector must change the result (1+2^-21)."""
    case = next(c for c in CASES if c.name == "order_k9")
    A = case.a[::-1].reshape(1, -1).copy()
    B = case.b[::-1].reshape(-1, 1).copy()
    c = oracle.matmul_f32(A, B)[0, 0]
    assert bits1(c) == 0x3F800004


# ---------------------------------------------------------------- closed forms
def test_k0_writes_positive_zero():
    A = np.zeros((3, 0), np.float32)
    B = np.zeros((0, 5), np.float32)
    out = np.full((3, 5), np.float32(7.0))
    oracle.matmul_f32(A, B, out=out)
    assert np.all(bits(out) == 0)


def test_empty_m_or_n():
    assert oracle.matmul_f32(np.zeros((0, 4), np.float32), np.ones((4, 3), np.float32)).shape == (0, 3)
    assert oracle.matmul_f32(np.ones((2, 4), np.float32), np.ones((4, 0), np.float32)).shape == (2, 0)


def test_k1_is_binary32_product():
    a = inputs.random_matrix((37, 1), 11)
    b = inputs.random_matrix((1, 29), 12)
    a[3, 0] = -0.0
    b[0, 4] = 0.0
    want = np.multiply(a, b, dtype=np.float32)  # numpy binary32 multiply, RNE
    want = want + np.float32(0.0)                # +0 + p turns -0 into +0
    got = oracle.matmul_f32(a, b)
    assert same_bits(got, want)
    assert not np.any(bits(got) == 0x80000000)


def test_k2_is_two_products_and_one_add():
    a = inputs.random_matrix((31, 2), 13)
    b = inputs.random_matrix((2, 23), 14)
    p0 = np.multiply(a[:, :1], b[:1, :], dtype=np.float32)
    p1 = np.multiply(a[:, 1:], b[1:, :], dtype=np.float32)
    want = np.add(np.add(np.float32(0.0), p0, dtype=np.float32), p1, dtype=np.float32)
    assert same_bits(oracle.matmul_f32(a, b), want)


def test_integer_workload_is_exact():
    A, B = inputs.make_operands("square256_int")
    got = oracle.matmul_f32(A, B)
    want = A.astype(np.int64) @ B.astype(np.int64)
    assert np.all(np.abs(want) < 2 ** 24)
    assert np.array_equal(got.astype(np.int64), want)
    assert not np.any(bits(got) == 0x80000000)


# ---------------------------------------------------------------- exact brute force
def _f32_from_bits(u):
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


SPECIAL = [0x00000000, 0x80000000, 0x3F800000, 0xBF800000, 0x00000001, 0x80000001,
           0x007FFFFF, 0x00800000, 0x1A000000, 0x1A400000, 0x9A000000, 0x1C800000,
           0x33800000, 0xB3800000, 0x4B800000, 0xCB800000, 0x7F7FFFFF, 0xFF7FFFFF,
           0x7F000000, 0x3F800001, 0x3F801000, 0x3F800800]
finite_bits = st.integers(0, 0xFFFFFFFF).filter(lambda u: (u >> 23) & 0xFF != 0xFF)
value_bits = st.one_of(st.sampled_from(SPECIAL), finite_bits,
                       st.integers(0x30000000, 0x4F000000),  # moderate magnitudes
                       st.integers(0xB0000000, 0xCF000000))


@st.composite
def small_problem(draw):
    M = draw(st.integers(1, 4))
    N = draw(st.integers(1, 4))
    K = draw(st.integers(0, 6))
    a = [draw(value_bits) for _ in range(M * K)]
    b = [draw(value_bits) for _ in range(K * N)]
    A = np.array(a, dtype=np.uint32).view(np.float32).reshape(M, K)
    B = np.array(b, dtype=np.uint32).view(np.float32).reshape(K, N)
    return A, B


@settings(max_examples=400, deadline=None, suppress_health_check=list(HealthCheck))
@given(small_problem())
def test_c_oracle_equals_exact_rational(problem):
    A, B = problem
    with np.errstate(all="ignore"):
        got = oracle.matmul_f32(A, B)
        emu = oracle.emulate_f64(A, B)
    want = oracle.exact_matmul(A, B)
    assert same_bits(got, want)
    assert same_bits(emu, want)


def test_rounder_matches_numpy_cast():
    """The hand-written rounder agrees with numpy's binary64 -> binary32 cast
    (RNE, gradual underflow, overflow to inf) on values exact in binary64."""
    from fractions import Fraction
    rng = np.random.Generator(np.random.PCG64(7))
    mant = rng.integers(1, 2 ** 52, size=3000)
    expo = rng.integers(-160, 140, size=3000)
    vals = [np.ldexp(float(m), int(e) - 52) * (1 if i % 2 else -1)
            for i, (m, e) in enumerate(zip(mant, expo))]
    ties = [np.ldexp(1.0 + 2.0 ** -24, -3), np.ldexp(1.0 + 3 * 2.0 ** -24, 5), 2.0 ** -150,
            3 * 2.0 ** -151, 2.0 ** 128 - 2.0 ** 103, 2.0 ** 128 - 2.0 ** 104]
    with np.errstate(over="ignore", under="ignore"):
        for v in vals + ties:
            want = int(np.array([v]).astype(np.float32).view(np.uint32)[0])
            got = oracle.round_binary32(1 if v < 0 else 0, abs(Fraction(v)))
            assert got == want, (v, hex(got), hex(want))


# ---------------------------------------------------------------- emulation route
@pytest.mark.parametrize("shape", [(1, 1, 1), (7, 5, 3), (33, 17, 65), (64, 48, 129)])
def test_c_oracle_equals_emulation_random(shape):
    M, N, K = shape
    A = inputs.random_matrix((M, K), 100 + M)
    B = inputs.random_matrix((K, N), 200 + N, "normal0.02")
    assert same_bits(oracle.matmul_f32(A, B), oracle.emulate_f64(A, B))


def test_c_oracle_equals_emulation_square256():
    A, B = inputs.make_operands("square256_uniform")
    assert same_bits(oracle.matmul_f32(A, B), oracle.emulate_f64(A, B))


@pytest.mark.slow
def test_c_oracle_equals_emulation_square1024():
    A, B = inputs.make_operands("square1024_normal")
    got = oracle.matmul_f32(A, B)
    assert same_bits(got, oracle.emulate_f64(A, B))


@pytest.mark.parametrize("name", ["llama1b_mlp_up", "llama8b_mlp_up", "llama1b_mlp_dW",
                                  "llama1b_mlp_dX"])
def test_c_oracle_entries_equal_emulation_on_large_workload_rows(name):
    """Sampled rows of the transformer-shaped workloads: the entries routine
    agrees with the binary64 emulation of those rows."""
    w = inputs.WORKLOADS[name]
    A, B = inputs.make_operands(name)
    rows = np.array([0, 1, w.M // 2, w.M - 1])
    cols = np.random.Generator(np.random.PCG64(5)).integers(0, w.N, size=96)
    ii = np.repeat(rows, cols.size)
    jj = np.tile(cols, rows.size)
    got = oracle.entries_f32(A, B, ii, jj, w.trans_a, w.trans_b)
    opA = A.T if w.trans_a else A
    opB = B.T if w.trans_b else B
    emu = oracle.emulate_f64(np.ascontiguousarray(opA[rows]), np.ascontiguousarray(opB[:, cols]))
    assert same_bits(got.reshape(rows.size, cols.size), emu)


# ---------------------------------------------------------------- error bound
def test_higham_error_bound():
    """|C - C_exact| <= gamma_K * sum_k |a_ik b_kj| (Higham, Accuracy and
    Stability of Numerical Algorithms, 2nd ed., section 3.1), with the exact
    value taken in binary64 and binary64's own bound as slack."""
    M, N, K = 48, 40, 4096
    A = inputs.random_matrix((M, K), 31)
    B = inputs.random_matrix((K, N), 32)
    C = oracle.matmul_f32(A, B).astype(np.float64)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    ref = A64 @ B64
    S = np.abs(A64) @ np.abs(B64)
    u32, u64 = 2.0 ** -24, 2.0 ** -53
    g32 = K * u32 / (1 - K * u32)
    g64 = K * u64 / (1 - K * u64)
    assert np.all(np.abs(C - ref) <= g32 * S + 2 * g64 * S)
    # and the bound is not vacuous: the error is of the size the bound says
    assert np.max(np.abs(C - ref) / S) > 1e-9


# ---------------------------------------------------------------- invariants
def _layouts(X):
    """The same logical matrix in several stored layouts: (stored, trans)."""
    yield X, False
    yield np.ascontiguousarray(X.T), True              # transposed storage
    pad = np.zeros((X.shape[0], X.shape[1] + 3), np.float32)
    pad[:, :X.shape[1]] = X
    yield pad[:, :X.shape[1]], False                  # padded leading dimension
    yield np.asfortranarray(X), False                  # column-major view
    big = np.zeros((X.shape[0] * 2, X.shape[1] * 3), np.float32)
    big[::2, ::3] = X
    yield big[::2, ::3], False                        # non-unit strides both ways
    yield X[::-1][::-1], False                         # negative-stride round trip


def test_layout_and_transpose_invariance():
    A = inputs.random_matrix((45, 70), 41)
    B = inputs.random_matrix((70, 38), 42)
    ref = oracle.matmul_f32(A, B)
    for sa, ta in _layouts(A):
        for sb, tb in _layouts(B):
            got = oracle.matmul_f32(sa, sb, trans_a=ta, trans_b=tb)
            assert same_bits(got, ref), (sa.strides, ta, sb.strides, tb)


def test_output_strides_and_threads_invariance():
    A = inputs.random_matrix((67, 90), 43)
    B = inputs.random_matrix((90, 51), 44)
    ref = oracle.matmul_f32(A, B, nthreads=1)
    for t in (2, 3, 8, 67, 200):
        assert same_bits(oracle.matmul_f32(A, B, nthreads=t), ref)
    outF = np.asfortranarray(np.empty((67, 51), np.float32))
    oracle.matmul_f32(A, B, out=outF)
    assert same_bits(outF, ref)


def test_row_and_column_permutation_equivariance():
    A = inputs.random_matrix((40, 64), 45)
    B = inputs.random_matrix((64, 36), 46)
    ref = oracle.matmul_f32(A, B)
    rng = np.random.Generator(np.random.PCG64(47))
    pr, pc = rng.permutation(40), rng.permutation(36)
    assert same_bits(oracle.matmul_f32(A[pr], B[:, pc]), ref[pr][:, pc])


def test_power_of_two_scaling_and_negation():
    A = inputs.random_matrix((30, 80), 48)
    B = inputs.random_matrix((80, 28), 49)
    ref = oracle.matmul_f32(A, B)
    for e in (-5, 3, 11):
        got = oracle.matmul_f32((A * np.float32(2.0 ** e)).astype(np.float32), B)
        assert same_bits(got, (ref * np.float32(2.0 ** e)).astype(np.float32))
    neg = oracle.matmul_f32(-A, B)
    nz = ref != 0
    assert same_bits(neg[nz], -ref[nz])
    assert np.all(bits(neg[~nz]) == 0)


def test_k_permutation_changes_order_sensitive_results():
    """Negative control: the definition is order-sensitive, so permuting k
    changes the output of the order and cancellation detectors."""
    for name in ("order_k9", "cancel_order"):
        case = next(c for c in CASES if c.name == name)
        perm = np.arange(case.a.size)[::-1]
        c = oracle.matmul_f32(case.a[perm].reshape(1, -1).copy(),
                              case.b[perm].reshape(-1, 1).copy())[0, 0]
        assert not matches(c, case)


# ---------------------------------------------------------------- mutation controls
SRC = os.path.join(os.path.dirname(oracle.__file__), "repops_oracle.c")

MUTANTS = {
    "fused_multiply_add": [("        const float prod = x[k * xs] * y[k * ys]; /* RN(x_k * y_k) */\n"
                            "        s = s + prod;                             /* RN(s_k + prod) */",
                            "        s = fmaf(x[k * xs], y[k * ys], s);")],
    "reversed_k": [("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = K - 1; k >= 0; --k) {")],
    "first_product_init": [
        ("    float s = 0.0f;\n", "    float s = K > 0 ? x[0] * y[0] : 0.0f;\n"),
        ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 1; k < K; ++k) {")],
    "binary64_accumulate": [("        s = s + prod;                             /* RN(s_k + prod) */",
                             "        s = (float)((double)s + (double)x[k * xs] * (double)y[k * ys]);")],
    "split_k": [("    float s = 0.0f;\n", "    float s = 0.0f, half = 0.0f;\n"),
                ("        const float prod = x[k * xs]",
                 "        if (k == K / 2) { half = s; s = 0.0f; }\n        const float prod = x[k * xs]"),
                ("    return s;\n}", "    return half + s;\n}")],
    # (the planted flush-to-zero mode is undone on return, so it does not leak
    # into later oracle calls on the same thread)
    "flush_to_zero": [("    float s = 0.0f;\n",
                       "    const unsigned csr0 = _mm_getcsr();\n"
                       "    _mm_setcsr(csr0 | 0x8040u);\n    float s = 0.0f;\n"),
                      ("    return s;\n}", "    _mm_setcsr(csr0);\n    return s;\n}")],
    "transposed_a_index": [("    *step = t->a_cs; return t->A + i * t->a_rs;",
                            "    *step = t->a_rs; return t->A + i * t->a_cs;")],
    "dropped_last_k": [("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k + 1 < K; ++k) {")],
    "wrong_b_index": [("    *step = t->b_rs; return t->B + j * t->b_cs;",
                       "    *step = t->b_cs; return t->B + j * t->b_rs;")],
}


def _build_mutant(name, tmpdir):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, (name, old)
        src = src.replace(old, new, 1)
    src = "#include <math.h>\n" + src
    path = os.path.join(tmpdir, name + ".c")
    with open(path, "w") as f:
        f.write(src)
    so = os.path.join(tmpdir, name + ".so")
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, path, "-lm"], check=True)
    lib = ctypes.CDLL(so)
    i64, fp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.repops_oracle_matmul_f32.argtypes = [fp, i64, i64, fp, i64, i64, fp, i64, i64,
                                            i64, i64, i64, ip, ip, ip]
    lib.repops_oracle_matmul_f32.restype = ip
    return lib


def _mutant_matmul(lib, A, B):
    M, K = A.shape
    N = B.shape[1]
    out = np.empty((M, N), np.float32)
    rc = lib.repops_oracle_matmul_f32(A.ctypes.data, A.strides[0] // 4, A.strides[1] // 4,
                                      B.ctypes.data, B.strides[0] // 4, B.strides[1] // 4,
                                      out.ctypes.data, N, 1, M, N, K, 0, 0, 1)
    return out if rc == 0 else None


def _pins_pass(lib):
    """True when the mutant passes every pin that does not need the real oracle."""
    with np.errstate(all="ignore"):
        for case in CASES:
            c = _mutant_matmul(lib, case.a.reshape(1, -1).copy(), case.b.reshape(-1, 1).copy())
            if c is None or not matches(c[0, 0], case):
                return False
        A = inputs.random_matrix((6, 9), 61)
        B = inputs.random_matrix((9, 6), 62)
        got = _mutant_matmul(lib, A, B)
        if got is None or not same_bits(got, oracle.exact_matmul(A, B)):
            return False
        Ai, Bi = inputs.random_matrix((8, 8), 63, "int8grid"), inputs.random_matrix((8, 8), 64, "int8grid")
        got = _mutant_matmul(lib, Ai, Bi)
        if got is None or not np.array_equal(got.astype(np.int64), Ai.astype(np.int64) @ Bi.astype(np.int64)):
            return False
    return True


def test_unmutated_copy_passes_the_mutation_harness():
    with tempfile.TemporaryDirectory() as d:
        src = open(SRC).read()
        path = os.path.join(d, "same.c")
        with open(path, "w") as f:
            f.write(src)
        so = os.path.join(d, "same.so")
        subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, path], check=True)
        lib = ctypes.CDLL(so)
        i64, fp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.repops_oracle_matmul_f32.argtypes = [fp, i64, i64, fp, i64, i64, fp, i64, i64,
                                                i64, i64, i64, ip, ip, ip]
        lib.repops_oracle_matmul_f32.restype = ip
        assert _pins_pass(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    with tempfile.TemporaryDirectory() as d:
        lib = _build_mutant(name, d)
        assert not _pins_pass(lib), "mutant %s slipped through the pins" % name


def test_oracle_source_has_no_fused_or_reassociating_constructs():
    src = open(SRC).read()
    assert re.search(r"\bfmaf?\s*\(", src) is None
    assert "STDC FP_CONTRACT OFF" in src
    assert "-ffp-contract=off" in oracle.GCC_FLAGS and "-fno-fast-math" in oracle.GCC_FLAGS
