"""Pins for the fold-average / SGD-step oracle (Zoo Per-LLM Chain Soundness,
"Detailed proof: deterministic ordering").

* hand-derived cases (tests/golden/fold_cases.txt): fold order, the reading
  of "(1/k) *" as a multiply by the rounded quotient, an unfused update,
  the fold starting from g_1, subnormals, overflow, NaN;
* an integer workload with power-of-two k and eta, where every operation is
  exact and numpy's integer arithmetic gives the answer;
* the exact-rational brute force on hypothesis-generated tiny cases;
* the canonical order: DID byte order (unsigned bytes, prefixes first),
  duplicates rejected, and the result independent of submission order;
* mutation controls: plausible mistakes planted in a copy of the C oracle
  fail at least one pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from bit_reproducible_fp32_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fold_cases.txt")


def f32(hexstr):
    return np.array([int(hexstr, 16)], dtype=np.uint32).view(np.float32)[0]


def load_cases():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, g, eta, theta, gbar, th1, why = [p.strip() for p in line.split("|", 6)]
        out.append(dict(name=name, g=[f32(x) for x in g.split()], eta=f32(eta),
                        theta=f32(theta), gbar=gbar, theta1=th1, why=why))
    return out


CASES = load_cases()


def bits(x):
    return int(np.asarray([x], dtype=np.float32).view(np.uint32)[0])


def matches(value, want):
    if want == "nan":
        return bool(np.isnan(value))
    return bits(value) == int(want, 16)


def same_bits(x, y):
    x = np.asarray(x, np.float32)
    y = np.asarray(y, np.float32)
    nx, ny = np.isnan(x), np.isnan(y)
    return (x.shape == y.shape and np.array_equal(nx, ny)
            and np.array_equal(np.where(nx, 0, x).view(np.uint32),
                               np.where(ny, 0, y).view(np.uint32)))


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_fold_c_oracle(case):
    grads = [np.array([g], np.float32) for g in case["g"]]
    with np.errstate(all="ignore"):
        th1, gbar = oracle.fold_mean_sgd_f32(grads, case["eta"], np.array([case["theta"]]))
    assert matches(gbar[0], case["gbar"]), (case["name"], hex(bits(gbar[0])), case["why"])
    assert matches(th1[0], case["theta1"]), (case["name"], hex(bits(th1[0])), case["why"])


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_fold_exact(case):
    G = np.array(case["g"], np.float32).reshape(-1, 1)
    th1, gbar = oracle.exact_fold_mean_sgd(G, case["eta"], np.array([case["theta"]], np.float32))
    assert matches(gbar[0], case["gbar"]) and matches(th1[0], case["theta1"]), case["name"]


def test_one_over_k_readings_differ_on_the_pinned_case():
    """The golden case really separates the two readings of "(1/k) *": the
    quotient-then-multiply reading gives 0x3f2aaaae, a division 0x3f2aaaad."""
    from fractions import Fraction
    S = Fraction(2) + Fraction(1, 2 ** 21)
    inv3 = Fraction(11184811, 2 ** 25)  # RN(1/3) = 0x3eaaaaab
    assert oracle.round_binary32(0, Fraction(1, 3)) == 0x3EAAAAAB
    assert oracle.round_binary32(0, inv3 * S) == 0x3F2AAAAE
    assert oracle.round_binary32(0, S / 3) == 0x3F2AAAAD


def test_integer_workload_is_exact():
    rng = np.random.Generator(np.random.PCG64(77))
    for k in (1, 2, 4, 8, 16):
        G = rng.integers(-1024, 1025, size=(k, 513)).astype(np.float32)
        theta = rng.integers(-2 ** 12, 2 ** 12, size=513).astype(np.float32)  # |result| < 2^13, step on a 2^-5 grid: exact
        eta = np.float32(0.5)
        th1, gbar = oracle.fold_mean_sgd_f32(list(G), eta, theta)
        S = G.astype(np.int64).sum(axis=0)
        assert np.array_equal(gbar.astype(np.float64), S / k)
        assert np.array_equal(th1.astype(np.float64), theta.astype(np.float64) - 0.5 * (S / k))


finite = st.integers(0, 0xFFFFFFFF).filter(lambda u: (u >> 23) & 0xFF != 0xFF)
special = st.sampled_from([0x00000000, 0x80000000, 0x3F800000, 0x00000001, 0x7F7FFFFF,
                           0x33800000, 0x3F800001, 0x7F800000, 0xFF800000, 0x1A000000])
moderate = st.integers(0x38000000, 0x48000000)
valbits = st.one_of(finite, special, moderate, moderate.map(lambda u: u | 0x80000000))


@st.composite
def fold_problem(draw):
    k = draw(st.integers(1, 6))
    d = draw(st.integers(1, 4))
    G = np.array([[draw(valbits) for _ in range(d)] for _ in range(k)], np.uint32).view(np.float32)
    theta = np.array([draw(valbits) for _ in range(d)], np.uint32).view(np.float32)
    eta = np.array([draw(st.one_of(moderate, special))], np.uint32).view(np.float32)[0]
    return G, eta, theta


@settings(max_examples=400, deadline=None, suppress_health_check=list(HealthCheck))
@given(fold_problem())
def test_c_oracle_equals_exact_rational(problem):
    G, eta, theta = problem
    with np.errstate(all="ignore"):
        th1, gbar = oracle.fold_mean_sgd_f32(list(G), eta, theta)
    th_x, gbar_x = oracle.exact_fold_mean_sgd(G, eta, theta)
    assert same_bits(gbar, gbar_x)
    assert same_bits(th1, th_x)


def test_random_against_exact_moderate_sizes():
    G = inputs.random_matrix((7, 64), 91, "normal0.02")
    theta = inputs.random_matrix((1, 64), 92)[0]
    th1, gbar = oracle.fold_mean_sgd_f32(list(G), np.float32(3e-4), theta)
    th_x, gbar_x = oracle.exact_fold_mean_sgd(G, np.float32(3e-4), theta)
    assert same_bits(gbar, gbar_x) and same_bits(th1, th_x)


# ---------------------------------------------------------------- canonical order
def test_canonical_order_is_byte_lexicographic():
    dids = [b"did:zoo:b", b"did:zoo:a", b"did:zoo:ab", b"did:zoo:", b"\x80", b"\x7f", b"did:zoo:B"]
    order = oracle.canonical_order(dids)
    ranked = [dids[i] for i in order]
    # 'd' = 0x64 < 0x7f < 0x80 (unsigned); a proper prefix first; 'B' < 'a'
    assert ranked == [b"did:zoo:", b"did:zoo:B", b"did:zoo:a", b"did:zoo:ab", b"did:zoo:b",
                      b"\x7f", b"\x80"]


def test_canonical_order_rejects_duplicates():
    with pytest.raises(ValueError):
        oracle.canonical_order([b"x", b"y", b"x"])


def test_result_is_independent_of_submission_order():
    rng = np.random.Generator(np.random.PCG64(5))
    k, d = 9, 300
    dids = [("did:zoo:%04x" % int(rng.integers(0, 65536))).encode() + bytes([i]) for i in range(k)]
    G = inputs.random_matrix((k, d), 93, "normal0.02")
    theta = inputs.random_matrix((1, d), 94)[0]
    order = oracle.canonical_order(dids)
    ref = oracle.fold_mean_sgd_f32([G[c] for c in order], np.float32(1e-3), theta)
    for seed in range(3):
        perm = np.random.Generator(np.random.PCG64(seed)).permutation(k)
        d2 = [dids[p] for p in perm]
        G2 = G[perm]
        o2 = oracle.canonical_order(d2)
        got = oracle.fold_mean_sgd_f32([G2[c] for c in o2], np.float32(1e-3), theta)
        assert same_bits(got[0], ref[0]) and same_bits(got[1], ref[1])
    # and a non-canonical order does change the bits somewhere
    bad = oracle.fold_mean_sgd_f32([G[c] for c in reversed(order)], np.float32(1e-3), theta)
    assert not same_bits(bad[1], ref[1])


# ---------------------------------------------------------------- mutation controls
SRC = os.path.join(os.path.dirname(oracle.__file__), "repops_oracle.c")
FOLD_MUTANTS = {
    "reversed_fold": [("        float s = grads[0][e];\n        for (int64_t c = 1; c < k; ++c) s = s + grads[c][e];",
                       "        float s = grads[k - 1][e];\n        for (int64_t c = k - 2; c >= 0; --c) s = s + grads[c][e];")],
    "divide_by_k": [("        const float gbar = inv_k * s;", "        const float gbar = s / (float)k;")],
    "fused_update": [("        const float step = eta * gbar;\n        theta_out[e] = theta_in[e] - step;",
                      "        theta_out[e] = fmaf(-eta, gbar, theta_in[e]);")],
    "fold_from_zero": [("        float s = grads[0][e];\n        for (int64_t c = 1; c < k; ++c)",
                        "        float s = 0.0f;\n        for (int64_t c = 0; c < k; ++c)")],
    "binary64_fold": [("        for (int64_t c = 1; c < k; ++c) s = s + grads[c][e];",
                       "        double t = s;\n        for (int64_t c = 1; c < k; ++c) t = t + grads[c][e];\n        s = (float)t;")],
}


def _fold_lib(name, d):
    src = open(SRC).read()
    for old, new in FOLD_MUTANTS[name]:
        assert old in src, (name, old)
        src = src.replace(old, new, 1)
    path = os.path.join(d, name + ".c")
    open(path, "w").write("#include <math.h>\n" + src)
    so = os.path.join(d, name + ".so")
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, path, "-lm"], check=True)
    lib = ctypes.CDLL(so)
    fp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.repops_oracle_fold_mean_sgd_f32.argtypes = [fp, i64, i64, ctypes.c_float, fp, fp, fp]
    lib.repops_oracle_fold_mean_sgd_f32.restype = ctypes.c_int
    return lib


def _fold_pins_pass(lib):
    with np.errstate(all="ignore"):
        for case in CASES:
            grads = [np.array([g], np.float32) for g in case["g"]]
            ptrs = (ctypes.c_void_p * len(grads))(*[g.ctypes.data for g in grads])
            th = np.array([case["theta"]], np.float32)
            out = np.empty(1, np.float32)
            gb = np.empty(1, np.float32)
            lib.repops_oracle_fold_mean_sgd_f32(ptrs, len(grads), 1, float(case["eta"]),
                                                th.ctypes.data, out.ctypes.data, gb.ctypes.data)
            if not (matches(gb[0], case["gbar"]) and matches(out[0], case["theta1"])):
                return False
    return True


@pytest.mark.parametrize("name", sorted(FOLD_MUTANTS))
def test_planted_fold_mistake_is_caught(name):
    with tempfile.TemporaryDirectory() as d:
        assert not _fold_pins_pass(_fold_lib(name, d)), name
