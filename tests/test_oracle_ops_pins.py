"""Pins for the ERF, GeLU and LayerNorm oracle (oracle/repops_oracle.c).

The Verde and RepOps article (section 4.3) names LayerNorm, GeLU and ERF as
RepOps operators without giving formulas; the oracle fixes one binary32
operation sequence for each.  What pins it, independently of its own code:

* the constants: the series coefficients equal (2/sqrt pi)(-1)^n/(n!(2n+1))
  computed here from pi; the Abramowitz and Stegun 7.1.28 decimals, evaluated
  in binary64, stay within the handbook's 3e-7 bound of scipy's erf;
* the operation sequence: an exact-rational evaluation of the same steps
  (oracle/exact.py, no hardware floating point) agrees bit for bit, on random,
  tiny, huge and special inputs and on random LayerNorm rows;
* accuracy against scipy's erf and a binary64 LayerNorm, at bounds derived
  from the approximation error and the rounding;
* special cases: signed zeros, infinities, NaN, odd symmetry, constant rows,
  a two-element row with an exact answer;
* mutation controls: plausible mistakes planted in a copy of the C oracle
  fail at least one pin.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
import subprocess
import tempfile
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import exact

special = pytest.importorskip("scipy.special")

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "repops_oracle.c")
PI_50 = "3.14159265358979323846264338327950288419716939937510"


def c_table(name, src=None):
    text = open(SRC).read() if src is None else src
    m = re.search(name + r"\[\d+\]\s*=\s*\{(.*?)\};", text, re.S)
    return [v for v in re.findall(r"(-?[0-9.]+(?:e[+-]?[0-9]+)?)f", m.group(1))]


# -- a uniform view of an oracle build (the real one or a mutant) --------------
class Ops:
    def __init__(self, lib):
        fp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.repops_oracle_erf_f32.argtypes = [fp, fp, i64]
        lib.repops_oracle_gelu_f32.argtypes = [fp, fp, i64]
        lib.repops_oracle_layernorm_f32.argtypes = [fp, i64, fp, fp, fp, i64, i64, i64,
                                                    ctypes.c_float, fp, fp]
        self.lib = lib

    def _unary(self, fn, x):
        x = np.ascontiguousarray(x, np.float32)
        y = np.empty_like(x)
        assert fn(x.ctypes.data, y.ctypes.data, x.size) == 0
        return y

    def erf(self, x):
        return self._unary(self.lib.repops_oracle_erf_f32, x)

    def gelu(self, x):
        return self._unary(self.lib.repops_oracle_gelu_f32, x)

    def layernorm(self, x, gamma=None, beta=None, eps=1e-5):
        x = np.ascontiguousarray(x, np.float32)
        rows, H = x.shape
        y = np.empty_like(x)
        mean = np.empty(rows, np.float32)
        rstd = np.empty(rows, np.float32)
        g = None if gamma is None else np.ascontiguousarray(gamma, np.float32)
        b = None if beta is None else np.ascontiguousarray(beta, np.float32)
        assert self.lib.repops_oracle_layernorm_f32(
            x.ctypes.data, H, None if g is None else g.ctypes.data,
            None if b is None else b.ctypes.data, y.ctypes.data, H, rows, H,
            float(np.float32(eps)), mean.ctypes.data, rstd.ctypes.data) == 0
        return y, mean, rstd


REAL = Ops(oracle._load())


def same_bits(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return (np.array_equal(na, nb)
            and np.array_equal(np.where(na, 0, a).view(np.uint32), np.where(nb, 0, b).view(np.uint32)))


def sample_inputs(n=300, seed=3):
    rng = np.random.default_rng(seed)
    parts = [rng.standard_normal(n).astype(np.float32) * 2,
             rng.uniform(-1, 1, n // 3).astype(np.float32),
             (rng.uniform(0.5, 1.5, n // 6) * np.float32(2.0) ** rng.integers(-149, 10, n // 6)
              * rng.choice([-1, 1], n // 6)).astype(np.float32),
             np.array([0.0, -0.0, 1.0, -1.0, 0.99999994, -0.99999994, 1.0000001, 2.0, 5.6, 5.7,
                       9.0, -12.0, 1e-40, -1e-45, 3.4e38, np.inf, -np.inf, np.nan], np.float32)]
    return np.concatenate(parts)


# -- pin groups, each returning True when it holds ---------------------------
def erf_exact_pass(ops):
    x = sample_inputs(240, 3)
    return same_bits(ops.erf(x), exact.exact_unary(exact.exact_erf, x))


def gelu_exact_pass(ops):
    x = sample_inputs(200, 4)
    return same_bits(ops.gelu(x), exact.exact_unary(exact.exact_gelu, x))


def erf_accuracy_pass(ops):
    x = np.linspace(-6, 6, 400_001, dtype=np.float64).astype(np.float32)
    with np.errstate(all="ignore"):
        y = ops.erf(x).astype(np.float64)
    ref = special.erf(x.astype(np.float64))
    inner = np.abs(x) < 1
    ulp = np.spacing(np.abs(ref[inner]).astype(np.float32)).astype(np.float64)
    ok_inner = np.all(np.abs(y[inner] - ref[inner]) <= 3 * np.maximum(ulp, 2.0 ** -149))
    ok_outer = np.all(np.abs(y[~inner] - ref[~inner]) <= 5e-7)
    return bool(ok_inner and ok_outer)


def gelu_accuracy_pass(ops):
    x = np.linspace(-8, 8, 400_001, dtype=np.float64).astype(np.float32)
    with np.errstate(all="ignore"):
        y = ops.gelu(x).astype(np.float64)
    xd = x.astype(np.float64)
    ref = xd * 0.5 * (1 + special.erf(xd / math.sqrt(2)))
    return bool(np.all(np.abs(y - ref) <= 3.5e-7 * np.maximum(np.abs(xd), 1)))


def layernorm_exact_pass(ops):
    rng = np.random.default_rng(7)
    for rows, H, eps in ((3, 37, 1e-5), (2, 64, 1e-12), (4, 5, 0.5)):
        x = (rng.standard_normal((rows, H)) * rng.uniform(0.01, 100) + rng.uniform(-50, 50)
             ).astype(np.float32)
        g = rng.standard_normal(H).astype(np.float32)
        b = rng.standard_normal(H).astype(np.float32)
        for gg, bb in ((g, b), (None, None), (g, None)):
            got = ops.layernorm(x, gg, bb, eps)
            want = exact.exact_layernorm(x, gg, bb, eps)
            if not all(same_bits(u, v) for u, v in zip(got, want)):
                return False
    return True


def layernorm_accuracy_pass(ops):
    rng = np.random.default_rng(8)
    H = 768
    x = (rng.standard_normal((64, H)) * 3 + 1).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    b = (0.1 * rng.standard_normal(H)).astype(np.float32)
    for eps in (1e-12, 1e-2):
        y, mean, rstd = ops.layernorm(x, g, b, eps)
        xd = x.astype(np.float64)
        mu = xd.mean(axis=1, keepdims=True)
        var = ((xd - mu) ** 2).mean(axis=1, keepdims=True)
        ref = (xd - mu) / np.sqrt(var + np.float64(np.float32(eps))) * g + b
        if not np.all(np.abs(y - ref) <= 2e-5 * (np.abs(ref) + 1)):
            return False
        if not np.allclose(rstd, 1 / np.sqrt(var[:, 0] + np.float32(eps)), rtol=1e-5):
            return False
    return True


# -- tests on the real oracle ----------------------------------------------------
def test_series_coefficients_follow_their_definition():
    getcontext().prec = 50
    k = Decimal(2) / Decimal(PI_50).sqrt()
    got = c_table("ERF_SERIES")
    assert len(got) == 11
    for n, dec in enumerate(got):
        want = k * (-1) ** n / (Decimal(math.factorial(n)) * (2 * n + 1))
        assert abs(Decimal(dec) - want) <= abs(want) * Decimal("1e-20"), n


def test_as7128_decimals_meet_the_handbook_bound():
    a = [float(v) for v in c_table("AS_7128")]
    assert len(a) == 6
    y = np.linspace(0, 8, 800_001)
    p = np.full_like(y, a[5])
    for c in a[4::-1]:
        p = p * y + c
    p = p * y + 1
    err = np.abs(1 - 1 / p ** 16 - special.erf(y))
    assert 1e-7 < err.max() <= 3e-7


def test_erf_matches_exact_evaluation():
    assert erf_exact_pass(REAL)


def test_gelu_matches_exact_evaluation():
    assert gelu_exact_pass(REAL)


def test_erf_accuracy():
    assert erf_accuracy_pass(REAL)


def test_gelu_accuracy():
    assert gelu_accuracy_pass(REAL)


def test_erf_special_values_and_symmetry():
    y = REAL.erf(np.array([0.0, -0.0, np.inf, -np.inf, np.nan], np.float32))
    assert y[0] == 0 and not np.signbit(y[0])
    assert y[1] == 0 and np.signbit(y[1])
    assert y[2] == 1 and y[3] == -1 and np.isnan(y[4])
    x = sample_inputs(400, 9)
    x = x[~np.isnan(x)]
    assert same_bits(REAL.erf(-x), -REAL.erf(x))


def test_gelu_special_values():
    y = REAL.gelu(np.array([0.0, np.inf, -np.inf, -20.0, 20.0], np.float32))
    assert y[0] == 0 and y[1] == np.inf and np.isnan(y[2])  # -inf * (1 + -1): IEEE NaN
    assert y[3] == 0 and np.signbit(y[3])                   # erf rounds to -1: -10 * +0
    assert y[4] == 20.0


def test_layernorm_matches_exact_evaluation():
    assert layernorm_exact_pass(REAL)


def test_layernorm_accuracy_against_binary64():
    assert layernorm_accuracy_pass(REAL)


def test_layernorm_closed_forms():
    # a constant row: every deviation is 0, so y = 0 * rstd * gamma + beta = beta
    x = np.full((2, 10), 3.25, np.float32)
    g = np.linspace(-2, 2, 10).astype(np.float32)
    b = np.linspace(1, 5, 10).astype(np.float32)
    y, mean, rstd = REAL.layernorm(x, g, b, 1e-5)
    assert np.array_equal(y, np.tile(b, (2, 1))) and np.all(mean == 3.25)
    assert rstd[0] == np.float32(1) / np.sqrt(np.float32(1e-5))
    # [1, 3] with eps = 0: mean 2, deviations -1 and 1, variance 1, rstd 1
    y, mean, rstd = REAL.layernorm(np.array([[1.0, 3.0]], np.float32), None, None, 0.0)
    assert y.tolist() == [[-1.0, 1.0]] and mean[0] == 2 and rstd[0] == 1
    # integer rows: the mean is exact
    x = np.arange(24, dtype=np.float32).reshape(3, 8)
    _, mean, _ = REAL.layernorm(x)
    assert mean.tolist() == [3.5, 11.5, 19.5]


# -- mutation controls ---------------------------------------------------------------
OPS_MUTANTS = {
    "series_ascending_horner": [(
        "        float s = ERF_SERIES[10];\n        for (int n = 9; n >= 0; --n) {",
        "        float s = ERF_SERIES[0];\n        for (int n = 1; n <= 10; ++n) {")],
    "eighth_power": [("    q = q * q;\n    q = q * q;\n    q = q * q;\n    const float r",
                      "    q = q * q;\n    q = q * q;\n    const float r")],
    "switch_at_two": [("    if (y < 1.0f) {", "    if (y < 2.0f) {")],
    "gelu_fused_scale": [("    const float h = x * 0.5f;\n    const float t = 1.0f + e;\n    return h * t;",
                          "    return fmaf(x * 0.5f, e, x * 0.5f);")],
    "unbiased_variance": [("        const float var = s2 / fh;", "        const float var = s2 / (fh - 1.0f);")],
    "eps_outside_sqrt": [("        const float ve = var + eps;\n        const float sd = sqrtf(ve);",
                          "        const float sd = sqrtf(var) + eps;")],
    "mean_by_reciprocal": [("        const float mu = s / fh;", "        const float mu = s * (1.0f / fh);")],
    "one_pass_variance": [
        ("        for (int64_t i = 0; i < H; ++i) {\n            const float d = xr[i] - mu;\n"
         "            const float sq = d * d;\n            s2 = s2 + sq;\n        }\n"
         "        const float var = s2 / fh;",
         "        for (int64_t i = 0; i < H; ++i) s2 = s2 + xr[i] * xr[i];\n"
         "        const float var = s2 / fh - mu * mu;")],
}


def _mutant(name, d):
    src = open(SRC).read()
    for old, new in OPS_MUTANTS[name]:
        assert old in src, (name, old)
        src = src.replace(old, new, 1)
    path = os.path.join(d, name + ".c")
    open(path, "w").write(src)
    so = os.path.join(d, name + ".so")
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, path, *oracle.GCC_LIBS], check=True)
    return Ops(ctypes.CDLL(so))


def all_pins_pass(ops):
    return all(f(ops) for f in (erf_exact_pass, gelu_exact_pass, erf_accuracy_pass,
                                gelu_accuracy_pass, layernorm_exact_pass,
                                layernorm_accuracy_pass))


@pytest.mark.parametrize("name", sorted(OPS_MUTANTS))
def test_planted_mistake_is_caught(name):
    with tempfile.TemporaryDirectory() as d:
        assert not all_pins_pass(_mutant(name, d)), name
