"""Host checks of the ERF, GeLU and LayerNorm entry points (no GPU needed).

* the constants in the kernel source follow their definitions: the series
  coefficients (2/sqrt pi)(-1)^n/(n!(2n+1)) and 1/sqrt 2 recomputed here from
  pi and 2, the Abramowitz and Stegun 7.1.28 decimals as printed in the
  handbook (within its 3e-7 bound when evaluated in binary64);
* every argument error, returned before any device work (the pointers are
  fake and never dereferenced; every call here is invalid in one way).
"""
from __future__ import annotations

import math
import os
import re
from decimal import Decimal, getcontext

import numpy as np
import pytest

import bit_reproducible_fp32_amd as rp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "bit_reproducible_fp32_amd", "csrc", "repops_ops.hip")
PI_50 = "3.14159265358979323846264338327950288419716939937510"
PX, PY, PG, PB, PM, PR = (0x10000000, 0x20000000, 0x30000000, 0x38000000, 0x40000000,
                          0x48000000)


def source_table(name):
    text = open(SRC).read()
    m = re.search(name + r"\[\d+\]\s*=\s*\{(.*?)\};", text, re.S)
    return re.findall(r"(-?[0-9.]+(?:e[+-]?[0-9]+)?)f", m.group(1))


def test_series_coefficients_follow_their_definition():
    getcontext().prec = 50
    k = Decimal(2) / Decimal(PI_50).sqrt()
    got = source_table("kErfSeries")
    assert len(got) == 11
    for n, dec in enumerate(got):
        want = k * (-1) ** n / (Decimal(math.factorial(n)) * (2 * n + 1))
        assert abs(Decimal(dec) - want) <= abs(want) * Decimal("1e-20"), n


def test_inverse_sqrt2_constant():
    getcontext().prec = 50
    dec = re.search(r"kInvSqrt2\s*=\s*([0-9.]+)f", open(SRC).read()).group(1)
    assert abs(Decimal(dec) - 1 / Decimal(2).sqrt()) < Decimal("1e-19")
    assert np.float32(float(Decimal(dec))).view(np.uint32) == 0x3F3504F3


def test_as7128_decimals_meet_the_handbook_bound():
    special = pytest.importorskip("scipy.special")
    a = [float(v) for v in source_table("kErfAS")]
    assert len(a) == 6
    y = np.linspace(0, 8, 400_001)
    p = np.full_like(y, a[5])
    for c in a[4::-1]:
        p = p * y + c
    p = p * y + 1
    assert np.abs(1 - 1 / p ** 16 - special.erf(y)).max() <= 3e-7


def test_unary_argument_errors():
    for fn in (rp.repops_erf_f32, rp.repops_gelu_f32):
        assert fn(PX, PY, -1, 0) == rp.REPOPS_ERR_DIM
        assert fn(PX, PY, (1 << 46) + 1, 0) == rp.REPOPS_ERR_DIM
        assert fn(None, PY, 16, 0) == rp.REPOPS_ERR_NULL
        assert fn(PX, None, 16, 0) == rp.REPOPS_ERR_NULL
        assert fn(PX, PX + 4, 16, 0) == rp.REPOPS_ERR_ALIAS   # partial overlap
        assert fn(None, None, 0, 0) == rp.REPOPS_OK           # empty: nothing queued


def ln(**kw):
    args = dict(x=PX, x_rs=768, gamma=PG, beta=PB, y=PY, y_rs=768, rows=64, H=768, eps=1e-5,
                mean=PM, rstd=PR, stream=0)
    args.update(kw)
    return rp.repops_layernorm_f32(**args)


def test_layernorm_argument_errors():
    assert ln(rows=-1) == rp.REPOPS_ERR_DIM
    assert ln(H=0) == rp.REPOPS_ERR_DIM
    assert ln(H=(1 << 24) + 1, x_rs=(1 << 24) + 1, y_rs=(1 << 24) + 1) == rp.REPOPS_ERR_DIM
    assert ln(x_rs=-768) == rp.REPOPS_ERR_STRIDE
    assert ln(y_rs=767) == rp.REPOPS_ERR_STRIDE
    assert ln(rows=1 << 30, x_rs=1 << 20, y_rs=1 << 20) == rp.REPOPS_ERR_DIM
    assert ln(x=None) == rp.REPOPS_ERR_NULL
    assert ln(y=None) == rp.REPOPS_ERR_NULL
    assert ln(y=PX + 4) == rp.REPOPS_ERR_ALIAS                 # overlaps x, not in place
    assert ln(y=PX, y_rs=800) == rp.REPOPS_ERR_ALIAS           # same start, other stride
    assert ln(gamma=PY + 4 * 100) == rp.REPOPS_ERR_ALIAS
    assert ln(beta=PY) == rp.REPOPS_ERR_ALIAS
    assert ln(mean=PX + 8) == rp.REPOPS_ERR_ALIAS
    assert ln(rstd=PY + 8) == rp.REPOPS_ERR_ALIAS
    assert ln(rstd=PM + 4) == rp.REPOPS_ERR_ALIAS
    assert ln(mean=PG) == rp.REPOPS_ERR_ALIAS
    assert ln(rows=0, x=None, y=None) == rp.REPOPS_OK          # empty: nothing queued


def test_python_wrappers_refuse_cpu_tensors():
    torch = pytest.importorskip("torch")
    for fn in (rp.erf, rp.gelu, rp.layernorm):
        with pytest.raises(ValueError):
            fn(torch.zeros(4, 8))
