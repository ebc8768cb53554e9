"""Every output of every matmul workload against the oracle, at full size.

tests/golden/full_output_sha256.txt holds the SHA-256 of the CPU oracle's
whole output C for each workload (written by make_full_output_hashes.py
beside it, which calls only the oracle and the seeded generators).  Each
finite output of the fixed-order matmul has exactly one correct bit pattern
(Verde and RepOps article, section 3.2, item 2), so equal digests mean every
one of the M x N outputs equals the oracle's.

Checked here, in the launch configuration the benchmark times (row-major
operands as the workload stores them, contiguous C):
* the automatically chosen variant;
* the register-blocked VALU variant (products and sums both on the VALU);
* the operand bytes themselves, so a different generator on this host shows
  up as an input mismatch rather than a kernel one.
"""
from __future__ import annotations

import hashlib
import os
import sys

import numpy as np
import pytest

from bit_reproducible_fp32_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_reproducible_fp32_amd as rp  # noqa: E402

DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "full_output_sha256.txt")
VALU_VARIANT = "valu_t128x128x16_r8x8_xcd"


def say(msg):
    print("[gpu-full] " + msg, flush=True)
    sys.stdout.flush()


def load_golden():
    rows = {}
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        name, mnk, ha, hb, hc = [p.strip() for p in line.split("|")]
        rows[name] = (tuple(int(x) for x in mnk.split()), ha, hb, hc)
    return rows


GOLD = load_golden()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def test_golden_covers_every_workload():
    assert sorted(GOLD) == sorted(inputs.WORKLOADS)
    for name, (mnk, _, _, _) in GOLD.items():
        w = inputs.WORKLOADS[name]
        assert mnk == (w.M, w.N, w.K), name


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_full_output_matches_oracle_digest(name):
    w = inputs.WORKLOADS[name]
    (_, ha, hb, hc) = GOLD[name]
    A, B = inputs.make_operands(name)
    assert hashlib.sha256(A.tobytes()).hexdigest() == ha, "operand A bytes differ on this host"
    assert hashlib.sha256(B.tobytes()).hexdigest() == hb, "operand B bytes differ on this host"
    ga = torch.from_numpy(A).to(DEV)
    gb = torch.from_numpy(B).to(DEV)
    del A, B
    out = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    for v in (None, rp.variant_names().index(VALU_VARIANT)):
        vn = "auto" if v is None else rp.repops_variant_name(v)
        say("%s %dx%dx%d variant %s" % (name, w.M, w.N, w.K, vn))
        out.fill_(float("nan"))
        rp.matmul(ga, gb, trans_a=w.trans_a, trans_b=w.trans_b, out=out, variant=v)
        torch.cuda.synchronize()
        got = hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest()
        assert got == hc, "%s/%s: full output digest %s, oracle %s" % (name, vn, got, hc)
