"""GPU parity of the automatic kernel choice: one product for each kernel the
choice can land on, each run through the automatic path and compared with the
oracle on every output.  The chosen variant is read back through
repops_pick_variant_f32 with the arguments of the call, so a policy change
that moves one of these shapes to another kernel fails here by name instead
of leaving that kernel untested through the automatic path.
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

# (M, N, K, trans_a, trans_b, expected automatic choice)
CASES = [
    (200, 300, 100, False, False, "srow_t4x64x32_r1c1_w4_row"),     # under 2^17 outputs
    (768, 512, 128, False, True, "srow_t16x64x32_r4c1_w4_xcd"),     # 384 tiles of 16x64
    (1024, 1024, 256, True, False, "srow_t32x128x32_r4c2_w8_xcd"),  # 256 tiles of 32x128
    (2048, 1024, 256, False, False, "mprod16_t128x64x32_w8_xcd"),   # 256 tiles of 128x64
    (4096, 2048, 64, False, True, "mprod1_t128x128x32_w8_xcd"),     # 512 tiles of 128x128
]


def bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


@pytest.mark.parametrize("case", CASES, ids=[c[5] for c in CASES])
def test_automatic_choice_matches_the_oracle(case):
    M, N, K, ta, tb, expected = case
    print("[auto-choice] %dx%dx%d trans %s/%s, expecting %s" % (M, N, K, ta, tb, expected),
          flush=True)
    sys.stdout.flush()
    seed = M * 31 + N * 7 + K
    A = inputs.random_matrix((K, M) if ta else (M, K), seed, "normal1")
    B = inputs.random_matrix((N, K) if tb else (K, N), seed + 1, "normal1")
    ga = torch.from_numpy(A).to(DEV)
    gb = torch.from_numpy(B).to(DEV)
    # the stored operands' strides as the call passes them
    a_rs, a_cs = ga.stride()
    b_rs, b_cs = gb.stride()
    chosen = rp.variant_names()[rp.repops_pick_variant_f32(
        ga.data_ptr(), a_rs, a_cs, gb.data_ptr(), b_rs, b_cs, M, N, K, int(ta), int(tb))]
    assert chosen == expected
    out = rp.matmul(ga, gb, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    want = oracle.matmul_f32(A, B, ta, tb)
    bad = np.argwhere(bits(out.cpu().numpy()) != bits(want))
    assert bad.size == 0, "%s: %d outputs differ, first at %s" % (expected, bad.shape[0],
                                                               tuple(bad[0]))
