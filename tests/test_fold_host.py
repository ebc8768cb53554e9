"""Host-side checks of the fold entry points that need no GPU: the library's
canonical contributor order against the oracle's (byte-lexicographic,
duplicates rejected) and the argument validation of
repops_fold_mean_sgd_f32 (invalid calls return before any device work)."""
from __future__ import annotations

import numpy as np
import pytest

import bit_reproducible_fp32_amd as rp
import oracle


def test_canonical_order_matches_oracle_on_random_identities():
    rng = np.random.Generator(np.random.PCG64(11))
    for trial in range(200):
        k = int(rng.integers(1, 40))
        ids = set()
        while len(ids) < k:
            n = int(rng.integers(0, 6))
            # small alphabet with NUL and high bytes: many shared prefixes
            ids.add(bytes(rng.choice([0, 1, 0x7F, 0x80, 0xFF, 0x61], size=n).astype(np.uint8)))
        ids = list(ids)
        st, order = rp.repops_canonical_order(ids)
        assert st == rp.REPOPS_OK
        assert order == oracle.canonical_order(ids)


def test_canonical_order_duplicates_and_errors():
    st, _ = rp.repops_canonical_order([b"did:a", b"did:b", b"did:a"])
    assert st == rp.REPOPS_ERR_DUPLICATE
    st, _ = rp.repops_canonical_order([b"", b""])
    assert st == rp.REPOPS_ERR_DUPLICATE
    assert rp.repops_canonical_order([])[0] == rp.REPOPS_OK
    assert rp.repops_canonical_order([b"only"]) == (rp.REPOPS_OK, [0])
    with pytest.raises(rp.RepopsError):
        rp.canonical_order(["x", "x"])
    assert rp.canonical_order(["b", "a", "ab"]) == [1, 2, 0]


# Fake, never-dereferenced device addresses.
G0, G1, TH, GB = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def test_fold_validation():
    f = rp.repops_fold_mean_sgd_f32
    assert f([G0], 0, 16, 0.1, TH, None, None) == rp.REPOPS_ERR_DIM      # k < 1
    assert f([G0], 1, -1, 0.1, TH, None, None) == rp.REPOPS_ERR_DIM     # d < 0
    assert f([G0], 1, 0, 0.1, TH, None, None) == rp.REPOPS_OK           # nothing to do
    assert f([G0], 1, 16, 0.1, None, None, None) == rp.REPOPS_ERR_NULL  # no theta
    assert f([0], 1, 16, 0.1, TH, None, None) == rp.REPOPS_ERR_NULL     # NULL gradient
    assert f([G0] * 65, 65, 16, 0.1, TH, None, None) == rp.REPOPS_ERR_NULL  # needs gbar
    assert f([G0], 1, 16, 0.1, G0 + 32, None, None) == rp.REPOPS_ERR_ALIAS  # theta in grad
    assert f([G0, G1], 2, 16, 0.1, TH, G1 + 60, None) == rp.REPOPS_ERR_ALIAS  # gbar in grad
    assert f([G0], 1, 16, 0.1, TH, TH + 4, None) == rp.REPOPS_ERR_ALIAS  # gbar in theta
    # (every call above fails validation, so none of them reaches a launch)
