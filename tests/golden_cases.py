"""Loader for tests/golden/adversarial_dots.txt (hand-derived dot products)."""
from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "adversarial_dots.txt")


@dataclass
class DotCase:
    name: str
    a: np.ndarray  # float32 (K,)
    b: np.ndarray  # float32 (K,)
    expect_bits: int | None  # None means "any NaN"
    why: str


def _bits(tokens):
    return np.array([int(t, 16) for t in tokens], dtype=np.uint32).view(np.float32)


def load_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, a, b, c, why = [p.strip() for p in line.split("|", 4)]
            av, bv = _bits(a.split()), _bits(b.split())
            assert av.shape == bv.shape, name
            cases.append(DotCase(name, av, bv, None if c == "nan" else int(c, 16), why))
    return cases


def matches(value: np.float32, case: DotCase) -> bool:
    bits = int(np.asarray(value, dtype=np.float32).view(np.uint32))
    if case.expect_bits is None:
        return bool(np.isnan(value))
    return bits == case.expect_bits
