"""Binary64 emulation of the fixed-order FP32 matmul -- TEST INFRASTRUCTURE ONLY.

Each step of the definition (Verde and RepOps article, section 3.2, item 2:
a running sum from zero, one term per k in ascending order) is done in binary64 and the
result rounded to binary32 by numpy's cast (round-to-nearest-even, gradual
underflow).  The binary64 product of two binary32 values is exact, and a
binary64 sum rounded again to binary32 equals the correctly rounded binary32
sum because 53 >= 2*24 + 2 (S. A. Figueroa, "When is double rounding
innocuous?", SIGNUM Newsletter 30(3), 1995).  So this computes the same bits
as the C oracle by a different route: vectorised over (i, j), k in an outer
Python loop.
"""
from __future__ import annotations

import numpy as np


def emulate_f64(A: np.ndarray, B: np.ndarray, trans_a: bool = False,
                trans_b: bool = False) -> np.ndarray:
    opA = np.asarray(A).T if trans_a else np.asarray(A)
    opB = np.asarray(B).T if trans_b else np.asarray(B)
    if opA.dtype != np.float32 or opB.dtype != np.float32:
        raise TypeError("operands must be float32")
    M, K = opA.shape
    K2, N = opB.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    a64 = opA.astype(np.float64)
    b64 = opB.astype(np.float64)
    s = np.zeros((M, N), dtype=np.float32)  # sum = +0
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        for k in range(K):
            p = (a64[:, k:k + 1] * b64[k:k + 1, :]).astype(np.float32)  # RN32(a*b)
            s = (s.astype(np.float64) + p.astype(np.float64)).astype(np.float32)  # RN32(s+p)
    return s
