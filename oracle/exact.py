"""Exact-rational brute force for the fixed-order FP32 matmul -- TEST INFRASTRUCTURE ONLY.

No hardware floating point is used for arithmetic: binary32 values are
decoded from their bits into exact rationals, every multiply and add is done
exactly with :class:`fractions.Fraction`, and each result is rounded to
binary32 by :func:`round_binary32`, a hand-written round-to-nearest-even
(ties to even) rounder with gradual underflow and overflow to infinity, as
IEEE 754-2008 section 4.3.1 and 7.4 define them.  Signed zeros follow
IEEE 754-2008 section 6.3: an exact zero sum is +0 under round-to-nearest
unless both addends are -0; a product's sign is the XOR of the operand signs.

The loop is the definition in the Verde and RepOps article (section 3.2,
item 2): a running sum from zero, one product added per k in ascending order,
with the multiply and the add rounded separately.  Intended for tiny shapes.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

QNAN_BITS = 0x7FC00000

# An exact binary32 datum: ("num", sign, magnitude) with magnitude a Fraction
# >= 0 (sign matters for zero), ("inf", sign, None) or ("nan", 0, None).


def decode_binary32(bits: int):
    sign = (bits >> 31) & 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    if e == 0xFF:
        return ("nan", 0, None) if m else ("inf", sign, None)
    if e == 0:
        mag = Fraction(m, 1 << 149)  # subnormal: m * 2^-149
    else:
        mag = Fraction((1 << 23) | m) * (Fraction(2) ** (e - 150))
    return ("num", sign, mag)


def round_binary32(sign: int, mag: Fraction) -> int:
    """Bits of the binary32 nearest to (-1)^sign * mag, ties to even."""
    if mag == 0:
        return sign << 31
    # 2^e <= mag < 2^(e+1)
    e = mag.numerator.bit_length() - mag.denominator.bit_length()
    if mag < Fraction(2) ** e:
        e -= 1
    q_exp = -149 if e < -126 else e - 23  # quantum of the binade (or subnormals)
    q = mag / (Fraction(2) ** q_exp)
    n = q.numerator // q.denominator
    rem = q - n
    half = Fraction(1, 2)
    if rem > half or (rem == half and n % 2 == 1):
        n += 1
    if n == 0:  # underflow to zero keeps the sign
        return sign << 31
    if n >= (1 << 24):  # carry into the next binade
        n >>= 1
        q_exp += 1
    if n < (1 << 23):  # only possible at q_exp == -149: subnormal
        return (sign << 31) | n
    biased = q_exp + 150
    if biased >= 0xFF:
        return (sign << 31) | 0x7F800000
    return (sign << 31) | (biased << 23) | (n - (1 << 23))


def exact_mul(x, y):
    if x[0] == "nan" or y[0] == "nan":
        return ("nan", 0, None)
    s = x[1] ^ y[1]
    if x[0] == "inf" or y[0] == "inf":
        other = y if x[0] == "inf" else x
        if other[0] == "num" and other[2] == 0:
            return ("nan", 0, None)  # inf * 0
        return ("inf", s, None)
    return decode_binary32(round_binary32(s, x[2] * y[2]))


def exact_add(x, y):
    if x[0] == "nan" or y[0] == "nan":
        return ("nan", 0, None)
    if x[0] == "inf" and y[0] == "inf":
        return ("inf", x[1], None) if x[1] == y[1] else ("nan", 0, None)
    if x[0] == "inf":
        return x
    if y[0] == "inf":
        return y
    vx = -x[2] if x[1] else x[2]
    vy = -y[2] if y[1] else y[2]
    v = vx + vy
    if v == 0:
        s = 1 if (x[1] == 1 and y[1] == 1 and x[2] == 0 and y[2] == 0) else 0
        return ("num", s, Fraction(0))
    return decode_binary32(round_binary32(1 if v < 0 else 0, abs(v)))


def encode(x) -> int:
    if x[0] == "nan":
        return QNAN_BITS
    if x[0] == "inf":
        return (x[1] << 31) | 0x7F800000
    return round_binary32(x[1], x[2])  # already representable: exact


def exact_matmul(A: np.ndarray, B: np.ndarray, trans_a: bool = False,
                 trans_b: bool = False) -> np.ndarray:
    """Fixed-order product by exact arithmetic; returns float32 (M, N)."""
    opA = np.asarray(A, dtype=np.float32)
    opB = np.asarray(B, dtype=np.float32)
    opA = opA.T if trans_a else opA
    opB = opB.T if trans_b else opB
    M, K = opA.shape
    K2, N = opB.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    abits = np.ascontiguousarray(opA).view(np.uint32)
    bbits = np.ascontiguousarray(opB).view(np.uint32)
    a = [[decode_binary32(int(abits[i, k])) for k in range(K)] for i in range(M)]
    b = [[decode_binary32(int(bbits[k, j])) for j in range(N)] for k in range(K)]
    out = np.empty((M, N), dtype=np.uint32)
    for i in range(M):
        for j in range(N):
            s = ("num", 0, Fraction(0))  # sum = +0
            for k in range(K):
                s = exact_add(s, exact_mul(a[i][k], b[k][j]))
            out[i, j] = encode(s)
    return out.view(np.float32)


def exact_neg(x):
    return x if x[0] == "nan" else (x[0], 1 - x[1], x[2])


def exact_fold_mean_sgd(G: np.ndarray, eta, theta: np.ndarray):
    """Left-fold average and SGD step by exact arithmetic (Zoo Per-LLM Chain
    Soundness, "Detailed proof: deterministic ordering"): S = left fold of the
    rows of G (k x d) in row order, gbar = RN(RN(1/k) * S),
    theta' = RN(theta - RN(eta * gbar)).  Returns (theta', gbar) float32."""
    G = np.asarray(G, dtype=np.float32)
    k, d = G.shape
    gbits = np.ascontiguousarray(G).view(np.uint32)
    tbits = np.ascontiguousarray(np.asarray(theta, dtype=np.float32)).view(np.uint32)
    ebits = int(np.array([eta], dtype=np.float32).view(np.uint32)[0])
    inv_k = decode_binary32(round_binary32(0, Fraction(1, k)))
    e = decode_binary32(ebits)
    out = np.empty(d, dtype=np.uint32)
    gbar = np.empty(d, dtype=np.uint32)
    for j in range(d):
        s = decode_binary32(int(gbits[0, j]))
        for c in range(1, k):
            s = exact_add(s, decode_binary32(int(gbits[c, j])))
        gb = exact_mul(inv_k, s)
        gbar[j] = encode(gb)
        step = exact_mul(e, gb)
        out[j] = encode(exact_add(decode_binary32(int(tbits[j])), exact_neg(step)))
    return out.view(np.float32), gbar.view(np.float32)


def exact_matmul_bias(A: np.ndarray, B: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """exact_matmul(A, B) followed by one rounded add of bias[j] per column:
    the bias enters after the whole fixed-order sum."""
    C = exact_matmul(A, B)
    cbits = C.view(np.uint32)
    bbits = np.ascontiguousarray(np.asarray(bias, dtype=np.float32)).view(np.uint32)
    out = np.empty_like(cbits)
    for i in range(C.shape[0]):
        for j in range(C.shape[1]):
            out[i, j] = encode(exact_add(decode_binary32(int(cbits[i, j])),
                                         decode_binary32(int(bbits[j]))))
    return out.view(np.float32)


# ---- ERF, GeLU and LayerNorm by exact arithmetic ---------------------------
# The same operation sequences as repops_oracle.c, each +, -, *, / and sqrt
# computed exactly and rounded once to binary32 by round_binary32.  Constants
# are the decimals of the definitions rounded exactly to binary32 here.

def exact_div(x, y):
    if x[0] == "nan" or y[0] == "nan":
        return ("nan", 0, None)
    s = x[1] ^ y[1]
    if x[0] == "inf":
        return ("nan", 0, None) if y[0] == "inf" else ("inf", s, None)
    if y[0] == "inf":
        return ("num", s, Fraction(0))
    if y[2] == 0:
        return ("nan", 0, None) if x[2] == 0 else ("inf", s, None)
    return decode_binary32(round_binary32(s, x[2] / y[2]))


def _next_up(m: Fraction) -> Fraction:
    bits = round_binary32(0, m)
    return decode_binary32(bits + 1)[2]


def _next_down(m: Fraction) -> Fraction:
    bits = round_binary32(0, m)
    return decode_binary32(bits - 1)[2]


def exact_sqrt(x):
    """Correctly rounded binary32 square root: the representable r whose
    rounding interval holds sqrt(m), found by comparing squared midpoints
    exactly (sqrt of a binary32 value is never a midpoint)."""
    if x[0] == "nan" or (x[1] == 1 and not (x[0] == "num" and x[2] == 0)):
        return ("nan", 0, None)
    if x[0] == "inf":
        return x
    m = x[2]
    if m == 0:
        return x
    # start from a binary32 near sqrt(m), then walk to the right one
    guess = Fraction(float(m) ** 0.5)
    r = decode_binary32(round_binary32(0, guess))[2]
    while True:
        lo = (_next_down(r) + r) / 2 if r > 0 else Fraction(0)
        hi = (r + _next_up(r)) / 2
        if lo * lo > m:
            r = _next_down(r)
        elif hi * hi < m:
            r = _next_up(r)
        else:
            return ("num", 0, r)


def _const(dec: str):
    v = Fraction(dec)
    return decode_binary32(round_binary32(1 if v < 0 else 0, abs(v)))


ERF_SERIES_DEC = ["1.128379167095512573896e+0", "-3.761263890318375246321e-1",
                  "1.128379167095512573896e-1", "-2.686617064513125175943e-2",
                  "5.223977625442187842112e-3", "-8.548327023450852832547e-4",
                  "1.205533298178966425103e-4", "-1.492565035840625097746e-5",
                  "1.646211436588924740161e-6", "-1.636584469123492431739e-7",
                  "1.480719281587921723955e-8"]
AS_7128_DEC = ["0.0705230784", "0.0422820123", "0.0092705272", "0.0001520143",
               "0.0002765672", "0.0000430638"]
INV_SQRT2_DEC = "0.70710678118654752440"

ONE = ("num", 0, Fraction(1))


def exact_erf(x):
    """erf in two pieces split at |x| = 1 (Maclaurin series below,
    Abramowitz and Stegun 7.1.28 at and above, and for NaN)."""
    if x[0] == "nan":
        return x
    y = ("inf", 0, None) if x[0] == "inf" else ("num", 0, x[2])
    if y[0] == "num" and y[2] < 1:
        c = [_const(d) for d in ERF_SERIES_DEC]
        w = exact_mul(x, x)
        s = c[10]
        for n in range(9, -1, -1):
            s = exact_add(exact_mul(s, w), c[n])
        return exact_mul(s, x)
    a = [_const(d) for d in AS_7128_DEC]
    p = a[5]
    for i in range(4, -1, -1):
        p = exact_add(exact_mul(p, y), a[i])
    p = exact_add(exact_mul(p, y), ONE)
    q = exact_mul(p, p)
    for _ in range(3):
        q = exact_mul(q, q)
    r = exact_div(ONE, q)
    e = exact_add(ONE, exact_neg(r))
    return e if e[0] == "nan" else (e[0], x[1], e[2])


def exact_gelu(x):
    """(x * 0.5) * (1 + erf(x * RN(1/sqrt 2)))."""
    u = exact_mul(x, _const(INV_SQRT2_DEC))
    e = exact_erf(u)
    h = exact_mul(x, ("num", 0, Fraction(1, 2)))
    t = exact_add(ONE, e)
    return exact_mul(h, t)


def exact_unary(fn, x: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    out = np.array([encode(fn(decode_binary32(int(b)))) for b in bits.reshape(-1)],
                   dtype=np.uint32)
    return out.view(np.float32).reshape(bits.shape)


def exact_layernorm(x: np.ndarray, gamma=None, beta=None, eps=1e-5):
    """Fixed-order LayerNorm of each row by exact arithmetic: S = +0 + x_0 +
    ... (ascending), mu = S / H, S2 = sum of (x_i - mu)^2 ascending from +0,
    var = S2 / H, rstd = 1 / sqrt(var + eps), y = ((x - mu) * rstd) * gamma +
    beta.  Returns (y, mean, rstd) float32."""
    X = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    rows, H = X.shape
    xb = X.view(np.uint32)
    g = None if gamma is None else [decode_binary32(int(b)) for b in
                                    np.asarray(gamma, np.float32).view(np.uint32)]
    bt = None if beta is None else [decode_binary32(int(b)) for b in
                                    np.asarray(beta, np.float32).view(np.uint32)]
    ep = decode_binary32(int(np.float32(eps).view(np.uint32)))
    fh = ("num", 0, Fraction(H))
    y = np.empty((rows, H), np.uint32)
    mean = np.empty(rows, np.uint32)
    rstd = np.empty(rows, np.uint32)
    for r in range(rows):
        v = [decode_binary32(int(b)) for b in xb[r]]
        s = ("num", 0, Fraction(0))
        for t in v:
            s = exact_add(s, t)
        mu = exact_div(s, fh)
        s2 = ("num", 0, Fraction(0))
        for t in v:
            d = exact_add(t, exact_neg(mu))
            s2 = exact_add(s2, exact_mul(d, d))
        var = exact_div(s2, fh)
        sd = exact_sqrt(exact_add(var, ep))
        rs = exact_div(ONE, sd)
        for i, t in enumerate(v):
            o = exact_mul(exact_add(t, exact_neg(mu)), rs)
            if g is not None:
                o = exact_mul(o, g[i])
            if bt is not None:
                o = exact_add(o, bt[i])
            y[r, i] = encode(o)
        mean[r] = encode(mu)
        rstd[r] = encode(rs)
    return y.view(np.float32), mean.view(np.float32), rstd.view(np.float32)
