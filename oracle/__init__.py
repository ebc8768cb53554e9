"""CPU oracle for the reproducible FP32 matmul -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The GPU library never imports, links or
calls it, and it imports nothing from the GPU library: the two share no code.

Three independent implementations of one definition (Verde and RepOps
article, section 3.2 "RepOps design principles", item 2, the matrix
multiplication example): C(i, j) is the inner product of row i of op(A) and
column j of op(B), accumulated term by term in one fixed k order from a
running sum that starts at zero.  Read as: ascending k, the running sum
starting at +0.0, each multiply and each add rounded on its own to binary32
round-to-nearest-even (the Zoo chain-soundness spec pins RNE and turns fused
multiply-add off), gradual underflow:

* :func:`matmul_f32` / :func:`entries_f32` -- the plain C triple loop in
  ``repops_oracle.c`` (the oracle proper), built with gcc;
* :func:`emulate_f64` -- the same steps in numpy binary64, each result
  rounded to binary32 (double rounding is innocuous for +, x because
  53 >= 2*24 + 2; S. A. Figueroa, "When is double rounding innocuous?",
  1995), vectorised over (i, j);
* :func:`exact_matmul` -- exact rational arithmetic with a hand-written
  binary32 round-to-nearest-even rounder; no hardware floating point.

The submodule :mod:`oracle.merkle` holds the tensor hash (SHA-256 in an
RFC 6962 Merkle tree) and the referee's re-execution of a disputed matmul.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .emulate import emulate_f64  # noqa: F401
from .exact import (exact_fold_mean_sgd, exact_matmul, exact_matmul_bias,  # noqa: F401
                    round_binary32)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "repops_oracle.c")
_LIB = os.path.join(_HERE, "librepops_oracle.so")

GCC_FLAGS = [
    "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
    "-fexcess-precision=standard", "-fPIC", "-shared", "-pthread",
]
GCC_LIBS = ["-lm"]

_lib = None


def build(force: bool = True) -> str:
    """Compile ``repops_oracle.c`` into ``librepops_oracle.so`` with gcc."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, *GCC_LIBS], check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, fp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.repops_oracle_matmul_f32.argtypes = [
            fp, i64, i64, fp, i64, i64, fp, i64, i64, i64, i64, i64, ip, ip, ip]
        lib.repops_oracle_matmul_f32.restype = ip
        lib.repops_oracle_entries_f32.argtypes = [
            fp, i64, i64, fp, i64, i64, i64, i64, i64, ip, ip, fp, fp, i64, fp, ip]
        lib.repops_oracle_entries_f32.restype = ip
        lib.repops_oracle_fold_mean_sgd_f32.argtypes = [fp, i64, i64, ctypes.c_float, fp, fp, fp]
        lib.repops_oracle_fold_mean_sgd_f32.restype = ip
        lib.repops_oracle_matmul_batched_f32.argtypes = [
            fp, i64, i64, i64, fp, i64, i64, i64, fp, i64, i64, i64, i64, i64, i64, i64,
            ip, ip, fp, i64, i64, ip]
        lib.repops_oracle_matmul_batched_f32.restype = ip
        lib.repops_oracle_erf_f32.argtypes = [fp, fp, i64]
        lib.repops_oracle_erf_f32.restype = ip
        lib.repops_oracle_gelu_f32.argtypes = [fp, fp, i64]
        lib.repops_oracle_gelu_f32.restype = ip
        lib.repops_oracle_layernorm_f32.argtypes = [fp, i64, fp, fp, fp, i64, i64, i64,
                                                    ctypes.c_float, fp, fp]
        lib.repops_oracle_layernorm_f32.restype = ip
        lib.repops_oracle_env_status.argtypes = []
        lib.repops_oracle_env_status.restype = ip
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def env_status() -> int:
    """0 when the host FP environment is RNE without FTZ/DAZ."""
    return _load().repops_oracle_env_status()


def _operand(x: np.ndarray):
    """Base pointer and element strides of a float32 array view."""
    if x.dtype != np.float32:
        raise TypeError("oracle operands must be float32")
    if x.ndim != 2:
        raise ValueError("oracle operands must be 2-D")
    rs, cs = (s // 4 for s in x.strides)
    if any(s % 4 for s in x.strides):
        raise ValueError("strides must be whole elements")
    return x.ctypes.data, rs, cs


def _logical_shapes(A, B, trans_a, trans_b):
    M, K = (A.shape[1], A.shape[0]) if trans_a else A.shape
    K2, N = (B.shape[1], B.shape[0]) if trans_b else B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    return M, N, K


def matmul_f32(A: np.ndarray, B: np.ndarray, trans_a: bool = False,
               trans_b: bool = False, nthreads: int | None = None,
               out: np.ndarray | None = None) -> np.ndarray:
    """C = op(A) op(B) by the fixed-order definition (the C triple loop).

    ``A``/``B`` are the *stored* matrices, any element strides (negative and
    zero included); ``trans_*`` are logical transposes.  Returns an M x N
    float32 array (or fills ``out``).
    """
    M, N, K = _logical_shapes(A, B, trans_a, trans_b)
    if out is None:
        out = np.empty((M, N), dtype=np.float32)
    if out.shape != (M, N) or out.dtype != np.float32:
        raise ValueError("out must be float32 of shape (M, N)")
    pa, ars, acs = _operand(A)
    pb, brs, bcs = _operand(B)
    pc, crs, ccs = _operand(out)
    rc = _load().repops_oracle_matmul_f32(
        pa, ars, acs, pb, brs, bcs, pc, crs, ccs, M, N, K,
        int(bool(trans_a)), int(bool(trans_b)), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle failed with status %d" % rc)
    return out


def entries_f32(A: np.ndarray, B: np.ndarray, ii, jj, trans_a: bool = False,
                trans_b: bool = False, nthreads: int | None = None) -> np.ndarray:
    """C(ii[e], jj[e]) for each e, by the same fixed-order definition."""
    M, N, K = _logical_shapes(A, B, trans_a, trans_b)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D of equal length")
    out = np.empty(ii.shape[0], dtype=np.float32)
    pa, ars, acs = _operand(A)
    pb, brs, bcs = _operand(B)
    rc = _load().repops_oracle_entries_f32(
        pa, ars, acs, pb, brs, bcs, M, N, K, int(bool(trans_a)), int(bool(trans_b)),
        ii.ctypes.data, jj.ctypes.data, ii.shape[0], out.ctypes.data,
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle failed with status %d" % rc)
    return out


def canonical_order(dids) -> list:
    """Contributor indices sorted by DID byte order (Zoo Per-LLM Chain
    Soundness, "Ordering subroutine": lexicographic on the DID bytes).
    Python compares bytes objects exactly that way (unsigned bytes, a proper
    prefix first).  Two equal DIDs are an error: the batch is keyed by
    contributor."""
    keys = [bytes(x) for x in dids]
    if len(set(keys)) != len(keys):
        raise ValueError("duplicate contributor DID")
    return sorted(range(len(keys)), key=lambda c: keys[c])


def fold_mean_sgd_f32(grads, eta, theta):
    """Left-fold average of the gradients (in the given order), then
    theta - eta * gbar; returns (new theta, gbar) as float32 arrays."""
    grads = [np.ascontiguousarray(g, dtype=np.float32) for g in grads]
    theta = np.ascontiguousarray(theta, dtype=np.float32)
    k = len(grads)
    if k < 1:
        raise ValueError("need at least one gradient")
    d = theta.shape[0]
    if any(g.shape != (d,) for g in grads):
        raise ValueError("gradients and theta must all have length d")
    ptrs = (ctypes.c_void_p * k)(*[g.ctypes.data for g in grads])
    out = np.empty(d, np.float32)
    gbar = np.empty(d, np.float32)
    rc = _load().repops_oracle_fold_mean_sgd_f32(ptrs, k, d, float(np.float32(eta)),
                                                theta.ctypes.data, out.ctypes.data,
                                                gbar.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle failed with status %d" % rc)
    return out, gbar


def matmul_batched_f32(A: np.ndarray, B: np.ndarray, trans_a: bool = False,
                       trans_b: bool = False, bias: np.ndarray | None = None,
                       nthreads: int | None = None) -> np.ndarray:
    """C_b = op(A_b) op(B_b) (+ bias_b) for stored 3-D A (batch, ., .) and B;
    bias is (N,) (shared by all batches) or (batch, N).  Any element strides."""
    if A.ndim != 3 or B.ndim != 3 or A.shape[0] != B.shape[0]:
        raise ValueError("A and B must be 3-D with equal batch")
    batch = A.shape[0]
    M, N, K = _logical_shapes(A[0] if batch else A.reshape(A.shape[1:]),
                              B[0] if batch else B.reshape(B.shape[1:]), trans_a, trans_b)
    out = np.empty((batch, M, N), dtype=np.float32)
    sa = [x // 4 for x in A.strides]
    sb = [x // 4 for x in B.strides]
    so = [x // 4 for x in out.strides]
    pb, bbs, bs = None, 0, 0
    if bias is not None:
        bias = np.asarray(bias)
        if bias.dtype != np.float32:
            raise TypeError("bias must be float32")
        if bias.ndim == 1:
            pb, bbs, bs = bias.ctypes.data, 0, bias.strides[0] // 4
        else:
            pb, bbs, bs = bias.ctypes.data, bias.strides[0] // 4, bias.strides[1] // 4
    rc = _load().repops_oracle_matmul_batched_f32(
        A.ctypes.data, sa[0], sa[1], sa[2], B.ctypes.data, sb[0], sb[1], sb[2],
        out.ctypes.data, so[0], so[1], so[2], M, N, K, batch, int(bool(trans_a)),
        int(bool(trans_b)), pb, bbs, bs, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle failed with status %d" % rc)
    return out


def _f32_1d(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).reshape(-1)


def erf_f32(x) -> np.ndarray:
    """erf by Abramowitz and Stegun 7.1.28 in the fixed binary32 order of
    repops_oracle.c; same shape as x."""
    x = np.asarray(x, dtype=np.float32)
    xf = _f32_1d(x)
    y = np.empty_like(xf)
    rc = _load().repops_oracle_erf_f32(xf.ctypes.data, y.ctypes.data, xf.size)
    if rc != 0:
        raise RuntimeError("oracle erf failed (%d)" % rc)
    return y.reshape(x.shape)


def gelu_f32(x) -> np.ndarray:
    """GeLU = (x * 0.5) * (1 + erf(x * RN(1/sqrt 2))) in the fixed binary32 order."""
    x = np.asarray(x, dtype=np.float32)
    xf = _f32_1d(x)
    y = np.empty_like(xf)
    rc = _load().repops_oracle_gelu_f32(xf.ctypes.data, y.ctypes.data, xf.size)
    if rc != 0:
        raise RuntimeError("oracle gelu failed (%d)" % rc)
    return y.reshape(x.shape)


def layernorm_f32(x, gamma=None, beta=None, eps=1e-5):
    """LayerNorm over the last dimension of a 2-D array, fixed order (see
    repops_oracle.c).  Returns (y, mean, rstd)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x.ndim != 2:
        raise ValueError("x must be 2-D (rows, H)")
    rows, H = x.shape
    g = None if gamma is None else _f32_1d(gamma)
    b = None if beta is None else _f32_1d(beta)
    for v in (g, b):
        if v is not None and v.size != H:
            raise ValueError("gamma and beta need H elements")
    y = np.empty_like(x)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    rc = _load().repops_oracle_layernorm_f32(
        x.ctypes.data, H, None if g is None else g.ctypes.data,
        None if b is None else b.ctypes.data, y.ctypes.data, H, rows, H,
        float(np.float32(eps)), mean.ctypes.data, rstd.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle layernorm failed (%d)" % rc)
    return y, mean, rstd
