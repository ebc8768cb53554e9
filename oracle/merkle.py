"""CPU oracle for tensor hashing and the referee's single-operator
re-execution -- TEST INFRASTRUCTURE ONLY (tests, the smoke check and the
benchmark's CPU leg; the GPU library never uses it).

What the pages fix (Verde and RepOps article, section 2.3.1 "extended
computation graph": every node carries hash lists of its input and output
tensors; section 2.3.2: checkpoint hashes are Merkle trees; section 2.4
"referee decision algorithm", case 3: when only an output-tensor hash
differs, the referee runs that one operator itself and sees which trainer's
hash it reproduces).  What they leave open, and the reading taken here:

* the hash function: SHA-256 (FIPS 180-4), taken from Python's ``hashlib``
  as a library primitive, and pinned by the standard's own example digests;
* the tensor hash: the Merkle Tree Hash of RFC 6962, section 2.1 (leaf
  hash SHA-256(0x00 || leaf), node hash SHA-256(0x01 || left || right), the
  left subtree holding the largest power of two of leaves smaller than n,
  the empty tree hashing to SHA-256 of the empty string);
* the leaves: the tensor's bytes cut into ``leaf_bytes`` pieces from the
  start, the last piece shorter when the length is not a multiple;
* the tensor's bytes: its elements in logical row-major order, each the
  little-endian binary32 encoding, so the hash does not depend on strides.

The tree is written as the RFC's recursive definition; nothing here builds it
level by level (the GPU path does, which is what the pins compare against).
"""
from __future__ import annotations

import hashlib

import numpy as np


def sha256(data: bytes) -> bytes:
    """The one hash primitive every function below goes through."""
    return hashlib.sha256(data).digest()


def leaf_hash(leaf: bytes) -> bytes:
    """RFC 6962 section 2.1: MTH({d}) = SHA-256(0x00 || d)."""
    return sha256(b"\x00" + leaf)


def node_hash(left: bytes, right: bytes) -> bytes:
    """RFC 6962 section 2.1: SHA-256(0x01 || MTH(left) || MTH(right))."""
    return sha256(b"\x01" + left + right)


def _split(n: int) -> int:
    """The largest power of two smaller than n (n >= 2)."""
    k = 1
    while 2 * k < n:
        k *= 2
    return k


def split_leaves(data: bytes, leaf_bytes: int):
    """The tensor's bytes cut into leaves of leaf_bytes, the last one shorter."""
    if leaf_bytes < 1:
        raise ValueError("leaf_bytes must be positive")
    return [data[i:i + leaf_bytes] for i in range(0, len(data), leaf_bytes)]


def _mth(hashes, lo: int, hi: int) -> bytes:
    n = hi - lo
    if n == 1:
        return hashes[lo]
    k = _split(n)
    return node_hash(_mth(hashes, lo, lo + k), _mth(hashes, lo + k, hi))


def mth(leaves) -> bytes:
    """Merkle Tree Hash of a list of leaf byte strings (RFC 6962 section 2.1)."""
    if len(leaves) == 0:
        return sha256(b"")
    hashes = [leaf_hash(d) for d in leaves]
    return _mth(hashes, 0, len(hashes))


def merkle_root(data: bytes, leaf_bytes: int) -> bytes:
    """Root of the tree over ``data`` cut into ``leaf_bytes`` leaves."""
    return mth(split_leaves(bytes(data), leaf_bytes))


def audit_path(m: int, leaves):
    """RFC 6962 section 2.1.1: the audit path of leaf m, bottom first."""
    def path(m, lo, hi):
        n = hi - lo
        if n == 1:
            return []
        k = _split(n)
        if m < k:
            return path(m, lo, lo + k) + [_mth(hashes, lo + k, hi)]
        return path(m - k, lo + k, hi) + [_mth(hashes, lo, lo + k)]

    hashes = [leaf_hash(d) for d in leaves]
    if not 0 <= m < len(hashes):
        raise IndexError(m)
    return path(m, 0, len(hashes))


def tensor_bytes(x) -> bytes:
    """Elements in logical row-major order, little-endian binary32 each."""
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).astype("<f4").tobytes()


def tensor_root(x, leaf_bytes: int) -> bytes:
    return merkle_root(tensor_bytes(x), leaf_bytes)


def referee_matmul(A, B, trans_a: bool, trans_b: bool, claims, leaf_bytes: int, nthreads=None):
    """Section 2.4, case 3, for the matmul operator: recompute C = op(A) op(B)
    with the fixed-order oracle, hash it, and report which claimed output
    hashes it reproduces.  Returns (root, [claim == root for each claim], C)."""
    from . import matmul_f32

    C = matmul_f32(A, B, trans_a=trans_a, trans_b=trans_b, nthreads=nthreads)
    root = tensor_root(C, leaf_bytes)
    return root, [bytes(c) == root for c in claims], C
