"""Pins for the tensor-hash and referee oracle (oracle/merkle.py).

The Verde and RepOps article (sections 2.3-2.4) has trainers hash every
operator's output and a referee re-run one disputed operator; it names no
hash.  The oracle reads that as SHA-256 in RFC 6962's Merkle tree.  What pins
it, independently of its own code:

* the primitive: the Secure Hash Standard's example digests
  (tests/golden/sha256_fips180.txt);
* the tree shape: every leaf's audit path (RFC 6962 section 2.1.1) checked by
  the inclusion verifier of RFC 9162 section 2.1.3.2, a bit-walking
  algorithm written here, with its own leaf and node hashing; perfect trees
  rebuilt by pairwise hashing; the one-leaf and empty trees;
* the byte layout: little-endian binary32 elements in logical row-major order;
* the referee: an honest claim is reproduced, a claim off by one bit in one
  element or computed in another summation order is not;
* mutation controls: plausible mistakes planted in the oracle (a balanced
  split, no domain-separation prefixes, big-endian elements) each fail a pin.
"""
from __future__ import annotations

import hashlib
import os

import numpy as np
import pytest

import oracle
from oracle import merkle
from bit_reproducible_fp32_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "sha256_fips180.txt")


def _message(spec):
    if spec == "empty":
        return b""
    kind, _, rest = spec.partition(":")
    if kind == "ascii":
        return rest.encode()
    if kind == "repeat":
        count, _, ch = rest.partition(":")
        return ch.encode() * int(count)
    raise ValueError(spec)


def fips_cases():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, spec, digest = line.rstrip("\n").split("\t")
        out.append((name, spec, digest))
    return out


# -- an independent verifier (RFC 9162 section 2.1.3.2), own hashing ---------
def _leaf(d):
    return hashlib.sha256(b"\x00" + d).digest()


def _node(left, right):
    return hashlib.sha256(b"\x01" + left + right).digest()


def verify_inclusion(index, size, leaf_h, path, root):
    if index >= size:
        return False
    fn, sn, r = index, size - 1, leaf_h
    for p in path:
        if sn == 0:
            return False
        if fn & 1 or fn == sn:
            r = _node(p, r)
            while not fn & 1 and fn != 0:
                fn >>= 1
                sn >>= 1
        else:
            r = _node(r, p)
        fn >>= 1
        sn >>= 1
    return sn == 0 and r == root


def leaves_for(n, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed + n))
    return [bytes(rng.integers(0, 256, size=int(rng.integers(0, 9)), dtype=np.uint8))
            for _ in range(n)]


def check_all_inclusions(max_n=40):
    for n in range(1, max_n + 1):
        leaves = leaves_for(n)
        root = merkle.mth(leaves)
        for m in range(n):
            path = merkle.audit_path(m, leaves)
            if not verify_inclusion(m, n, _leaf(leaves[m]), path, root):
                return False
    return True


# -- the primitive ------------------------------------------------------------
@pytest.mark.parametrize("name,spec,digest", fips_cases())
def test_sha256_standard_vectors(name, spec, digest):
    assert merkle.sha256(_message(spec)).hex() == digest


# -- the tree -------------------------------------------------------------------
def test_empty_tree_is_hash_of_empty_string():
    digest = dict((n, d) for n, _, d in fips_cases())["empty"]
    assert merkle.mth([]).hex() == digest
    assert merkle.merkle_root(b"", 1024).hex() == digest


def test_single_leaf_tree():
    for d in (b"", b"\x01", b"abc" * 50):
        assert merkle.mth([d]) == hashlib.sha256(b"\x00" + d).digest()


def test_every_audit_path_verifies():
    assert check_all_inclusions(40)


def test_verifier_rejects_wrong_index_and_tampered_path():
    leaves = leaves_for(13)
    root = merkle.mth(leaves)
    path = merkle.audit_path(5, leaves)
    assert verify_inclusion(5, 13, _leaf(leaves[5]), path, root)
    assert not verify_inclusion(6, 13, _leaf(leaves[5]), path, root)
    bad = list(path)
    bad[1] = bytes([bad[1][0] ^ 1]) + bad[1][1:]
    assert not verify_inclusion(5, 13, _leaf(leaves[5]), bad, root)


@pytest.mark.parametrize("j", range(0, 7))
def test_perfect_tree_is_pairwise_hashing(j):
    leaves = leaves_for(1 << j, seed=99)
    level = [_leaf(d) for d in leaves]
    while len(level) > 1:
        level = [_node(level[i], level[i + 1]) for i in range(0, len(level), 2)]
    assert merkle.mth(leaves) == level[0]


def test_one_past_a_power_of_two():
    # n = 2^j + 1: the root joins the perfect tree of the first 2^j leaves
    # with the last leaf alone.
    for j in range(0, 6):
        leaves = leaves_for((1 << j) + 1, seed=7)
        assert merkle.mth(leaves) == _node(merkle.mth(leaves[:-1]), _leaf(leaves[-1]))


def test_leaf_split_ragged_tail():
    data = bytes(range(256)) * 10  # 2560 bytes
    leaves = merkle.split_leaves(data, 1024)
    assert [len(x) for x in leaves] == [1024, 1024, 512]
    assert b"".join(leaves) == data
    assert merkle.split_leaves(data, 4096) == [data]
    assert merkle.merkle_root(data, 4096) == _leaf(data)


# -- the tensor bytes ---------------------------------------------------------
def test_tensor_bytes_little_endian_row_major():
    assert merkle.tensor_bytes(np.array([[1.0]], dtype=np.float32)) == b"\x00\x00\x80\x3f"
    x = np.array([[1.0, 2.0], [3.0, 4.0]], dtype=np.float32)
    expect = b"".join(np.float32(v).tobytes() for v in (1.0, 2.0, 3.0, 4.0))
    assert merkle.tensor_bytes(x) == expect
    # a transposed view hashes its logical order, not its storage
    xt = np.array([[1.0, 3.0], [2.0, 4.0]], dtype=np.float32).T
    assert merkle.tensor_bytes(xt) == expect
    assert merkle.tensor_root(xt, 4) == merkle.mth([np.float32(v).tobytes()
                                                    for v in (1.0, 2.0, 3.0, 4.0)])


def test_any_byte_flip_changes_the_root():
    data = bytearray(range(200))
    root = merkle.merkle_root(bytes(data), 16)
    for i in range(len(data)):
        data[i] ^= 0x40
        assert merkle.merkle_root(bytes(data), 16) != root
        data[i] ^= 0x40


# -- the referee ----------------------------------------------------------------
def _reverse_order_matmul(A, B):
    # a trainer who summed k in descending order (float32 numpy, unfused)
    M, K = A.shape
    N = B.shape[1]
    s = np.zeros((M, N), dtype=np.float32)
    for k in range(K - 1, -1, -1):
        s = (s + (A[:, k:k + 1] * B[k:k + 1, :]).astype(np.float32)).astype(np.float32)
    return s


def test_referee_picks_the_honest_trainer():
    A = inputs.random_matrix((24, 300), 11)
    B = inputs.random_matrix((300, 17), 12)
    C = oracle.matmul_f32(A, B)
    honest = merkle.tensor_root(C, 64)
    C1 = C.copy()
    C1.view(np.uint32)[7, 3] ^= 1  # one ulp in one element
    off_by_one = merkle.tensor_root(C1, 64)
    reordered = merkle.tensor_root(_reverse_order_matmul(A, B), 64)
    assert reordered != honest
    root, match, C_ref = merkle.referee_matmul(A, B, False, False,
                                               [honest, off_by_one, reordered], 64)
    assert root == honest and match == [True, False, False]
    assert np.array_equal(C_ref.view(np.uint32), C.view(np.uint32))


def test_referee_transposed_operands():
    A = inputs.random_matrix((40, 9), 13)   # stored K x M
    B = inputs.random_matrix((15, 40), 14)  # stored N x K
    C = oracle.matmul_f32(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T))
    root, match, _ = merkle.referee_matmul(A, B, True, True, [merkle.tensor_root(C, 32)], 32)
    assert match == [True]


# -- mutation controls ------------------------------------------------------------
def test_mutant_balanced_split_is_caught(monkeypatch):
    monkeypatch.setattr(merkle, "_split", lambda n: n // 2)
    assert not check_all_inclusions(12)


def test_mutant_no_leaf_prefix_is_caught(monkeypatch):
    monkeypatch.setattr(merkle, "leaf_hash", lambda d: hashlib.sha256(d).digest())
    with pytest.raises(AssertionError):
        test_single_leaf_tree()


def test_mutant_no_node_prefix_is_caught(monkeypatch):
    monkeypatch.setattr(merkle, "node_hash", lambda l, r: hashlib.sha256(l + r).digest())
    assert not check_all_inclusions(6)


def test_mutant_big_endian_elements_is_caught(monkeypatch):
    monkeypatch.setattr(merkle, "tensor_bytes",
                        lambda x: np.ascontiguousarray(x, dtype=np.float32).astype(">f4").tobytes())
    with pytest.raises(AssertionError):
        test_tensor_bytes_little_endian_row_major()
