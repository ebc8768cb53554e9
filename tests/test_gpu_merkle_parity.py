"""GPU parity of the tensor hash (repops_merkle_root) and the referee's
re-execution of a disputed matmul (repops_referee_matmul_f32), through the C
ABI, against the CPU oracle (oracle/merkle.py), byte for byte.

Covered: the empty input; one-block and two-block padding boundaries; a
tree of exactly one workgroup (256 leaves) and trees needing two, three and
four launches (the first hashes the leaves and folds 0, 2 or more levels
depending on the leaf size, later ones fold groups of 1024 digests); leaf
sizes from 4 bytes to 2^24 bytes, and seeded random sizes and leaf lengths; the narrow-load path
(leaves not a multiple of 16 bytes, data only 4-byte aligned); workspace
reuse across calls; the tensor hash of matmul outputs; the referee's verdicts
(an honest claim, a claim one bit off, a claim from another summation order,
two honest trainers, no claims, transposed operands, empty and K = 0
products); and the full-size Llama-8B-shaped up-projection output in the
launch configuration the benchmark times."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import merkle
from bit_reproducible_fp32_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_reproducible_fp32_amd as rp  # noqa: E402

DEV = "cuda:0"


def say(msg):
    print("[gpu-merkle] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def random_bytes(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 256, size=n, dtype=np.uint8)


def on_gpu(data: np.ndarray, offset_words=0):
    """A uint8 device view of data starting offset_words * 4 bytes into a
    fresh allocation (torch allocations are 256-byte aligned)."""
    buf = torch.zeros(data.size + 4 * offset_words + 16, dtype=torch.uint8, device=DEV)
    view = buf[4 * offset_words:4 * offset_words + data.size]
    view.copy_(torch.from_numpy(data))
    return view


CASES = [
    # (nbytes, leaf_bytes, offset_words)
    (0, 1024, 0),
    (4, 4, 0),
    (8, 4, 0),
    (52, 64, 0), (56, 64, 0), (60, 64, 0), (64, 64, 0), (68, 64, 0),
    (116, 1024, 0), (120, 1024, 0), (124, 1024, 0), (128, 1024, 0),
    (1024, 1024, 0), (1028, 1024, 0),
    (256 * 1024, 1024, 0),          # 256 leaves: one launch
    (256 * 1024 + 4, 1024, 0),      # 257 leaves: 257 digests, then the root
    (1025 * 1024, 1024, 0),         # 1025 digests: three launches
    (65536 * 4, 4, 0),              # 4-byte leaves fold 6 levels: 1024 digests
    (65537 * 4, 4, 0),              # 1025 digests: three launches
    ((1024 * 1024 + 1) * 1024, 1024, 0),  # 1048577 digests: four launches (1 GiB)
    (4097 * 256, 256, 0),           # 256-byte leaves fold 2 levels: 1025 digests
    (4096 * 1020 + 8, 1020, 0),     # just under 1 KiB: 2 levels, last leaf short
    (1000 * 52 + 12, 52, 0),        # leaves not a multiple of 16 bytes
    (300 * 1024 + 8, 1024, 1),      # data 4-byte but not 16-byte aligned
    (77 * 4096 + 2048, 4096, 0),
    (3 * (1 << 20) + 12, 1 << 20, 0),
    ((1 << 24) + 8, 1 << 24, 0),    # the largest leaf
]


@pytest.mark.parametrize("nbytes,leaf,offset", CASES)
def test_root_of_bytes(nbytes, leaf, offset):
    say("root nbytes=%d leaf=%d offset=%d" % (nbytes, leaf, offset))
    data = random_bytes(nbytes, seed=nbytes * 7 + leaf)
    got = rp.merkle_root(on_gpu(data, offset), leaf_bytes=leaf)
    assert got == merkle.merkle_root(data.tobytes(), leaf)


def test_random_sizes_and_leaf_lengths():
    """12 seeded random (size, leaf length, alignment) cases on both sides of
    the first launch's fold policy."""
    rng = np.random.default_rng(77)
    for case in range(12):
        leaf = 4 * int(rng.integers(1, 1025))               # 4 .. 4096 bytes
        n_leaves = int(rng.integers(1, 20001))
        nbytes = max(0, (n_leaves - 1) * leaf + 4 * int(rng.integers(1, leaf // 4 + 1)))
        offset = int(rng.integers(0, 4))
        say("random case %d: nbytes=%d leaf=%d offset=%d" % (case, nbytes, leaf, offset))
        data = random_bytes(nbytes, seed=1000 + case)
        got = rp.merkle_root(on_gpu(data, offset), leaf_bytes=leaf)
        assert got == merkle.merkle_root(data.tobytes(), leaf), case


def test_workspace_reused_across_calls_and_async_out():
    say("workspace reuse")
    big = random_bytes(4 * 70000, 1)
    small = random_bytes(4 * 300, 2)
    ws = torch.empty(rp.repops_merkle_workspace_bytes(big.size, 4), dtype=torch.uint8, device=DEV)
    out = torch.empty(32, dtype=torch.uint8, device=DEV)
    rp.merkle_root(on_gpu(big), leaf_bytes=4, workspace=ws, out=out)
    torch.cuda.synchronize()
    assert bytes(out.cpu().numpy()) == merkle.merkle_root(big.tobytes(), 4)
    assert rp.merkle_root(on_gpu(small), leaf_bytes=4, workspace=ws) == \
        merkle.merkle_root(small.tobytes(), 4)


@pytest.mark.parametrize("M,N,K,leaf", [(300, 190, 270, 1024), (64, 64, 16, 64),
                                        (1, 1000, 3, 4)])
def test_tensor_hash_of_matmul_output(M, N, K, leaf):
    say("tensor hash of a %dx%dx%d product, leaf %d" % (M, N, K, leaf))
    A = inputs.random_matrix((M, K), 31)
    B = inputs.random_matrix((K, N), 32)
    C = rp.matmul(torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV))
    expect = merkle.tensor_root(oracle.matmul_f32(A, B), leaf)
    assert rp.merkle_root(C, leaf_bytes=leaf) == expect


def _reverse_order(A, B):
    s = np.zeros((A.shape[0], B.shape[1]), dtype=np.float32)
    for k in range(A.shape[1] - 1, -1, -1):
        s = (s + (A[:, k:k + 1] * B[k:k + 1, :]).astype(np.float32)).astype(np.float32)
    return s


@pytest.mark.parametrize("leaf", [64, 1024, 4096])
def test_referee_verdicts(leaf):
    say("referee verdicts, leaf %d" % leaf)
    A = inputs.random_matrix((200, 333), 41)
    B = inputs.random_matrix((333, 150), 42)
    C = oracle.matmul_f32(A, B)
    honest = merkle.tensor_root(C, leaf)
    C1 = C.copy()
    C1.view(np.uint32)[199, 149] ^= 1
    tampered = merkle.tensor_root(C1, leaf)
    reordered = merkle.tensor_root(_reverse_order(A, B), leaf)
    assert len({honest, tampered, reordered}) == 3
    a, b = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    root, match, out = rp.referee_matmul(a, b, [honest, tampered, reordered], leaf_bytes=leaf)
    assert root == honest and match == [True, False, False]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), C.view(np.uint32))
    root, match, _ = rp.referee_matmul(a, b, [tampered, honest, honest], leaf_bytes=leaf)
    assert match == [False, True, True]
    root, match, _ = rp.referee_matmul(a, b, [], leaf_bytes=leaf)
    assert root == honest and match == []


def test_referee_transposed_operands():
    say("referee, transposed operands")
    A = inputs.random_matrix((90, 70), 43)   # stored K x M
    B = inputs.random_matrix((50, 90), 44)   # stored N x K
    C = oracle.matmul_f32(A, B, trans_a=True, trans_b=True)
    claim = merkle.tensor_root(C, 1024)
    root, match, _ = rp.referee_matmul(torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV),
                                       [claim], trans_a=True, trans_b=True)
    assert match == [True] and root == claim


def test_referee_empty_and_k0():
    say("referee, empty and K = 0")
    empty = merkle.merkle_root(b"", 1024)
    a = torch.zeros((0, 5), device=DEV)
    b = torch.zeros((5, 7), device=DEV)
    root, match, _ = rp.referee_matmul(a, b, [empty])
    assert root == empty and match == [True]
    a = torch.zeros((6, 0), device=DEV)
    b = torch.zeros((0, 9), device=DEV)
    zeros = merkle.tensor_root(np.zeros((6, 9), np.float32), 1024)
    root, match, out = rp.referee_matmul(a, b, [zeros])
    assert root == zeros and match == [True]


def test_full_size_up_projection_output():
    """The benchmark's configuration: the Llama-8B-shaped up-projection
    (4096 x 14336, K = 4096), 1 KiB leaves.  The matmul's bits are checked
    on sampled outputs against the oracle; the hash over all 235 MB is
    checked against the oracle's hash of the same bytes."""
    w = inputs.WORKLOADS["llama8b_mlp_up"]
    say("full size %s" % w.name)
    A, B = inputs.make_operands(w.name)
    a, b = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    C = rp.matmul(a, b)
    host = C.cpu().numpy()
    ii, jj = inputs.sample_entries(w.M, w.N, 128, seed=77)
    ref = oracle.entries_f32(A, B, ii, jj)
    assert np.array_equal(host[ii, jj].view(np.uint32), ref.view(np.uint32))
    expect = merkle.tensor_root(host, 1024)
    assert rp.merkle_root(C, leaf_bytes=1024) == expect
    bad = host.copy()
    bad.view(np.uint32)[w.M // 2, w.N - 1] ^= 0x80000000
    tampered = merkle.tensor_root(bad, 1024)
    root, match, out = rp.referee_matmul(a, b, [tampered, expect])
    assert root == expect and match == [False, True]
