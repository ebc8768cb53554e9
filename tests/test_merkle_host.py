"""Host checks of the tensor-hash and referee entry points (no GPU needed).

* the SHA-256 constants in the kernel source follow their FIPS 180-4
  definitions (sections 4.2.2 and 5.3.3), recomputed here with exact integer
  roots of the primes;
* the workspace query and every argument error of repops_merkle_root and
  repops_referee_matmul_f32, each returned before any device work (the
  pointers here are fake and never dereferenced);
* the hash kernels keep everything in registers (no spills).
"""
from __future__ import annotations

import math
import os
import re

import pytest

import bit_reproducible_fp32_amd as rp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "bit_reproducible_fp32_amd", "csrc", "repops_merkle.hip")
ASM = os.path.join(ROOT, "bit_reproducible_fp32_amd", "librepops_gfx950.s")

PD, PW, PR = 0x10000000, 0x20000000, 0x30000000   # data, workspace, root
PA, PB, PC, PCL, PM = 0x40000000, 0x50000000, 0x60000000, 0x70000000, 0x78000000


def primes(n):
    out, k = [], 2
    while len(out) < n:
        if all(k % p for p in out if p * p <= k):
            out.append(k)
        k += 1
    return out


def icbrt(x):
    lo, hi = 0, 1 << ((x.bit_length() + 2) // 3 + 1)
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if mid ** 3 <= x:
            lo = mid
        else:
            hi = mid - 1
    return lo


def source_table(name):
    text = open(SRC).read()
    m = re.search(name + r"\[\d+\]\s*=\s*\{(.*?)\};", text, re.S)
    return [int(v, 16) for v in re.findall(r"0x([0-9a-fA-F]+)u", m.group(1))]


def test_round_constants_are_cube_roots_of_primes():
    want = [icbrt(p << 96) & 0xffffffff for p in primes(64)]
    assert source_table("kRound") == want


def test_initial_state_is_square_roots_of_primes():
    want = [math.isqrt(p << 64) & 0xffffffff for p in primes(8)]
    assert source_table("kInit") == want


def test_workspace_query():
    ws = rp.repops_merkle_workspace_bytes
    assert ws(0, 1024) == 0
    assert ws(256 * 1024, 1024) == 0            # 256 leaves: one workgroup
    # Leaves of 256 bytes or more: the first launch writes one digest per
    # leaf; shorter leaves are folded until 256 bytes sit under each digest.
    assert ws(256 * 1024 + 4, 1024) == 8448     # 257 digests (8224 B, rounded to 256)
    assert ws(4096 * 14336 * 4, 1024) == 7340032 + 7168   # 229376 digests, then 224
    assert ws(4 * (256 * 1024 + 1), 4) == 131328 + 256    # 4-byte leaves, 64 per digest:
    #                                                        4097 digests, then 5
    assert ws(256 * 1024 + 64, 64) == 33024 + 256  # 64-byte leaves, 4 per digest: 1025, then 2
    for nbytes, leaf in ((6, 4), (-4, 4), (8, 6), (8, 0), (8, 2), (8, (1 << 24) + 4),
                         ((1 << 50) + 4, 1024)):
        assert ws(nbytes, leaf) == -1, (nbytes, leaf)


def root_call(**kw):
    # 1 MiB in 1 KiB leaves: 1024 digests after the first stage, 32768 bytes
    # of workspace.  Every call made with this helper is invalid in one way.
    args = dict(data=PD, nbytes=1 << 20, leaf_bytes=1024, workspace=PW, workspace_bytes=1 << 16,
                root=PR, stream=0)
    args.update(kw)
    return rp.repops_merkle_root(**args)


def test_merkle_root_argument_errors():
    assert root_call(nbytes=6) == rp.REPOPS_ERR_DIM
    assert root_call(leaf_bytes=1022) == rp.REPOPS_ERR_DIM
    assert root_call(leaf_bytes=1 << 25) == rp.REPOPS_ERR_DIM
    assert root_call(root=None) == rp.REPOPS_ERR_NULL
    assert root_call(data=None) == rp.REPOPS_ERR_NULL
    assert root_call(root=PR + 2) == rp.REPOPS_ERR_ALIGN
    assert root_call(data=PD + 2) == rp.REPOPS_ERR_ALIGN
    assert root_call(workspace=PW + 4) == rp.REPOPS_ERR_ALIGN
    assert root_call(workspace=None) == rp.REPOPS_ERR_WORKSPACE
    assert root_call(workspace_bytes=32767) == rp.REPOPS_ERR_WORKSPACE  # 32768 needed
    assert root_call(root=PD + 1024) == rp.REPOPS_ERR_ALIAS
    assert root_call(workspace=PD + 4096) == rp.REPOPS_ERR_ALIAS
    assert root_call(root=PW + 32) == rp.REPOPS_ERR_ALIAS


def referee_call(**kw):
    # 1024 x 512 outputs = 2048 leaves of 1 KiB: 65536 + 256 bytes of
    # workspace are needed
    args = dict(A=PA, a_rs=64, a_cs=1, B=PB, b_rs=512, b_cs=1, C=PC, M=1024, N=512, K=64,
                trans_a=0, trans_b=0, leaf_bytes=1024, workspace=PW, workspace_bytes=65792,
                claims=PCL, nclaims=2, root=PR, match=PM, stream=0)
    args.update(kw)
    return rp.repops_referee_matmul_f32(**args)


def test_referee_argument_errors():
    # every call below fails validation, so nothing is launched
    assert referee_call(C=PA) == rp.REPOPS_ERR_ALIAS            # matmul's own checks first
    assert referee_call(M=-1) == rp.REPOPS_ERR_DIM
    assert referee_call(leaf_bytes=1002) == rp.REPOPS_ERR_DIM
    assert referee_call(nclaims=-1) == rp.REPOPS_ERR_DIM
    assert referee_call(claims=None) == rp.REPOPS_ERR_NULL
    assert referee_call(match=None) == rp.REPOPS_ERR_NULL
    assert referee_call(match=PM + 2) == rp.REPOPS_ERR_ALIGN
    assert referee_call(workspace_bytes=0) == rp.REPOPS_ERR_WORKSPACE
    assert referee_call(workspace_bytes=65791) == rp.REPOPS_ERR_WORKSPACE
    assert referee_call(match=PC + 64) == rp.REPOPS_ERR_ALIAS
    assert referee_call(claims=PC) == rp.REPOPS_ERR_ALIAS
    assert referee_call(root=PC + 32) == rp.REPOPS_ERR_ALIAS
    assert referee_call(match=PR) == rp.REPOPS_ERR_ALIAS


def test_status_strings():
    assert "aligned" in rp.repops_strerror(rp.REPOPS_ERR_ALIGN)
    assert "workspace" in rp.repops_strerror(rp.REPOPS_ERR_WORKSPACE)


def test_python_wrappers_refuse_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        rp.merkle_root(torch.zeros(16))
    with pytest.raises(ValueError):
        rp.referee_matmul(torch.zeros(4, 4), torch.zeros(4, 4), [])


def test_hash_kernels_do_not_spill():
    text = open(ASM).read()
    seen = 0
    for block in text.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        if "merkle" not in name:
            continue
        seen += 1
        spill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1))
        priv = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
        assert spill == 0 and priv == 0, name
    assert seen >= 4
