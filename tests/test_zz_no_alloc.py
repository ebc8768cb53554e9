"""The no-allocation tensor hash, repops_merkle_root_noalloc, against the
workspace entry point repops_merkle_root, through the C ABI.

The no-allocation call keeps its intermediate digests in the library's static
16 MiB device array instead of a caller's workspace; its root must be
byte-identical to repops_merkle_root's on the same bytes.  Two calls in a row
(the second on a smaller input, so the array still holds the first call's
digests), then one that needs no scratch at all, each also against the CPU
oracle where that is quick.  Sizes beyond the array are refused on the host
before anything is queued.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import bit_reproducible_fp32_amd as rp

torch = pytest.importorskip("torch")


def say(msg):
    print("[no-alloc] " + msg, flush=True)
    sys.stdout.flush()


def test_oversized_and_invalid_inputs_are_refused_on_the_host():
    rp.load()
    max_b = rp.REPOPS_NOALLOC_SCRATCH_BYTES
    # 1 KiB leaves need 32 bytes of scratch per leaf: 2^19 leaves fill 16 MiB.
    too_big = (max_b // 32 + 4096) * 1024
    assert rp.repops_merkle_workspace_bytes(too_big, 1024) > max_b
    fake = 1 << 20     # never dereferenced: the call returns before any launch
    assert rp.repops_merkle_root_noalloc(fake, too_big, 1024, fake + (1 << 40), None) \
        == rp.REPOPS_ERR_SCRATCH
    assert rp.repops_merkle_root_noalloc(fake, 6, 1024, fake + (1 << 40), None) == rp.REPOPS_ERR_DIM
    assert rp.repops_merkle_root_noalloc(fake, 1024, 1024, None, None) == rp.REPOPS_ERR_NULL
    assert "static" in rp.repops_strerror(rp.REPOPS_ERR_SCRATCH)


@pytest.mark.gpu
def test_noalloc_root_equals_workspace_root_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    from oracle import merkle
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rng = np.random.Generator(np.random.PCG64(424242))
    # (bytes, leaf bytes, check against the CPU oracle too)
    cases = [(400 * 1024 * 1024 + 12, 1024, False),   # 12.5 MiB of scratch
             (3 * 1024 * 1024 + 36, 64, True),        # smaller; short leaves fold in LDS
             (200 * 1024, 1024, True),                # 200 leaves: no scratch at all
             (0, 1024, True)]                         # the empty input
    for nbytes, leaf, with_oracle in cases:
        need = rp.repops_merkle_workspace_bytes(nbytes, leaf)
        say("nbytes %d leaf %d: scratch %d of %d bytes"
            % (nbytes, leaf, need, rp.REPOPS_NOALLOC_SCRATCH_BYTES))
        assert need <= rp.REPOPS_NOALLOC_SCRATCH_BYTES
        host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
        data = torch.from_numpy(host).to(dev) if nbytes else torch.empty(16, dtype=torch.uint8,
                                                                           device=dev)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        root_ws = torch.zeros(32, dtype=torch.uint8, device=dev)
        root_na = torch.full((32,), 0xAB, dtype=torch.uint8, device=dev)
        st = rp.repops_merkle_root(data.data_ptr(), nbytes, leaf, ws.data_ptr(), need,
                                   root_ws.data_ptr(), stream.cuda_stream)
        assert st == rp.REPOPS_OK, rp.repops_strerror(st)
        st = rp.repops_merkle_root_noalloc(data.data_ptr(), nbytes, leaf, root_na.data_ptr(),
                                           stream.cuda_stream)
        assert st == rp.REPOPS_OK, rp.repops_strerror(st)
        torch.cuda.synchronize()
        a, b = bytes(root_ws.cpu().numpy()), bytes(root_na.cpu().numpy())
        assert a == b, (nbytes, leaf, a.hex(), b.hex())
        if with_oracle:
            assert b == merkle.merkle_root(host.tobytes(), leaf), (nbytes, leaf)
        say("root %s equal" % b.hex())
        del data, ws
