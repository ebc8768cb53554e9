"""GPU parity at the largest sizes the entry points are built for: an output
with more than 2^31 elements (64-bit offsets in every kernel's epilogue),
a very long fixed-order sum (K = 2^17 + 3), a LayerNorm row of 2^20 + 5
elements, and LayerNorm launches with more row groups than workgroups, all
against the CPU oracle bit for bit (the huge outputs on sampled entries,
read back on the device)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bit_reproducible_fp32_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_reproducible_fp32_amd as rp  # noqa: E402

DEV = "cuda:0"


def say(msg):
    print("[gpu-max] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def same_bits(x, y, what=""):
    x = np.ascontiguousarray(x, np.float32).view(np.uint32)
    y = np.ascontiguousarray(y, np.float32).view(np.uint32)
    bad = np.flatnonzero(x.reshape(-1) != y.reshape(-1))
    assert bad.size == 0, "%s: %d differ, first at %d" % (what, bad.size, bad[0])


def test_output_beyond_2_pow_31_elements():
    """C of 65536 x 32770 (2147614720 elements, 8.6 GB): entries past
    element 2^31 are written at the right place by the automatic variant, a
    VALU variant and the naive kernel."""
    M, N, K = 65536, 32770, 3
    assert M * N > 2 ** 31
    A = inputs.random_matrix((M, K), 61)
    B = inputs.random_matrix((K, N), 62)
    ii, jj = inputs.sample_entries(M, N, 2048, 63)
    ii = np.concatenate([ii, [M - 1, M - 1, 65535 - 1], np.full(64, 65535)])
    jj = np.concatenate([jj, [N - 1, N - 2, N - 1], np.arange(N - 64, N)])
    want = oracle.entries_f32(A, B, ii, jj)
    ga, gb = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    out = torch.empty((M, N), device=DEV)
    it = torch.from_numpy(ii).to(DEV)
    jt = torch.from_numpy(jj).to(DEV)
    names = rp.variant_names()
    for v in (None, names.index("valu_t128x128x16_r8x8_xcd"), names.index("naive_lane_per_output")):
        say("C > 2^31 elements, variant %s" % (v if v is None else names[v]))
        out.fill_(float("nan"))
        rp.matmul(ga, gb, out=out, variant=v)
        got = out[it, jt].cpu().numpy()
        same_bits(got, want, "variant %s" % v)
    del out
    torch.cuda.empty_cache()


def test_long_fixed_order_sum():
    M, N, K = 37, 41, (1 << 17) + 3
    say("K = %d, every variant" % K)
    A = inputs.random_matrix((M, K), 71)
    B = inputs.random_matrix((K, N), 72, "normal0.02")
    want = oracle.matmul_f32(A, B)
    ga, gb = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    for v in range(rp.repops_variant_count()):
        same_bits(rp.matmul(ga, gb, variant=v).cpu().numpy(), want, rp.repops_variant_name(v))


def test_layernorm_long_row():
    rows, H = 3, (1 << 20) + 5
    say("LayerNorm rows=%d H=%d" % (rows, H))
    x = (inputs.random_matrix((rows, H), 81) * np.float32(3)).astype(np.float32)
    g = inputs.random_matrix((H,), 82)
    b = inputs.random_matrix((H,), 83)
    want = oracle.layernorm_f32(x, g, b, 1e-5)
    y, mean, rstd = rp.layernorm(torch.from_numpy(x).to(DEV), torch.from_numpy(g).to(DEV),
                                 torch.from_numpy(b).to(DEV), 1e-5, return_stats=True)
    same_bits(y.cpu().numpy(), want[0], "y")
    same_bits(mean.cpu().numpy(), want[1], "mean")
    same_bits(rstd.cpu().numpy(), want[2], "rstd")


@pytest.mark.parametrize("rows,H", [((1 << 24) + 5, 8), ((1 << 22) + 3, 776)])
def test_layernorm_more_row_groups_than_workgroups(rows, H):
    """More row groups than the 2^20 workgroups a register-form launch uses
    (16 rows per group at H = 8, 4 at H = 776), so workgroups take a second
    group; sampled rows (first, last, around the wrap) against the oracle."""
    say("LayerNorm rows=%d H=%d (grid-stride)" % (rows, H))
    gen = torch.Generator(device=DEV).manual_seed(91 + H)
    x = torch.randn(rows, H, device=DEV, generator=gen) * 2 + 0.25
    g = torch.from_numpy(inputs.random_matrix((H,), 92)).to(DEV)
    b = torch.from_numpy(inputs.random_matrix((H,), 93)).to(DEV)
    y, mean, rstd = rp.layernorm(x, g, b, 1e-5, return_stats=True)
    per = 16 if H <= 768 else 4
    wrap = (1 << 20) * per
    pick = np.unique(np.r_[0, 1, per - 1, per, wrap - 1, wrap, wrap + 1, rows - per - 1,
                           rows - 2, rows - 1,
                           np.random.default_rng(94).integers(0, rows, 48)])
    it = torch.from_numpy(pick).to(DEV)
    xs = x[it].cpu().numpy()
    want = oracle.layernorm_f32(xs, g.cpu().numpy(), b.cpu().numpy(), 1e-5)
    same_bits(y[it].cpu().numpy(), want[0], "y")
    same_bits(mean[it].cpu().numpy(), want[1], "mean")
    same_bits(rstd[it].cpu().numpy(), want[2], "rstd")
    del x, y
    torch.cuda.empty_cache()
