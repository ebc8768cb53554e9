"""GPU parity of ERF, GeLU and LayerNorm (repops_erf_f32, repops_gelu_f32,
repops_layernorm_f32 through the C ABI) against the CPU oracle, bit for bit
(NaN as a class).

Covered: hand-picked and random inputs with tiny, subnormal, huge and special
values; a sweep of 2^24 bit patterns spread over every exponent; lengths 0 to
2^20 + 3 on the 16-byte and the element-wise paths; in-place calls;
LayerNorm for H from 1 to 8193 (both sides of every kernel form's limit) and
1 to 4099 rows, with and without gamma and beta, strided and misaligned rows, in place, rows whose variance is subnormal
or zero and rows holding infinities and NaN; and the full DistilBERT-shaped
workloads the benchmark times, compared in full."""
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
    print("[gpu-ops] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def same_bits(x, y, what=""):
    x = np.asarray(x, np.float32)
    y = np.asarray(y, np.float32)
    assert x.shape == y.shape, what
    nx, ny = np.isnan(x), np.isnan(y)
    assert np.array_equal(nx, ny), "%s: NaN positions differ" % what
    xb = np.where(nx, 0, x).view(np.uint32).reshape(-1)
    yb = np.where(ny, 0, y).view(np.uint32).reshape(-1)
    bad = np.flatnonzero(xb != yb)
    assert bad.size == 0, "%s: %d differ, first at %d: %08x vs %08x" % (
        what, bad.size, bad[0], xb[bad[0]], yb[bad[0]])


def placed(x: np.ndarray, offset=0):
    """x copied into a fresh device buffer `offset` floats in."""
    buf = torch.zeros(x.size + offset + 4, device=DEV)
    v = buf[offset:offset + x.size]
    v.copy_(torch.from_numpy(np.ascontiguousarray(x, np.float32).reshape(-1)))
    return v


def mixed_values(n, seed):
    rng = np.random.default_rng(seed)
    vals = [rng.standard_normal(n).astype(np.float32) * 3,
            rng.uniform(-1.2, 1.2, n).astype(np.float32),
            (rng.uniform(0.5, 1.5, n) * np.float32(2.0) ** rng.integers(-149, 20, n)
             * rng.choice([-1, 1], n)).astype(np.float32),
            np.array([0.0, -0.0, 1.0, -1.0, 0.99999994, -0.99999994, 1.0000001, 5.6, 5.7,
                      12.0, -30.0, 1e-45, -1e-40, 3.4e38, -3.4e38, np.inf, -np.inf, np.nan],
                     np.float32)]
    return np.concatenate(vals)


OPS = {"erf": (rp.repops_erf_f32, oracle.erf_f32), "gelu": (rp.repops_gelu_f32, oracle.gelu_f32)}


def run_unary(name, x, offset=0, in_place=False):
    fn, _ = OPS[name]
    src = placed(x, offset)
    dst = src if in_place else placed(np.zeros_like(x), offset)
    st = fn(src.data_ptr(), dst.data_ptr(), x.size, torch.cuda.current_stream().cuda_stream)
    assert st == rp.REPOPS_OK, rp.repops_strerror(st)
    torch.cuda.synchronize()
    return dst.cpu().numpy()


@pytest.mark.parametrize("name", sorted(OPS))
@pytest.mark.parametrize("offset", [0, 1])
def test_unary_mixed_values(name, offset):
    say("%s mixed values, offset %d" % (name, offset))
    x = mixed_values(5000, 11)
    same_bits(run_unary(name, x, offset), OPS[name][1](x), name)


@pytest.mark.parametrize("name", sorted(OPS))
def test_unary_bit_pattern_sweep(name):
    """Every 256th binary32 bit pattern (plus a seeded offset): all exponents,
    signs, subnormals, infinities and NaNs."""
    say("%s bit-pattern sweep" % name)
    bits = (np.arange(1 << 24, dtype=np.uint64) * 256 + 97).astype(np.uint32)
    x = bits.view(np.float32)
    with np.errstate(all="ignore"):
        same_bits(run_unary(name, x), OPS[name][1](x), name)


@pytest.mark.parametrize("name", sorted(OPS))
@pytest.mark.parametrize("n", [1, 3, 4, 5, 255, 1023, 4096 + 7, (1 << 20) + 3])
def test_unary_lengths(name, n):
    say("%s n=%d" % (name, n))
    x = inputs.random_matrix((n,), 100 + n, "normal1") * np.float32(2.5)
    same_bits(run_unary(name, x, offset=n % 2), OPS[name][1](x), name)


@pytest.mark.parametrize("name", sorted(OPS))
def test_unary_in_place_and_empty(name):
    say("%s in place" % name)
    x = mixed_values(700, 12)
    same_bits(run_unary(name, x, in_place=True), OPS[name][1](x), name)
    fn, _ = OPS[name]
    assert fn(0, 0, 0, 0) == rp.REPOPS_OK


def test_torch_wrappers():
    say("torch wrappers")
    x = mixed_values(300, 13)[:280].reshape(40, 7)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    same_bits(rp.erf(t).cpu().numpy(), oracle.erf_f32(x))
    same_bits(rp.gelu(t).cpu().numpy(), oracle.gelu_f32(x))


# -- LayerNorm ------------------------------------------------------------------------
def gpu_layernorm(x, gamma, beta, eps, x_rs=None, offset=0, in_place=False):
    rows, H = x.shape
    x_rs = H if x_rs is None else x_rs
    wide = np.zeros((rows, x_rs), np.float32)
    wide[:, :H] = x
    xd = placed(wide, offset)
    yd = xd if in_place else placed(np.zeros((rows, x_rs), np.float32), offset)
    g = placed(gamma) if gamma is not None else None
    b = placed(beta) if beta is not None else None
    mean = torch.empty(rows, device=DEV)
    rstd = torch.empty(rows, device=DEV)
    st = rp.repops_layernorm_f32(xd.data_ptr(), x_rs, g.data_ptr() if g is not None else None,
                                 b.data_ptr() if b is not None else None, yd.data_ptr(), x_rs,
                                 rows, H, float(np.float32(eps)), mean.data_ptr(),
                                 rstd.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == rp.REPOPS_OK, rp.repops_strerror(st)
    torch.cuda.synchronize()
    y = yd.cpu().numpy().reshape(rows, x_rs)[:, :H]
    return y, mean.cpu().numpy(), rstd.cpu().numpy()


def check_layernorm(x, gamma, beta, eps, **kw):
    got = gpu_layernorm(x, gamma, beta, eps, **kw)
    want = oracle.layernorm_f32(x, gamma, beta, eps)
    for g, w, what in zip(got, want, ("y", "mean", "rstd")):
        same_bits(g, w, what)


@pytest.mark.parametrize("rows,H", [(1, 1), (3, 2), (5, 3), (64, 4), (65, 5), (17, 63),
                                    (31, 256), (16, 257), (33, 512), (47, 513), (63, 768),
                                    (18, 767), (19, 769), (130, 1023), (5, 1024), (6, 1025),
                                    (7, 1536), (9, 1537), (7, 2044), (9, 2048), (10, 2049),
                                    (5, 3072), (6, 3073), (7, 4096), (3, 4097), (5, 6144),
                                    (6, 6145), (7, 8192), (3, 8193), (4099, 8)])
def test_layernorm_shapes(rows, H):
    say("layernorm rows=%d H=%d" % (rows, H))
    rng = np.random.default_rng(rows * 31 + H)
    x = (rng.standard_normal((rows, H)) * rng.uniform(0.1, 10) + rng.uniform(-5, 5)
         ).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    b = (0.1 * rng.standard_normal(H)).astype(np.float32)
    check_layernorm(x, g, b, 1e-5)
    check_layernorm(x, None, None, 1e-12)
    check_layernorm(x, g, None, 0.5)


# Rows over 2048 keep their first chunks on chip: up to 4096 ten chunks of
# 256 elements (five in LDS, five in registers; the first eight need no bounds
# test), above that three of 512.  Lengths on both sides of each edge, with
# partly filled row groups, in place, and through the scalar-load form (H odd).
@pytest.mark.parametrize("rows,H", [(13, 2052), (6, 2300), (7, 2304), (9, 2308), (5, 2556),
                                    (11, 2560), (6, 2564), (10, 4092), (7, 4100), (9, 4104),
                                    (5, 4608), (6, 5124), (5, 2305), (6, 4099)])
def test_layernorm_stream_kept_chunks(rows, H):
    say("layernorm kept chunks rows=%d H=%d" % (rows, H))
    rng = np.random.default_rng(rows * 7 + H)
    x = (rng.standard_normal((rows, H)) * 3 + 1).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    b = (0.1 * rng.standard_normal(H)).astype(np.float32)
    check_layernorm(x, g, b, 1e-5)
    check_layernorm(x, None, b, 1e-6)
    check_layernorm(x, g, b, 1e-5, in_place=True)


@pytest.mark.parametrize("H,x_rs,offset", [(768, 772, 0), (768, 771, 0), (768, 768, 1),
                                          (768, 1000, 3), (1024, 1030, 0), (1024, 1027, 2),
                                          (2500, 2600, 0), (4096, 4100, 1), (6000, 6004, 0),
                                          (8192, 8200, 3)])
def test_layernorm_strided_and_misaligned(H, x_rs, offset):
    say("layernorm H=%d x_rs=%d offset=%d" % (H, x_rs, offset))
    rng = np.random.default_rng(x_rs + offset)
    x = rng.standard_normal((70, H)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    b = (0.1 * rng.standard_normal(H)).astype(np.float32)
    check_layernorm(x, g, b, 1e-12, x_rs=x_rs, offset=offset)


@pytest.mark.parametrize("H", [96, 1024, 3000, 7000])
def test_layernorm_in_place(H):
    say("layernorm in place H=%d" % H)
    rng = np.random.default_rng(5 + H)
    x = rng.standard_normal((37, H)).astype(np.float32)
    g = rng.standard_normal(H).astype(np.float32)
    b = rng.standard_normal(H).astype(np.float32)
    check_layernorm(x, g, b, 1e-5, in_place=True)


@pytest.mark.parametrize("H", [33, 1500, 5000])
def test_layernorm_extreme_rows(H):
    say("layernorm extreme rows H=%d" % H)
    rows = [np.full(H, 7.5), np.zeros(H), np.full(H, -0.0),
            np.linspace(-1e-30, 1e-30, H),           # subnormal variance
            np.linspace(-1e-21, 1e-21, H),
            np.linspace(-3e19, 3e19, H),             # the squared deviations overflow
            np.r_[np.ones(H - 1), np.inf], np.r_[np.ones(H - 1), np.nan],
            np.r_[1e-45, np.zeros(H - 1)]]
    x = np.array(rows, dtype=np.float32)
    g = np.linspace(-3, 3, H).astype(np.float32)
    b = np.linspace(1, 2, H).astype(np.float32)
    with np.errstate(all="ignore"):
        for eps in (0.0, 1e-12, 1e-5):
            check_layernorm(x, g, b, eps)
            check_layernorm(x, None, None, eps)


def test_layernorm_random_configurations():
    """40 seeded random configurations across every kernel form: H log-uniform
    in [1, 20000], 1 to 300 rows, padded row strides, misaligned starts,
    gamma and beta present or not, four eps values."""
    rng = np.random.default_rng(2024)
    for case in range(40):
        H = int(np.exp(rng.uniform(0, np.log(20000))))
        rows = int(rng.integers(1, 301))
        rows = max(1, min(rows, 1_500_000 // max(H, 1)))
        pad = int(rng.integers(0, 8)) if rng.random() < 0.5 else 0
        offset = int(rng.integers(0, 4)) if rng.random() < 0.5 else 0
        eps = float(rng.choice([0.0, 1e-12, 1e-5, 0.5]))
        x = (rng.standard_normal((rows, H)) * rng.uniform(0.01, 100) + rng.uniform(-10, 10)
             ).astype(np.float32)
        g = rng.standard_normal(H).astype(np.float32) if rng.random() < 0.7 else None
        b = rng.standard_normal(H).astype(np.float32) if rng.random() < 0.7 else None
        say("layernorm random case %d: rows=%d H=%d pad=%d offset=%d gamma=%s beta=%s eps=%g"
            % (case, rows, H, pad, offset, g is not None, b is not None, eps))
        check_layernorm(x, g, b, eps, x_rs=H + pad, offset=offset)


def test_layernorm_torch_wrapper():
    say("layernorm torch wrapper")
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 10, 48)).astype(np.float32)
    g = rng.standard_normal(48).astype(np.float32)
    b = rng.standard_normal(48).astype(np.float32)
    y, mean, rstd = rp.layernorm(torch.from_numpy(x).to(DEV), torch.from_numpy(g).to(DEV),
                                 torch.from_numpy(b).to(DEV), 1e-5, return_stats=True)
    want = oracle.layernorm_f32(x.reshape(-1, 48), g, b, 1e-5)
    same_bits(y.cpu().numpy().reshape(-1, 48), want[0])
    same_bits(mean.cpu().numpy(), want[1])
    same_bits(rstd.cpu().numpy(), want[2])


@pytest.mark.parametrize("name", sorted(inputs.OPS_WORKLOADS))
def test_full_size_workload(name):
    """The benchmark's workloads, in its launch configuration, compared in full."""
    w = inputs.OPS_WORKLOADS[name]
    say("full size %s" % name)
    x, g, b = inputs.make_ops_operands(name)
    xt = torch.from_numpy(x).to(DEV)
    if w.op == "layernorm":
        y, mean, rstd = rp.layernorm(xt, torch.from_numpy(g).to(DEV),
                                     torch.from_numpy(b).to(DEV), w.eps, return_stats=True)
        want = oracle.layernorm_f32(x, g, b, w.eps)
        same_bits(y.cpu().numpy(), want[0], "y")
        same_bits(mean.cpu().numpy(), want[1], "mean")
        same_bits(rstd.cpu().numpy(), want[2], "rstd")
    else:
        y = (rp.erf if w.op == "erf" else rp.gelu)(xt)
        same_bits(y.cpu().numpy(), (oracle.erf_f32 if w.op == "erf" else oracle.gelu_f32)(x))
