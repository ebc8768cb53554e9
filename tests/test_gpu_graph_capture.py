"""GPU: the whole hot path recorded once as a HIP graph and replayed.

Every entry point of the library only launches kernels on the caller's
stream. None allocates, sets memory or synchronises, so a caller can record
them on a capturing stream (torch.cuda.graph) and replay the graph. One graph
here holds, on one stream:
- a ragged multi-tile matmul;
- a batched Q·Kᵀ with a bias;
- the fold and SGD step;
- ERF and GeLU;
- LayerNorm with gamma and beta;
- the multi-launch tensor hash of the matmul's output.

Between replays, eager work overwrites every output and the stream is
synchronised. Each replay must reproduce the eager results bit for bit, and
those equal the oracle's. A replay after new values are copied into the
input buffers must give the oracle's results for the new values."""
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
LEAF = 256  # bytes: the 312,000-byte matmul output spans 1219 leaves, three launches


def say(msg):
    print("[gpu-graph] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rp.load()
    yield


def host_inputs(seed):
    def r(shape, s, dist="normal1"):
        return inputs.random_matrix(shape, seed + s, dist)

    return {
        "A": r((300, 77), 1), "B": r((77, 260), 2),
        "Q": r((3, 33, 64), 3), "Kh": r((3, 47, 64), 4), "bias": r((3, 47), 5),
        "g0": r((1000,), 10), "g1": r((1000,), 11), "g2": r((1000,), 12),
        "theta": r((1000,), 20), "x": (r((5000,), 30) * np.float32(3)).astype(np.float32),
        "ln": r((37, 1000), 40), "gamma": r((1000,), 41), "beta": r((1000,), 42),
    }


ETA = np.float32(0.01)


def expected(h):
    """The oracle's results for host inputs h."""
    C = oracle.matmul_f32(h["A"], h["B"])
    theta, gbar = oracle.fold_mean_sgd_f32([h["g0"], h["g1"], h["g2"]], ETA, h["theta"])
    return {
        "C": C,
        "S": oracle.matmul_batched_f32(h["Q"], h["Kh"], trans_b=True, bias=h["bias"]),
        "theta": theta, "gbar": gbar,
        "erf": oracle.erf_f32(h["x"]), "gelu": oracle.gelu_f32(h["x"]),
        "y": oracle.layernorm_f32(h["ln"], h["gamma"], h["beta"])[0],
        "root": np.frombuffer(merkle.tensor_root(C, LEAF), np.uint8),
    }


def same_bits(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, what
    g = got.view(np.uint32) if got.dtype == np.float32 else got
    w = want.view(np.uint32) if want.dtype == np.float32 else want
    bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
    assert bad.size == 0, "%s: %d elements differ, first at %d" % (what, bad.size, bad[0])


class Buffers:
    """Device buffers that stay at fixed addresses for the graph's life."""

    def __init__(self, h):
        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)

        self.inp = {k: dev(v) for k, v in h.items()}
        self.theta0 = self.inp["theta"].clone()
        self.C = torch.empty((300, 260), device=DEV)
        self.S = torch.empty((3, 33, 47), device=DEV)
        self.gbar = torch.empty(1000, device=DEV)
        self.erf = torch.empty(5000, device=DEV)
        self.gelu = torch.empty(5000, device=DEV)
        self.y = torch.empty((37, 1000), device=DEV)
        self.root = torch.empty(32, dtype=torch.uint8, device=DEV)
        need = rp.repops_merkle_workspace_bytes(self.C.numel() * 4, LEAF)
        assert need > 0
        self.ws = torch.empty(need, dtype=torch.uint8, device=DEV)

    def run(self):
        """The hot path, launched on the current stream, allocating nothing."""
        i = self.inp
        rp.matmul(i["A"], i["B"], out=self.C)
        rp.matmul_batched(i["Q"], i["Kh"], trans_b=True, bias=i["bias"], out=self.S)
        rp.fold_mean_sgd([i["g0"], i["g1"], i["g2"]], i["theta"], float(ETA), gbar=self.gbar)
        rp.erf(i["x"], out=self.erf)
        rp.gelu(i["x"], out=self.gelu)
        rp.layernorm(i["ln"], i["gamma"], i["beta"], out=self.y)
        rp.merkle_root(self.C, leaf_bytes=LEAF, out=self.root, workspace=self.ws)

    def outputs(self):
        return {"C": self.C, "S": self.S, "theta": self.inp["theta"], "gbar": self.gbar,
                "erf": self.erf, "gelu": self.gelu, "y": self.y, "root": self.root}

    def scribble(self):
        """Eager work between replays: every output overwritten, theta reset."""
        for k, t in self.outputs().items():
            if k == "theta":
                t.copy_(self.theta0)
            elif t.dtype == torch.uint8:
                t.fill_(0xA5)
            else:
                t.fill_(float("nan"))
        torch.cuda.synchronize()


def snapshot(buf):
    torch.cuda.synchronize()
    return {k: t.cpu().numpy().copy() for k, t in buf.outputs().items()}


def check(got, want, label):
    for k in want:
        same_bits(got[k], want[k], "%s: %s" % (label, k))


def test_hot_path_in_one_graph_replays_bit_exactly():
    h = host_inputs(7000)
    want = expected(h)
    buf = Buffers(h)

    say("eager run on a side stream")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        buf.run()
    torch.cuda.current_stream().wait_stream(side)
    eager = snapshot(buf)
    check(eager, want, "eager")

    say("capture")
    buf.scribble()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        buf.run()
    torch.cuda.synchronize()

    for rep in range(3):
        say("replay %d" % rep)
        buf.scribble()
        g.replay()
        check(snapshot(buf), eager, "replay %d" % rep)

    say("replay on new input values")
    h2 = host_inputs(7100)
    for k, v in h2.items():
        buf.inp[k].copy_(torch.from_numpy(np.ascontiguousarray(v)))
    buf.theta0.copy_(buf.inp["theta"])
    buf.scribble()
    g.replay()
    check(snapshot(buf), expected(h2), "replay on new inputs")
    del g
    torch.cuda.synchronize()
