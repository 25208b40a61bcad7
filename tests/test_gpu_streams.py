"""GPU parity of the stream-mixed scan (shared A; the experts' B X injections
and C readouts mixed by the router weights) against the fp64 oracle on the
same seeded inputs, through the C ABI.

Bars as for the parameter-mixed scan: y and final state within rel 1e-4
(fp32 inputs) or 2e-3 (bf16 inputs, fp32 arithmetic); bf16 y faithfully
rounded.  Full-size shapes run in the benchmark's launch configuration and
are compared on sampled channels (every (b, d) recurrence is independent)."""
import functools

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, HipEvents, assert_faithful_bf16, host, rel_err
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
STREAM_KEYS = ("X", "dt_raw", "Bs", "Cs")


def to_dev(inp, dtype):
    out = {}
    for k_, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k_ in STREAM_KEYS and dtype == "bf16":
            t = t.to(torch.bfloat16)  # values are already bf16-representable
        out[k_] = t.to(DEV)
    return out


def case(B, L, D, k=2, dtype="f32", seed=0, h0=False):
    w = workloads.Workload("streams", B=B, L=L, D=D, N=16, E=k, k=k, dtype=dtype, seed=seed)
    inp = workloads.generate_streams(w)
    if h0:
        inp["h0"] = np.random.default_rng(seed + 7).standard_normal((B, D, 16)).astype(np.float32)
    return w, inp, to_dev(inp, dtype)


@functools.lru_cache(maxsize=1)
def full_case(name, k):
    w = workloads.BY_NAME[name]
    inp = workloads.generate_streams(w, k=k)
    return w, inp, to_dev(inp, w.dtype)


def args(t):
    return (t["X"], t["dt_raw"], t["Bs"], t["Cs"], t["gate"], t["A"], t["dt_bias"])


def ref(inp, dsel=None, h0=None):
    sl = slice(None) if dsel is None else dsel
    if h0 is not None:
        h0 = h0[:, sl]
    return oracle.scan_streams(inp["X"][..., sl], inp["dt_raw"][..., sl], inp["Bs"], inp["Cs"],
                               inp["gate"], inp["A"][sl], inp["dt_bias"][sl], h0=h0)


@pytest.mark.parametrize("carry", ["fixup", "rewalk"])
@pytest.mark.parametrize("chunk", [0, 16, 64, 100, 256])
@pytest.mark.parametrize("with_h0", [False, True])
def test_streams_tiny(chunk, carry, with_h0):
    """One tile, one to sixteen chunks (a ragged last one for 100), both
    chunk joins, with and without an initial state."""
    w, inp, t = case(B=1, L=256, D=64, k=2, seed=1, h0=with_h0)
    y, hf = swimba.scan_streams(*args(t), h0=t.get("h0"), chunk=chunk, carry=carry)
    ry, rh = ref(inp, h0=inp.get("h0"))
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32, rel_err(host(hf), rh)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("chunk", [0, 64])
def test_streams_slot_counts(k, chunk):
    """Every compiled slot count, several tiles plus a ragged tail (D = 130),
    a sequence that is not a whole number of chunks or staging blocks."""
    w, inp, t = case(B=2, L=301, D=130, k=k, seed=10 + k, h0=True)
    y, hf = swimba.scan_streams(*args(t), h0=t["h0"], chunk=chunk)
    ry, rh = ref(inp, h0=inp["h0"])
    assert rel_err(host(y), ry) < TOL_F32, (k, chunk, rel_err(host(y), ry))
    assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("chunk", [0, 77, 128, 700])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_streams_ragged_bf16(chunk, ydt):
    """bf16 streams, fp32 or bf16 y, ragged D (200) and ragged chunks."""
    w, inp, t = case(B=2, L=700, D=200, k=2, dtype="bf16", seed=3, h0=True)
    ydtype = torch.float32 if ydt == "f32" else torch.bfloat16
    y, hf = swimba.scan_streams(*args(t), h0=t["h0"], chunk=chunk, y_dtype=ydtype)
    ry, rh = ref(inp, h0=inp["h0"])
    if ydt == "f32":
        assert rel_err(host(y), ry) < TOL_BF16, rel_err(host(y), ry)
    else:
        assert_faithful_bf16(y, ry, "y")
    assert rel_err(host(hf), rh) < TOL_BF16


def test_streams_fp32_in_bf16_out():
    w, inp, t = case(B=1, L=333, D=96, k=3, seed=4)
    y, hf = swimba.scan_streams(*args(t), y_dtype=torch.bfloat16, chunk=50)
    ry, rh = ref(inp)
    assert_faithful_bf16(y, ry, "y")
    assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("k", [1, 2])
def test_streams_full_size_sampled(k):
    """The 130M-like layer shape (B=4, L=2048, D=1536, bf16) in the launch
    configuration the benchmark times; 24 sampled channels vs the oracle."""
    w, inp, t = full_case("mamba130m_layer", k)
    rng = np.random.default_rng(2)
    dsel = np.sort(rng.choice(w.D, 24, replace=False))
    ry, rh = ref(inp, dsel=dsel)
    for ydtype in (torch.bfloat16, torch.float32):
        y, hf = swimba.scan_streams(*args(t), y_dtype=ydtype)
        ys = y[:, :, torch.from_numpy(dsel).to(DEV)]
        if ydtype == torch.float32:
            assert rel_err(host(ys), ry) < TOL_BF16, rel_err(host(ys), ry)
        else:
            assert_faithful_bf16(ys, ry, "y")
        assert rel_err(host(hf)[:, dsel], rh) < TOL_BF16
        del y, hf


def test_streams_chunking_and_carry_agree():
    """Chunk size and the carry method change rounding only."""
    w, inp, t = case(B=1, L=2048, D=128, k=2, dtype="bf16", seed=5)
    ry, _ = ref(inp)
    outs = []
    for chunk in (0, 32, 256, 2048):
        for carry in ("fixup", "rewalk"):
            y, _ = swimba.scan_streams(*args(t), chunk=chunk, carry=carry, y_dtype=torch.float32)
            assert rel_err(host(y), ry) < TOL_BF16
            outs.append(host(y))
    for o in outs[1:]:
        assert rel_err(o, outs[0]) < 1e-4


def test_streams_degenerate_shapes():
    # L = 0: h_final = h0 (or zeros); B = 0: nothing to do
    w, inp, t = case(B=2, L=0, D=70, k=2, h0=True)
    y, hf = swimba.scan_streams(*args(t), h0=t["h0"])
    assert torch.equal(hf, t["h0"])
    y, hf = swimba.scan_streams(*args(t))
    assert torch.count_nonzero(hf) == 0
    w, inp, t = case(B=0, L=10, D=70, k=2)
    y, hf = swimba.scan_streams(*args(t))
    assert y.shape == (0, 10, 70)
    # L = 1, D = 1, one token per chunk
    for (B, L, D) in ((1, 1, 64), (3, 5, 1), (1, 130, 1)):
        w, inp, t = case(B=B, L=L, D=D, k=2, seed=B + L + D)
        for chunk in (0, 1, 2):
            y, hf = swimba.scan_streams(*args(t), chunk=chunk)
            ry, rh = ref(inp)
            assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_streams_zero_gate_slot():
    """A slot with weight zero contributes nothing, whatever its streams."""
    w, inp, t = case(B=1, L=200, D=64, k=3, seed=6)
    gate = inp["gate"].copy()
    gate[:, :, 1] = 0.0
    X = inp["X"].copy()
    X[:, :, 1] = 1e30  # huge but finite: 0 * value = 0
    t["gate"] = torch.from_numpy(gate).to(DEV)
    t["X"] = torch.from_numpy(X).to(DEV)
    y, hf = swimba.scan_streams(*args(t), chunk=64)
    keep = [0, 2]
    ry, rh = oracle.scan_streams(X[:, :, keep], inp["dt_raw"], inp["Bs"][:, :, keep],
                                 inp["Cs"][:, :, keep], gate[:, :, keep], inp["A"],
                                 inp["dt_bias"])
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_streams_noncontractive_falls_back_to_rewalk():
    """A >= 0 somewhere: no contraction, so the fix-up recomputes whole chunks."""
    w, inp, t = case(B=1, L=600, D=64, k=2, seed=7)
    A = inp["A"].copy()
    A[5, 3] = 0.02
    inp["A"] = A
    t["A"] = torch.from_numpy(A).to(DEV)
    y, hf = swimba.scan_streams(*args(t), chunk=64)
    ry, rh = ref(inp)
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32


def test_streams_split_composition():
    w, inp, t = case(B=2, L=1000, D=96, k=2, dtype="bf16", seed=8)
    y, hf = swimba.scan_streams(*args(t), y_dtype=torch.float32)
    cut = 377
    a = args(t)
    a1 = [v[:, :cut].contiguous() for v in a[:5]] + list(a[5:])
    a2 = [v[:, cut:].contiguous() for v in a[:5]] + list(a[5:])
    y1, h1 = swimba.scan_streams(*a1, y_dtype=torch.float32)
    y2, h2 = swimba.scan_streams(*a2, h0=h1, y_dtype=torch.float32)
    assert rel_err(host(torch.cat([y1, y2], 1)), host(y)) < 1e-4
    assert rel_err(host(h2), host(hf)) < 1e-4


def test_streams_deterministic_and_prepared():
    w, inp, t = full_case("mamba130m_layer", 2)
    y1, h1 = swimba.scan_streams(*args(t))
    y2, h2 = swimba.scan_streams(*args(t))
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    y3 = torch.empty_like(y1)
    h3 = torch.empty_like(h1)
    call = swimba.PreparedStreams(*args(t), y=y3, h_final=h3)
    call()
    torch.cuda.synchronize()
    assert torch.equal(y1, y3) and torch.equal(h1, h3)


@pytest.mark.parametrize("chunk", [0, 64])
def test_streams_phase_events(chunk):
    w, inp, t = case(B=2, L=300, D=128, k=2, dtype="bf16", seed=9)
    y0, h0_ = swimba.scan_streams(*args(t), chunk=chunk)
    ev = HipEvents(6)
    try:
        y1, h1 = swimba.scan_streams(*args(t), chunk=chunk, phase_events=ev.address)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(h0_, h1)
        for i in range(5):
            assert ev.ms(i, i + 1) >= 0.0
        assert ev.ms(0, 1) > 0.0
        if chunk:
            assert ev.ms(4, 5) > 0.0
    finally:
        ev.close()


def test_streams_constant_inputs_closed_form_at_length():
    """L = 65536, constant streams and gates: h_t = u (1 - a^t) / (1 - a)
    pins every chunk boundary of the carry without the oracle."""
    B, L, D, N, k = 1, 65536, 64, 16, 2
    rng = np.random.default_rng(43)
    Xv = rng.uniform(0.5, 1.0, (k, D)).astype(np.float32)
    rv = np.full(D, -6.0, np.float32)                       # Delta ~ 2.5e-3
    Bv = rng.uniform(0.5, 1.0, (k, N)).astype(np.float32)
    Cv = rng.uniform(-1.0, 1.0, (k, N)).astype(np.float32)
    A = -rng.uniform(0.3, 0.6, (D, N)).astype(np.float32)
    bias = np.zeros(D, np.float32)
    g = np.array([0.7, 0.3], np.float32)
    X = torch.from_numpy(np.broadcast_to(Xv, (B, L, k, D)).copy()).to(DEV)
    dt = torch.from_numpy(np.broadcast_to(rv, (B, L, D)).copy()).to(DEV)
    Bs = torch.from_numpy(np.broadcast_to(Bv, (B, L, k, N)).copy()).to(DEV)
    Cs = torch.from_numpy(np.broadcast_to(Cv, (B, L, k, N)).copy()).to(DEV)
    gate = torch.from_numpy(np.broadcast_to(g, (B, L, k)).copy()).to(DEV)
    y, hf = swimba.scan_streams(X, dt, Bs, Cs, gate, torch.from_numpy(A).to(DEV),
                                torch.from_numpy(bias).to(DEV), chunk=256)
    Dt = np.log1p(np.exp(rv.astype(np.float64)))
    a = np.exp(Dt[:, None] * A.astype(np.float64))                          # [D, N]
    u = Dt[:, None] * (g[0] * Xv[0][:, None] * Bv[0][None] + g[1] * Xv[1][:, None] * Bv[1][None])
    c = g[0] * Cv[0].astype(np.float64) + g[1] * Cv[1]
    ts = np.array([1, 255, 256, 257, 4096, 30000, 65535, 65536])
    h = u[None] * (1 - a[None] ** ts[:, None, None]) / (1 - a[None])       # [T, D, N]
    want = h @ c
    got = host(y)[0, ts - 1]
    assert rel_err(got, want) < 2e-3, rel_err(got, want)
    assert rel_err(host(hf)[0], h[-1]) < 2e-3
