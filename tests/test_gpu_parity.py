"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bars: router idx bit-exact wherever the fp32 ranking is certain (certified
near-ties may order either way, and must be consistent with the tolerance);
gates within the bound implied by the logit error; y and final state within
rel 1e-4 (fp32 inputs) or 2e-3 (bf16 inputs, fp32 accumulation), bf16 y
faithfully rounded.  The scan comparisons feed the GPU router's idx/gate to
the oracle so that they do not depend on router rounding.  Full-size
workloads run in the launch configuration the benchmark times and are
compared on sampled channels (every (b, d) recurrence is independent)."""
import functools
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL_BF16, TOL_F32, HipEvents, assert_faithful_bf16, check_route,
                         dev_tensors, gate_bound, host, rel_err, route_tolerance)
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


@functools.lru_cache(maxsize=2)
def workload(name):
    w = workloads.BY_NAME[name]
    inp = workloads.generate(w)
    return w, inp, dev_tensors(inp, w.dtype, DEV)


def small_case(B, L, D, N=16, E=4, k=2, dtype="f32", seed=0, h0=False):
    w = workloads.Workload("case", B=B, L=L, D=D, N=N, E=E, k=k, dtype=dtype, seed=seed)
    inp = workloads.generate(w)
    if h0:
        rng = np.random.default_rng(seed + 100)
        inp["h0"] = rng.standard_normal((B, D, N)).astype(np.float32)
    return w, inp, dev_tensors(inp, dtype, DEV)


def route_on_gpu(t, w):
    idx, gate = swimba.route(t["x"], t["Wr"], w.k)
    return idx, gate


def scan_args(t, idx, gate):
    return (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"], t["Dskip"])


def oracle_scan(inp, idx, gate, dsel=None, h0=None, separate=False):
    """Oracle on all channels or on the channel subset `dsel`."""
    idx = host(idx).astype(np.int32) if isinstance(idx, torch.Tensor) else idx
    gate = host(gate) if isinstance(gate, torch.Tensor) else gate
    sl = slice(None) if dsel is None else dsel
    args = (inp["x"][:, :, sl], inp["dt_raw"][:, :, sl], inp["Bm"], inp["Cm"], idx, gate,
            inp["A"][:, sl], inp["dt_bias"][:, sl], inp["Dskip"][:, sl])
    if h0 is not None:
        h0 = h0[:, :, sl] if separate else h0[:, sl]
    fn = oracle.scan_separate if separate else oracle.scan
    return fn(*args, h0=h0)


def tol_for(w):
    return TOL_F32 if w.dtype == "f32" else TOL_BF16


# ---------------------------------------------------------------- router
@pytest.mark.parametrize("name", ["tiny", "mamba130m_layer", "mamba1p4b_layer", "long_context"])
def test_route_workload(name):
    w, inp, t = workload(name)
    idx, gate = route_on_gpu(t, w)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy().reshape(-1, w.k)
    gg = gate.cpu().numpy().reshape(-1, w.k).astype(np.float64)
    T = gi.shape[0]
    # properties of every token at full size
    assert gi.min() >= 0 and gi.max() < w.E
    assert np.all(np.sort(gi, axis=1)[:, 1:] != np.sort(gi, axis=1)[:, :-1]) if w.k > 1 else True
    assert np.all(gg > 0) and np.max(np.abs(gg.sum(1) - 1)) < 1e-6
    assert np.all(np.diff(gg, axis=1) <= 1e-7)
    # oracle on sampled tokens
    rng = np.random.default_rng(7)
    sel = np.arange(T) if T <= 4096 else np.sort(rng.choice(T, 4096, replace=False))
    xs = inp["x"].reshape(T, w.D)[sel]
    ridx, rgate, logits, absdot = oracle.route(xs, inp["Wr"], w.k)
    tol = route_tolerance(absdot, w.D)
    ties = check_route(gi[sel], logits, tol, w.k)
    same = np.all(gi[sel] == ridx, axis=1)
    gerr = np.abs(gg[sel] - rgate)
    assert np.all(gerr[same] <= gate_bound(ridx, tol)[same]), float(gerr[same].max())
    assert np.median(gerr[same]) < 1e-6
    assert ties <= max(2, len(sel) // 200), ties


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,E,k", [(100, 1, 1), (100, 3, 2), (96, 5, 5), (64, 17, 3),
                                   (72, 64, 4), (1, 8, 2), (513, 16, 16), (1030, 5, 2),
                                   (2048, 8, 2), (1100, 33, 4), (4099, 16, 3), (96, 48, 2),
                                   (128, 64, 20), (64, 64, 64), (200, 40, 2), (5, 23, 7)])
def test_route_shapes(dtype, D, E, k):
    """Ragged D (scalar staging path), E not a kernel width, the wide-E path
    (17..64 experts: 2, 3 and 4 slices of 16, more than 16 slots, k = E),
    k = E, D = 1, a token count that is not a multiple of 64, and wide rows."""
    w, inp, t = small_case(B=3, L=45, D=D, E=E, k=k, dtype=dtype, seed=D + E)
    idx, gate = route_on_gpu(t, w)
    gi = idx.cpu().numpy().reshape(-1, k)
    gg = gate.cpu().numpy().reshape(-1, k).astype(np.float64)
    ridx, rgate, logits, absdot = oracle.route(inp["x"].reshape(-1, D), inp["Wr"], k)
    tol = route_tolerance(absdot, D)
    check_route(gi, logits, tol, k)
    same = np.all(gi == ridx, axis=1)
    assert np.all(np.abs(gg - rgate)[same] <= gate_bound(ridx, tol)[same])


def test_route_exact_ties_prefer_lower_expert():
    w, inp, t = small_case(B=1, L=200, D=64, E=6, k=3, dtype="bf16", seed=3)
    Wr = inp["Wr"].copy()
    Wr[:, 4] = Wr[:, 1]
    Wr[:, 5] = Wr[:, 2]
    idx, gate = swimba.route(t["x"], torch.from_numpy(Wr).to(DEV), 3)
    ridx, _, logits, _ = oracle.route(inp["x"].reshape(-1, 64), Wr, 3)
    gi = idx.cpu().numpy().reshape(-1, 3)
    for tk in range(gi.shape[0]):
        s = list(gi[tk])
        for a, b in ((1, 4), (2, 5)):
            if a in s and b in s:
                assert s.index(a) < s.index(b)


@pytest.mark.parametrize("E", [40, 64])
def test_route_exact_ties_prefer_lower_expert_wide(E):
    """Duplicated Wr columns across 16-expert slices tie exactly: the lower
    expert comes first."""
    w, inp, t = small_case(B=1, L=200, D=256, E=E, k=4, dtype="bf16", seed=E)
    Wr = inp["Wr"].copy()
    Wr[:, 33] = Wr[:, 2]
    Wr[:, E - 1] = Wr[:, 17]
    idx, gate = swimba.route(t["x"], torch.from_numpy(Wr).to(DEV), 4)
    gi = idx.cpu().numpy().reshape(-1, 4)
    for tk in range(gi.shape[0]):
        s_ = list(gi[tk])
        for a, b in ((2, 33), (17, E - 1)):
            if a in s_ and b in s_:
                assert s_.index(a) < s_.index(b)
        assert len(set(s_)) == 4


def test_route_wide_layer():
    """64 experts at B = 2, L = 4096, D = 4096 (bf16): every token against the
    oracle's router."""
    w, inp, t = small_case(B=2, L=4096, D=4096, E=64, k=2, dtype="bf16", seed=640)
    idx, gate = route_on_gpu(t, w)
    gi = idx.cpu().numpy().reshape(-1, 2)
    gg = gate.cpu().numpy().reshape(-1, 2).astype(np.float64)
    ridx, rgate, logits, absdot = oracle.route(inp["x"].reshape(-1, w.D), inp["Wr"], 2)
    tol = route_tolerance(absdot, w.D)
    ties = check_route(gi, logits, tol, 2)
    same = np.all(gi == ridx, axis=1)
    assert np.all(np.abs(gg - rgate)[same] <= gate_bound(ridx, tol)[same])
    assert ties <= max(2, gi.shape[0] // 200), ties


def test_route_empty():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    Wr = torch.zeros((64, 4), dtype=torch.float32, device=DEV)
    idx, gate = swimba.route(x, Wr, 2)
    assert idx.shape == (0, 2)


# ------------------------------------------------------------- mixed scan
@pytest.mark.parametrize("carry", ["fixup", "rewalk"])
@pytest.mark.parametrize("chunk", [0, 16, 64, 100, 256])
@pytest.mark.parametrize("with_h0", [False, True])
def test_scan_tiny(chunk, carry, with_h0):
    w, inp, t = workload("tiny")
    idx, gate = route_on_gpu(t, w)
    h0 = np.random.default_rng(5).standard_normal((w.B, w.D, 16)).astype(np.float32) \
        if with_h0 else None
    y, hf = swimba.scan(*scan_args(t, idx, gate), h0=None if h0 is None else
                        torch.from_numpy(h0).to(DEV), chunk=chunk, carry=carry)
    ry, rh = oracle_scan(inp, idx, gate, h0=h0)
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32, rel_err(host(hf), rh)


@pytest.mark.parametrize("chunk", [0, 77, 128, 700])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_scan_ragged_bf16(chunk, ydt):
    """Several 64-channel tiles plus a ragged tail (D = 200), several chunks
    plus a ragged last chunk, an initial state."""
    w, inp, t = small_case(B=2, L=700, D=200, E=8, k=2, dtype="bf16", seed=11, h0=True)
    idx, gate = route_on_gpu(t, w)
    ydtype = torch.float32 if ydt == "f32" else torch.bfloat16
    y, hf = swimba.scan(*scan_args(t, idx, gate), h0=t["h0"], chunk=chunk, y_dtype=ydtype)
    ry, rh = oracle_scan(inp, idx, gate, h0=inp["h0"])
    if ydt == "f32":
        assert rel_err(host(y), ry) < TOL_BF16
    else:
        assert_faithful_bf16(y, ry, "y")
    assert rel_err(host(hf), rh) < TOL_BF16


@pytest.mark.parametrize("name", ["mamba130m_layer", "mamba1p4b_layer", "long_context"])
def test_scan_workload_sampled(name):
    """Full-size workload in the benchmark's launch configuration (chunk 0 =
    the library's plan, 256 for the long context); sampled channels checked
    against the oracle, bf16 y faithfully rounded and fp32 y within 2e-3."""
    w, inp, t = workload(name)
    idx, gate = route_on_gpu(t, w)
    rng = np.random.default_rng(1)
    dsel = np.sort(rng.choice(w.D, 24, replace=False))
    ry, rh = oracle_scan(inp, idx, gate, dsel=dsel)
    for ydtype in (torch.bfloat16, torch.float32):
        y, hf = swimba.scan(*scan_args(t, idx, gate), chunk=w.chunk, y_dtype=ydtype)
        ys = y[:, :, torch.from_numpy(dsel).to(DEV)]
        if ydtype == torch.float32:
            assert rel_err(host(ys), ry) < TOL_BF16, rel_err(host(ys), ry)
        else:
            assert_faithful_bf16(ys, ry, name)
        assert rel_err(host(hf)[:, dsel], rh) < TOL_BF16, rel_err(host(hf)[:, dsel], rh)
        del y, hf


@pytest.mark.parametrize("E,k", [(1, 1), (8, 3), (8, 8), (16, 2), (16, 5), (2, 2)])
def test_scan_expert_counts(E, k):
    """Dense E = 1, runtime-k kernels (k = 3, 5, 8), the 8-wave workgroup for E > 8."""
    w, inp, t = small_case(B=2, L=300, D=130, E=E, k=k, dtype="f32", seed=E * 10 + k)
    idx, gate = route_on_gpu(t, w)
    for chunk in (0, 64):
        y, hf = swimba.scan(*scan_args(t, idx, gate), chunk=chunk)
        ry, rh = oracle_scan(inp, idx, gate)
        assert rel_err(host(y), ry) < TOL_F32, (chunk, rel_err(host(y), ry))
        assert rel_err(host(hf), rh) < TOL_F32


def test_scan_degenerate_shapes():
    # L = 0: h_final = h0 (or zeros)
    w, inp, t = small_case(B=2, L=0, D=70, E=4, k=2, h0=True)
    idx = torch.zeros((2, 0, 2), dtype=torch.int32, device=DEV)
    gate = torch.zeros((2, 0, 2), dtype=torch.float32, device=DEV)
    y, hf = swimba.scan(*scan_args(t, idx, gate), h0=t["h0"])
    assert torch.equal(hf, t["h0"])
    y, hf = swimba.scan(*scan_args(t, idx, gate))
    assert torch.count_nonzero(hf) == 0
    # L = 1, D = 1
    for (B, L, D) in ((1, 1, 64), (3, 5, 1), (1, 130, 1)):
        w, inp, t = small_case(B=B, L=L, D=D, E=3, k=2, seed=B + L + D)
        idx, gate = route_on_gpu(t, w)
        for chunk in (0, 2):
            y, hf = swimba.scan(*scan_args(t, idx, gate), chunk=chunk)
            ry, rh = oracle_scan(inp, idx, gate)
            assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_scan_chunking_and_carry_agree():
    """Chunk size and the carry method change rounding only."""
    w, inp, t = small_case(B=1, L=2048, D=128, E=8, k=2, dtype="bf16", seed=21)
    idx, gate = route_on_gpu(t, w)
    ref, rh = oracle_scan(inp, idx, gate)
    outs = []
    for chunk in (0, 32, 256, 2048):
        for carry in ("fixup", "rewalk"):
            y, hf = swimba.scan(*scan_args(t, idx, gate), chunk=chunk, carry=carry,
                                y_dtype=torch.float32)
            assert rel_err(host(y), ref) < TOL_BF16
            outs.append(host(y))
    for o in outs[1:]:
        assert rel_err(o, outs[0]) < 1e-4


def test_scan_deterministic():
    w, inp, t = workload("mamba130m_layer")
    idx, gate = route_on_gpu(t, w)
    y1, h1 = swimba.scan(*scan_args(t, idx, gate))
    y2, h2 = swimba.scan(*scan_args(t, idx, gate))
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    i2, g2 = route_on_gpu(t, w)
    assert torch.equal(idx, i2) and torch.equal(gate, g2)


@pytest.mark.parametrize("separate", [False, True])
@pytest.mark.parametrize("chunk", [0, 64])
def test_scan_phase_events(separate, chunk):
    """The six phase events are stamped in pass order, the chunk and fix-up
    passes take time when the sequence is chunked, and timing changes no output."""
    w, inp, t = small_case(B=2, L=300, D=128, E=4, k=2, dtype="bf16", seed=33)
    idx, gate = route_on_gpu(t, w)
    fn = swimba.scan_separate if separate else swimba.scan
    y0, h0_ = fn(*scan_args(t, idx, gate), chunk=chunk)
    ev = HipEvents(6)
    try:
        y1, h1 = fn(*scan_args(t, idx, gate), chunk=chunk, phase_events=ev.address)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(h0_, h1)
        for i in range(5):
            assert ev.ms(i, i + 1) >= 0.0, (i, ev.ms(i, i + 1))
        assert ev.ms(0, 1) > 0.0
        if chunk:
            assert ev.ms(4, 5) > 0.0
    finally:
        ev.close()


def test_scan_split_composition():
    w, inp, t = small_case(B=2, L=1000, D=96, E=4, k=2, dtype="bf16", seed=31)
    idx, gate = route_on_gpu(t, w)
    y, hf = swimba.scan(*scan_args(t, idx, gate), y_dtype=torch.float32)
    cut = 377
    a1 = [v[:, :cut].contiguous() for v in scan_args(t, idx, gate)[:6]] + list(
        scan_args(t, idx, gate)[6:])
    a2 = [v[:, cut:].contiguous() for v in scan_args(t, idx, gate)[:6]] + list(
        scan_args(t, idx, gate)[6:])
    y1, h1 = swimba.scan(*a1, y_dtype=torch.float32)
    y2, h2 = swimba.scan(*a2, h0=h1, y_dtype=torch.float32)
    assert rel_err(host(torch.cat([y1, y2], 1)), host(y)) < 1e-4
    assert rel_err(host(h2), host(hf)) < 1e-4


def test_scan_constant_inputs_closed_form_at_length():
    """L = 65536 with constant inputs and routing: every chunk boundary of the
    carry is pinned by h_t = b (1 - a^t) / (1 - a) without the oracle.  Slow
    decay (1 - a ~ 1e-3) keeps the carry significant across all 256 chunks."""
    B, L, D, N, E, k = 1, 65536, 64, 16, 2, 2
    rng = np.random.default_rng(41)
    xv = rng.uniform(0.5, 1.0, D).astype(np.float32)
    rv = np.full(D, -6.0, np.float32)                       # Delta ~ 2.5e-3
    Bv = rng.uniform(0.5, 1.0, N).astype(np.float32)
    Cv = rng.uniform(-1.0, 1.0, N).astype(np.float32)
    A = -rng.uniform(0.3, 0.6, (E, D, N)).astype(np.float32)
    bias = np.zeros((E, D), np.float32)
    Dsk = rng.standard_normal((E, D)).astype(np.float32)
    g = np.array([0.7, 0.3], np.float32)
    x = torch.from_numpy(np.broadcast_to(xv, (B, L, D)).copy()).to(DEV)
    dt = torch.from_numpy(np.broadcast_to(rv, (B, L, D)).copy()).to(DEV)
    Bm = torch.from_numpy(np.broadcast_to(Bv, (B, L, N)).copy()).to(DEV)
    Cm = torch.from_numpy(np.broadcast_to(Cv, (B, L, N)).copy()).to(DEV)
    idx = torch.from_numpy(np.broadcast_to(np.array([0, 1], np.int32), (B, L, k)).copy()).to(DEV)
    gate = torch.from_numpy(np.broadcast_to(g, (B, L, k)).copy()).to(DEV)
    y, hf = swimba.scan(x, dt, Bm, Cm, idx, gate, torch.from_numpy(A).to(DEV),
                        torch.from_numpy(bias).to(DEV), torch.from_numpy(Dsk).to(DEV), chunk=256)
    Dt = np.log1p(np.exp(rv.astype(np.float64)))
    a = np.exp(Dt[:, None] * (g[0] * A[0].astype(np.float64) + g[1] * A[1]))  # [D, N]
    b = Dt[:, None] * Bv[None].astype(np.float64) * xv[:, None]
    ts = np.array([1, 255, 256, 257, 4096, 30000, 65535, 65536])
    h = b[None] * (1 - a[None] ** ts[:, None, None]) / (1 - a[None])        # [T, D, N]
    want = h @ Cv.astype(np.float64) + (g[0] * Dsk[0] + g[1] * Dsk[1]) * xv
    got = host(y)[0, ts - 1]
    # relative error of (1 - a) in fp32 is ~ 2^-24 / (Delta |Abar|) ~ 1e-4 here
    assert rel_err(got, want) < 2e-3, rel_err(got, want)
    assert rel_err(host(hf)[0], h[-1]) < 2e-3


def test_scan_noncontractive_falls_back_to_rewalk():
    """A > 0 somewhere (no contraction): the fix-up may not stop early; the
    kernels detect it and recompute whole chunks, still matching the oracle."""
    w, inp, t = small_case(B=1, L=600, D=64, E=4, k=2, dtype="f32", seed=51)
    A = inp["A"].copy()
    A[2, :, 3] = 0.02
    inp["A"] = A
    t["A"] = torch.from_numpy(A).to(DEV)
    idx, gate = route_on_gpu(t, w)
    y, hf = swimba.scan(*scan_args(t, idx, gate), chunk=64)
    ry, rh = oracle_scan(inp, idx, gate)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


# --------------------------------------------------------------- separate
@pytest.mark.parametrize("chunk", [0, 32, 100, 256])
def test_separate_tiny(chunk):
    w, inp, t = workload("tiny")
    idx, gate = route_on_gpu(t, w)
    y, hf = swimba.scan_separate(*scan_args(t, idx, gate), chunk=chunk)
    ry, rh = oracle_scan(inp, idx, gate, separate=True)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("E,k", [(8, 2), (4, 4), (16, 2), (3, 1)])
@pytest.mark.parametrize("chunk", [0, 96])
def test_separate_bf16(E, k, chunk):
    w, inp, t = small_case(B=2, L=500, D=136, E=E, k=k, dtype="bf16", seed=E + k)
    rng = np.random.default_rng(9)
    H0 = rng.standard_normal((2, E, 136, 16)).astype(np.float32)
    idx, gate = route_on_gpu(t, w)
    y, hf = swimba.scan_separate(*scan_args(t, idx, gate), h0=torch.from_numpy(H0).to(DEV),
                                 chunk=chunk, y_dtype=torch.float32)
    ry, rh = oracle_scan(inp, idx, gate, h0=H0, separate=True)
    assert rel_err(host(y), ry) < TOL_BF16 and rel_err(host(hf), rh) < TOL_BF16


def test_separate_workload_sampled():
    w, inp, t = workload("mamba1p4b_layer")
    idx, gate = route_on_gpu(t, w)
    dsel = np.sort(np.random.default_rng(2).choice(w.D, 16, replace=False))
    ry, rh = oracle_scan(inp, idx, gate, dsel=dsel, separate=True)
    y, hf = swimba.scan_separate(*scan_args(t, idx, gate))
    assert_faithful_bf16(y[:, :, torch.from_numpy(dsel).to(DEV)], ry, "separate y")
    assert rel_err(host(hf)[:, :, dsel], rh) < TOL_BF16


def test_separate_long_context_sampled():
    """The long-context workload in the separate design at the library's own
    chunking (the launch the benchmark times: a few long chunks whose fix-up
    stops once every expert's carried state has decayed), on sampled
    channels."""
    w, inp, t = workload("long_context")
    idx, gate = route_on_gpu(t, w)
    chunk, nchunks = swimba.scan_plan(t["x"], t["A"], idx, separate=swimba.DESIGN_SEPARATE)
    assert nchunks > 1
    dsel = np.sort(np.random.default_rng(4).choice(w.D, 12, replace=False))
    ry, rh = oracle_scan(inp, idx, gate, dsel=dsel, separate=True)
    y, hf = swimba.scan_separate(*scan_args(t, idx, gate))
    assert_faithful_bf16(y[:, :, torch.from_numpy(dsel).to(DEV)], ry, "separate y")
    assert rel_err(host(hf)[:, :, dsel], rh) < TOL_BF16


@pytest.mark.parametrize("D", [100, 72])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_separate_many_experts_ragged_channels(D, dtype):
    """16 experts (a workgroup fills a CU; rounds are prefetched in 16-byte
    packets when D allows it, element by element otherwise) with a ragged
    last tile, several chunks and h0."""
    w, inp, t = small_case(B=2, L=700, D=D, E=16, k=2, dtype=dtype, seed=D)
    rng = np.random.default_rng(D)
    H0 = rng.standard_normal((2, 16, D, 16)).astype(np.float32)
    idx, gate = route_on_gpu(t, w)
    y, hf = swimba.scan_separate(*scan_args(t, idx, gate), h0=torch.from_numpy(H0).to(DEV),
                                 chunk=192, y_dtype=torch.float32)
    ry, rh = oracle_scan(inp, idx, gate, h0=H0, separate=True)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert rel_err(host(y), ry) < tol and rel_err(host(hf), rh) < tol


def test_separate_unaligned_streams():
    """x and dt_raw at a 2-byte offset (views into larger buffers): the
    16-expert workgroups stage rounds element by element instead of in
    16-byte packets, with the same results as aligned copies."""
    w, inp, t = small_case(B=1, L=400, D=128, E=16, k=2, dtype="bf16", seed=88)
    idx, gate = route_on_gpu(t, w)
    def shifted(a):
        flat = torch.empty(a.numel() + 1, dtype=a.dtype, device=DEV)
        v = flat[1:].view(a.shape)
        v.copy_(a)
        assert v.data_ptr() % 16 != 0
        return v
    ta = dict(t)
    ta["x"], ta["dt_raw"] = shifted(t["x"]), shifted(t["dt_raw"])
    y0, h0 = swimba.scan_separate(*scan_args(t, idx, gate), chunk=128, y_dtype=torch.float32)
    y1, h1 = swimba.scan_separate(*scan_args(ta, idx, gate), chunk=128, y_dtype=torch.float32)
    assert torch.equal(y0, y1) and torch.equal(h0, h1)
    ry, rh = oracle_scan(inp, idx, gate, separate=True)
    assert rel_err(host(y1), ry) < TOL_BF16 and rel_err(host(h1), rh) < TOL_BF16


@pytest.mark.parametrize("E,k", [(4, 2), (16, 2), (8, 1), (12, 1)])
def test_separate_fixup_stops_and_matches_rewalk(E, k):
    """Chunks much longer than the decay horizon: the fix-up stops early, and
    its y equals the full re-walk's to fp32 resolution; both match the
    oracle, with h0."""
    w, inp, t = small_case(B=2, L=3000, D=136, E=E, k=k, dtype="f32", seed=70 + E)
    rng = np.random.default_rng(11)
    H0 = rng.standard_normal((2, E, 136, 16)).astype(np.float32)
    h0 = torch.from_numpy(H0).to(DEV)
    idx, gate = route_on_gpu(t, w)
    ya, ha = swimba.scan_separate(*scan_args(t, idx, gate), h0=h0, chunk=1024)
    yr, hr = swimba.scan_separate(*scan_args(t, idx, gate), h0=h0, chunk=1024, carry="rewalk")
    ry, rh = oracle_scan(inp, idx, gate, h0=H0, separate=True)
    assert rel_err(host(ya), ry) < TOL_F32 and rel_err(host(ha), rh) < TOL_F32
    assert rel_err(host(yr), ry) < TOL_F32 and rel_err(host(hr), rh) < TOL_F32
    assert rel_err(host(ya), host(yr)) < 1e-5
    assert torch.equal(ha, hr)  # final states come from the carry pass in both


def test_separate_idle_expert_keeps_fixup_running():
    """One expert is selected in the first chunk only, so its carried state
    never decays in later chunks: the fix-up must walk them to the end (it
    cannot stop), and still match the oracle."""
    w, inp, t = small_case(B=1, L=2048, D=64, E=4, k=1, dtype="f32", seed=73)
    idx = np.zeros((1, 2048, 1), dtype=np.int32)
    idx[0, :300, 0] = np.arange(300) % 4          # every expert early on
    idx[0, 300:, 0] = 1 + np.arange(1748) % 2     # then experts 1 and 2 only
    idx[0, 1900:, 0] = 3                          # expert 3 comes back late
    gate = np.ones((1, 2048, 1), dtype=np.float32)
    y, hf = swimba.scan_separate(*scan_args(t, torch.from_numpy(idx).to(DEV),
                                            torch.from_numpy(gate).to(DEV)), chunk=512)
    ry, rh = oracle_scan(inp, idx, gate, separate=True)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_separate_noncontractive_falls_back_to_rewalk():
    """Some A > 0: the separate design's fix-up may not stop early; it
    re-walks whole chunks and still matches the oracle."""
    w, inp, t = small_case(B=1, L=1500, D=64, E=4, k=2, dtype="f32", seed=75)
    A = inp["A"].copy()
    A[1, :, 5] = 0.01
    inp["A"] = A
    t["A"] = torch.from_numpy(A).to(DEV)
    idx, gate = route_on_gpu(t, w)
    y, hf = swimba.scan_separate(*scan_args(t, idx, gate), chunk=512)
    ry, rh = oracle_scan(inp, idx, gate, separate=True)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("E,k,dtype", [(17, 2, "bf16"), (32, 2, "bf16"), (33, 3, "f32"),
                                       (64, 2, "bf16"), (64, 1, "f32")])
@pytest.mark.parametrize("chunk", [0, 160])
def test_separate_many_experts(E, k, dtype, chunk):
    """17..64 experts: 16 waves of two or four experts each (rows reloaded per
    staged round), chunked and not, with h0 and a ragged last tile."""
    w, inp, t = small_case(B=2, L=520, D=136, E=E, k=k, dtype=dtype, seed=E + 3 * k)
    rng = np.random.default_rng(E)
    H0 = rng.standard_normal((2, E, 136, 16)).astype(np.float32)
    idx, gate = route_on_gpu(t, w)
    y, hf = swimba.scan_separate(*scan_args(t, idx, gate), h0=torch.from_numpy(H0).to(DEV),
                                 chunk=chunk, y_dtype=torch.float32)
    ry, rh = oracle_scan(inp, idx, gate, h0=H0, separate=True)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert rel_err(host(y), ry) < tol and rel_err(host(hf), rh) < tol


def test_separate_64_experts_layer_sampled():
    """64 experts at the 1.4B-like layer shape (B = 8, L = 4096, D = 4096,
    top-2, bf16) in the library's own launch, on sampled channels."""
    w = workloads.Workload("wide", B=8, L=4096, D=4096, N=16, E=64, k=2, dtype="bf16", seed=9)
    inp = workloads.generate(w)
    t = dev_tensors(inp, "bf16", DEV)
    idx, gate = route_on_gpu(t, w)
    dsel = np.sort(np.random.default_rng(5).choice(w.D, 8, replace=False))
    ry, rh = oracle_scan(inp, idx, gate, dsel=dsel, separate=True)
    y, hf = swimba.scan_separate(*scan_args(t, idx, gate))
    assert_faithful_bf16(y[:, :, torch.from_numpy(dsel).to(DEV)], ry, "separate y")
    assert rel_err(host(hf)[:, :, dsel], rh) < TOL_BF16


def test_separate_constant_top1_equals_mixed():
    w, inp, t = small_case(B=1, L=400, D=64, E=4, k=1, dtype="f32", seed=61)
    idx = torch.full((1, 400, 1), 2, dtype=torch.int32, device=DEV)
    gate = torch.ones((1, 400, 1), dtype=torch.float32, device=DEV)
    ym, hm = swimba.scan(*scan_args(t, idx, gate), chunk=64)
    ys, hs = swimba.scan_separate(*scan_args(t, idx, gate), chunk=64)
    assert rel_err(host(ys), host(ym)) < 1e-5
    assert rel_err(host(hs)[:, 2], host(hm)) < 1e-5
    assert torch.count_nonzero(hs[:, [0, 1, 3]]) == 0


# ------------------------------------------------------------------ step
def step_tensors(s, dtype):
    return dev_tensors(s, dtype, DEV)


def test_step_decode_workload():
    """Decode workload (B 256, D 5120, E 8, top-2): 8 routed steps, all
    channels, against the oracle's step fed with the GPU's routing."""
    w = workloads.BY_NAME["decode"]
    p, steps = workloads.decode_steps(w, steps=8)
    tp = dev_tensors(p, "f32", DEV)
    state = torch.zeros((w.B, w.D, 16), dtype=torch.float32, device=DEV)
    rstate = np.zeros((w.B, w.D, 16))
    idx_out = torch.empty((w.B, w.k), dtype=torch.int32, device=DEV)
    gate_out = torch.empty((w.B, w.k), dtype=torch.float32, device=DEV)
    for s in steps:
        ts = step_tensors(s, w.dtype)
        y = swimba.step(ts["x"], ts["dt_raw"], ts["Bm"], ts["Cm"], tp["A"], tp["dt_bias"],
                        tp["Dskip"], state, Wr=tp["Wr"], k=w.k, idx_out=idx_out,
                        gate_out=gate_out, y_dtype=torch.float32)
        gi = idx_out.cpu().numpy()
        ridx, rgate, logits, absdot = oracle.route(s["x"], p["Wr"], w.k)
        check_route(gi, logits, route_tolerance(absdot, w.D), w.k)
        ry, _, _ = oracle.step(s["x"], s["dt_raw"], s["Bm"], s["Cm"], p["A"], p["dt_bias"],
                               p["Dskip"], rstate, idx=gi, gate=host(gate_out))
        assert rel_err(host(y), ry) < TOL_BF16
    assert rel_err(host(state), rstate) < TOL_BF16


def test_step_128_steps_sampled_and_resume():
    """128 steps on the decode workload: sampled channels against the oracle,
    and a state saved to the host at step 64 and restored into a fresh buffer
    continues bit-identically."""
    w = workloads.BY_NAME["decode"]
    p, steps = workloads.decode_steps(w)
    tp = dev_tensors(p, "f32", DEV)
    dsel = np.sort(np.random.default_rng(3).choice(w.D, 32, replace=False))
    dsel_t = torch.from_numpy(dsel).to(DEV)
    state = torch.zeros((w.B, w.D, 16), dtype=torch.float32, device=DEV)
    rstate = np.zeros((w.B, len(dsel), 16))
    Ap, bp, Dp = p["A"][:, dsel], p["dt_bias"][:, dsel], p["Dskip"][:, dsel]
    idx_out = torch.empty((w.B, w.k), dtype=torch.int32, device=DEV)
    gate_out = torch.empty((w.B, w.k), dtype=torch.float32, device=DEV)
    saved = None
    ys = []
    all_steps = list(steps)
    for i, s in enumerate(all_steps):
        ts = step_tensors(s, w.dtype)
        y = swimba.step(ts["x"], ts["dt_raw"], ts["Bm"], ts["Cm"], tp["A"], tp["dt_bias"],
                        tp["Dskip"], state, Wr=tp["Wr"], k=w.k, idx_out=idx_out,
                        gate_out=gate_out, y_dtype=torch.float32)
        ys.append(y.clone())
        ry, _, _ = oracle.step(s["x"][:, dsel], s["dt_raw"][:, dsel], s["Bm"], s["Cm"], Ap, bp,
                               Dp, rstate, idx=idx_out.cpu().numpy(), gate=host(gate_out))
        assert rel_err(host(y[:, dsel_t]), ry) < TOL_BF16, i
        if i == 63:
            saved = state.cpu().clone()
    assert rel_err(host(state)[:, dsel], rstate) < TOL_BF16
    final = state.clone()
    # resume from the host copy taken after step 64
    state2 = torch.empty_like(state)
    state2.copy_(saved.to(DEV))
    for i, s in enumerate(all_steps[64:]):
        ts = step_tensors(s, w.dtype)
        y = swimba.step(ts["x"], ts["dt_raw"], ts["Bm"], ts["Cm"], tp["A"], tp["dt_bias"],
                        tp["Dskip"], state2, Wr=tp["Wr"], k=w.k, y_dtype=torch.float32)
        assert torch.equal(y, ys[64 + i])
    assert torch.equal(state2, final)


def test_steps_equal_scan():
    """128 forced-routing steps on a carried state equal one scan of L = 128."""
    w, inp, t = small_case(B=4, L=128, D=200, E=8, k=2, dtype="bf16", seed=71, h0=True)
    idx, gate = route_on_gpu(t, w)
    y, hf = swimba.scan(*scan_args(t, idx, gate), h0=t["h0"], y_dtype=torch.float32)
    state = t["h0"].clone()
    for s in range(128):
        ys = swimba.step(t["x"][:, s].contiguous(), t["dt_raw"][:, s].contiguous(),
                         t["Bm"][:, s].contiguous(), t["Cm"][:, s].contiguous(), t["A"],
                         t["dt_bias"], t["Dskip"], state, idx=idx[:, s].contiguous(),
                         gate=gate[:, s].contiguous(), y_dtype=torch.float32)
        assert rel_err(host(ys), host(y[:, s])) < 1e-4, s
    assert rel_err(host(state), host(hf)) < 1e-4


@pytest.mark.parametrize("B,D,E,k,dtype", [(1, 100, 4, 2, "f32"), (3, 64, 1, 1, "bf16"),
                                           (5, 333, 16, 3, "bf16"), (2, 7, 64, 2, "f32")])
def test_step_shapes(B, D, E, k, dtype):
    w, inp, t = small_case(B=B, L=1, D=D, E=E, k=k, dtype=dtype, seed=B * D, h0=True)
    state = t["h0"].clone()
    rstate = inp["h0"].astype(np.float64).copy()
    idx_out = torch.empty((B, k), dtype=torch.int32, device=DEV)
    gate_out = torch.empty((B, k), dtype=torch.float32, device=DEV)
    y = swimba.step(t["x"][:, 0].contiguous(), t["dt_raw"][:, 0].contiguous(),
                    t["Bm"][:, 0].contiguous(), t["Cm"][:, 0].contiguous(), t["A"], t["dt_bias"],
                    t["Dskip"], state, Wr=t["Wr"], k=k, idx_out=idx_out, gate_out=gate_out,
                    y_dtype=torch.float32)
    ridx, rgate, logits, absdot = oracle.route(inp["x"][:, 0], inp["Wr"], k)
    check_route(idx_out.cpu().numpy(), logits, route_tolerance(absdot, D), k)
    ry, _, _ = oracle.step(inp["x"][:, 0], inp["dt_raw"][:, 0], inp["Bm"][:, 0], inp["Cm"][:, 0],
                           inp["A"], inp["dt_bias"], inp["Dskip"], rstate,
                           idx=idx_out.cpu().numpy(), gate=host(gate_out))
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert rel_err(host(y), ry) < tol and rel_err(host(state), rstate) < tol


def test_prepared_step_matches_step():
    """PreparedStep (marshalled once) gives bit-identical results to step()."""
    w = workloads.Workload("case", B=5, L=1, D=200, N=16, E=6, k=2, dtype="bf16", seed=61)
    p, steps = workloads.decode_steps(w, steps=3)
    P = {kk: torch.from_numpy(v).to(DEV) for kk, v in p.items()}
    S = [{kk: torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(DEV)
          for kk, v in s.items()} for s in steps]
    st1 = torch.zeros((w.B, w.D, 16), dtype=torch.float32, device=DEV)
    st2 = st1.clone()
    y1 = torch.empty((w.B, w.D), dtype=torch.float32, device=DEV)
    y2 = torch.empty_like(y1)
    for s in S:
        swimba.step(s["x"], s["dt_raw"], s["Bm"], s["Cm"], P["A"], P["dt_bias"], P["Dskip"], st1,
                    Wr=P["Wr"], k=w.k, y=y1)
        swimba.PreparedStep(s["x"], s["dt_raw"], s["Bm"], s["Cm"], P["A"], P["dt_bias"],
                            P["Dskip"], st2, Wr=P["Wr"], k=w.k, y=y2)()
        assert torch.equal(y1, y2)
    assert torch.equal(st1, st2)


@pytest.mark.parametrize("E", [4, 20])
def test_out_of_range_expert_ids_are_clamped(E):
    """Expert ids below 0 or at E and above in a caller's routing are read as
    0 and E - 1 (include/swimba.h): the scans (LDS-table and rows-from-memory
    paths), the separate design (E <= 16) and the decode step give the same
    bits as with the clamped ids, and the mixed scan matches the oracle fed
    the clamped ids."""
    w, inp, t = small_case(B=2, L=200, D=96, E=E, k=2, seed=E + 3)
    rng = np.random.default_rng(E)
    bad = rng.integers(-3, E + 4, size=(2, 200, 2)).astype(np.int32)
    bad[0, :4] = [[-1, E], [E + 3, -3], [0, E - 1], [-2, 2]]
    good = np.clip(bad, 0, E - 1).astype(np.int32)
    gate = torch.from_numpy(rng.uniform(0.1, 0.9, size=(2, 200, 2)).astype(np.float32)).to(DEV)
    ib, ig = torch.from_numpy(bad).to(DEV), torch.from_numpy(good).to(DEV)
    args = lambda idx: (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"],
                        t["Dskip"])
    for chunk in (0, 64):
        yb, hb = swimba.scan(*args(ib), chunk=chunk)
        yg, hg = swimba.scan(*args(ig), chunk=chunk)
        assert torch.equal(yb, yg) and torch.equal(hb, hg), chunk
    ry, rh = oracle.scan(inp["x"], inp["dt_raw"], inp["Bm"], inp["Cm"], good, host(gate),
                         inp["A"], inp["dt_bias"], inp["Dskip"])
    assert rel_err(host(yb), ry) < TOL_F32 and rel_err(host(hb), rh) < TOL_F32
    if E <= 16:
        yb, hb = swimba.scan_separate(*args(ib), chunk=64)
        yg, hg = swimba.scan_separate(*args(ig), chunk=64)
        assert torch.equal(yb, yg) and torch.equal(hb, hg)
    # decode step with the routing given
    st_b = torch.zeros((2, 96, 16), dtype=torch.float32, device=DEV)
    st_g = torch.zeros_like(st_b)
    for s in range(3):
        xs, rs = t["x"][:, s].contiguous(), t["dt_raw"][:, s].contiguous()
        bs, cs = t["Bm"][:, s].contiguous(), t["Cm"][:, s].contiguous()
        gs = gate[:, s].contiguous()
        y1 = swimba.step(xs, rs, bs, cs, t["A"], t["dt_bias"], t["Dskip"], st_b,
                         idx=ib[:, s].contiguous(), gate=gs)
        y2 = swimba.step(xs, rs, bs, cs, t["A"], t["dt_bias"], t["Dskip"], st_g,
                         idx=ig[:, s].contiguous(), gate=gs)
        assert torch.equal(y1, y2) and torch.equal(st_b, st_g), s
