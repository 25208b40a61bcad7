"""GPU parity of the zero-order-hold input term (disc = SWIMBA_DISC_ZOH:
B_bar = A^{-1}(exp(Delta A) - I) B, "Mamba y las SSMs", section "Mamba")
for the mixed scan (diagonal and scalar transitions), the separate design and
the decode step, against the oracle's zoh option on the same seeded inputs;
plus the continuous equilibrium at L = 65536, which pins the carry and the
small-|Delta A| numerics without the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, assert_faithful_bf16, dev_tensors, host, rel_err
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def case(B, L, D, E=4, k=2, dtype="f32", seed=0, h0=False, scalar=False):
    w = workloads.Workload("zoh", B=B, L=L, D=D, N=16, E=E, k=k, dtype=dtype, seed=seed)
    inp = workloads.generate(w)
    if scalar:
        inp["A"] = np.ascontiguousarray(inp["A"][:, :, 0])
    if h0:
        inp["h0"] = np.random.default_rng(seed + 5).standard_normal((B, D, 16)).astype(np.float32)
    return w, inp, dev_tensors(inp, dtype, DEV)


def diag_of(A):
    return A if A.ndim == 3 else np.ascontiguousarray(np.repeat(A[:, :, None], 16, axis=2))


def args(t, idx, gate):
    return (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"], t["Dskip"])


def ref(inp, idx, gate, h0=None, separate=False):
    fn = oracle.scan_separate if separate else oracle.scan
    return fn(inp["x"], inp["dt_raw"], inp["Bm"], inp["Cm"], host(idx).astype(np.int32),
              host(gate), diag_of(inp["A"]), inp["dt_bias"], inp["Dskip"], h0=h0, zoh=True)


@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("carry", ["fixup", "rewalk"])
@pytest.mark.parametrize("chunk", [0, 64, 100])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_zoh_mixed(scalar, carry, chunk, k):
    w, inp, t = case(B=2, L=300, D=130, E=5, k=k, seed=40 + k, h0=True, scalar=scalar)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    y, hf = swimba.scan(*args(t, idx, gate), h0=t["h0"], chunk=chunk, carry=carry, zoh=True)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"])
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_zoh_bf16_ragged(ydt):
    w, inp, t = case(B=2, L=700, D=200, E=8, k=2, dtype="bf16", seed=45)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    ydtype = torch.float32 if ydt == "f32" else torch.bfloat16
    y, hf = swimba.scan(*args(t, idx, gate), chunk=77, y_dtype=ydtype, zoh=True)
    ry, rh = ref(inp, idx, gate)
    if ydt == "f32":
        assert rel_err(host(y), ry) < TOL_BF16
    else:
        assert_faithful_bf16(y, ry, "y")
    assert rel_err(host(hf), rh) < TOL_BF16


@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("chunk", [0, 64])
@pytest.mark.parametrize("E", [4, 16, 24, 40])
def test_zoh_separate(scalar, chunk, E):
    w, inp, t = case(B=2, L=300, D=100, E=E, k=2, seed=46 + E, scalar=scalar)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y, hf = swimba.scan_separate(*args(t, idx, gate), chunk=chunk, zoh=True)
    ry, rh = ref(inp, idx, gate, separate=True)
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("scalar", [False, True])
def test_zoh_step(scalar):
    w, inp, t = case(B=8, L=5, D=300, E=6, k=2, seed=47, scalar=scalar)
    state = torch.zeros((8, 300, 16), dtype=torch.float32, device=DEV)
    rstate = np.zeros((8, 300, 16))
    for s in range(5):
        io = torch.empty((8, 2), dtype=torch.int32, device=DEV)
        go = torch.empty((8, 2), dtype=torch.float32, device=DEV)
        y = swimba.step(t["x"][:, s].contiguous(), t["dt_raw"][:, s].contiguous(),
                        t["Bm"][:, s].contiguous(), t["Cm"][:, s].contiguous(), t["A"],
                        t["dt_bias"], t["Dskip"], state, Wr=t["Wr"], k=2, idx_out=io,
                        gate_out=go, zoh=True)
        ry, _, _ = oracle.step(inp["x"][:, s], inp["dt_raw"][:, s], inp["Bm"][:, s],
                               inp["Cm"][:, s], diag_of(inp["A"]), inp["dt_bias"], inp["Dskip"],
                               rstate, idx=host(io).astype(np.int32), gate=host(go), zoh=True)
        assert rel_err(host(y), ry) < TOL_F32, (s, rel_err(host(y), ry))
    assert rel_err(host(state), rstate) < TOL_F32


@pytest.mark.parametrize("zoh", [False, True])
def test_extreme_decays(zoh):
    """Large step sizes and transitions (exp(Delta A) underflows to 0; the
    zero-order-hold factor is 1/|Delta A|) and tiny ones (dt_raw ~ -12, so
    Delta ~ 6e-6 needs an accurate log1p inside softplus, and Delta A ~ -1e-8,
    where exp(Delta A) - 1 cancels), for both input terms."""
    w, inp, t = case(B=1, L=200, D=64, E=2, k=1, seed=48)
    for scale, shift in ((1.0, 12.0), (1e-3, -12.0)):
        A = (inp["A"] * scale).astype(np.float32)
        dt = (inp["dt_raw"] + shift).astype(np.float32)
        t2 = dict(t, A=torch.from_numpy(A).to(DEV), dt_raw=torch.from_numpy(dt).to(DEV))
        inp2 = dict(inp, A=A, dt_raw=dt)
        idx, gate = swimba.route(t2["x"], t2["Wr"], 1)
        y, hf = swimba.scan(*args(t2, idx, gate), chunk=64, zoh=zoh)
        ry, rh = oracle.scan(inp2["x"], inp2["dt_raw"], inp2["Bm"], inp2["Cm"],
                             host(idx).astype(np.int32), host(gate), inp2["A"],
                             inp2["dt_bias"], inp2["Dskip"], zoh=zoh)
        assert rel_err(host(y), ry) < TOL_F32, (scale, rel_err(host(y), ry))
        assert rel_err(host(hf), rh) < TOL_F32


def test_zoh_equilibrium_at_length():
    """L = 65536, constant inputs and routing, chunk 256: the zero-order-hold
    state approaches the continuous equilibrium -B x / Abar as
    h_t = (1 - a^t) h*, with 1 - a ~ 1e-3 so that the carry matters across
    all 256 chunks."""
    B, L, D, N, E, k = 1, 65536, 64, 16, 2, 2
    rng = np.random.default_rng(49)
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
                        torch.from_numpy(bias).to(DEV), torch.from_numpy(Dsk).to(DEV), chunk=256,
                        zoh=True)
    Dt = np.log1p(np.exp(rv.astype(np.float64)))
    Abar = g[0] * A[0].astype(np.float64) + g[1] * A[1]                    # [D, N]
    a = np.exp(Dt[:, None] * Abar)
    hstar = -Bv[None].astype(np.float64) * xv[:, None] / Abar
    ts = np.array([1, 255, 256, 257, 4096, 30000, 65535, 65536])
    h = (1 - a[None] ** ts[:, None, None]) * hstar[None]
    want = h @ Cv.astype(np.float64) + (g[0] * Dsk[0] + g[1] * Dsk[1]) * xv
    got = host(y)[0, ts - 1]
    assert rel_err(got, want) < 2e-3, rel_err(got, want)
    assert rel_err(host(hf)[0], h[-1]) < 2e-3
