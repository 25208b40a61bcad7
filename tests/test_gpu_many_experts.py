"""GPU parity of the mixed scan with more than 16 experts (up to 64): the
selected experts' rows are read from memory per token instead of an LDS
table.  The router picks the top k of E ("Swimba: Switch Mamba Model Scales
State Space Models", Spanish summary "Escalabilidad": more total experts at
a fixed number of active ones).  Every case is checked against the oracle
fed with the GPU's routing, at the usual bars."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL_BF16, TOL_F32, assert_faithful_bf16, dev_tensors, host, rel_err)
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def case(B, L, D, E, k, dtype, seed, h0=False, scalar_a=False):
    w = workloads.Workload("many", B=B, L=L, D=D, N=16, E=E, k=k, dtype=dtype, seed=seed)
    inp = workloads.generate(w)
    if scalar_a:
        inp["A"] = np.ascontiguousarray(inp["A"][:, :, 0])
    if h0:
        inp["h0"] = np.random.default_rng(seed + 5).standard_normal((B, D, 16)).astype(np.float32)
    return w, inp, dev_tensors(inp, dtype, DEV)


def args(t, idx, gate):
    return (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"], t["Dskip"])


def ref(inp, idx, gate, h0=None, dsel=None, zoh=False):
    sl = slice(None) if dsel is None else dsel
    A = inp["A"]
    if A.ndim == 2:  # scalar A: the same value in every state entry
        A = np.repeat(A[:, :, None], 16, axis=2)
    return oracle.scan(inp["x"][:, :, sl], inp["dt_raw"][:, :, sl], inp["Bm"], inp["Cm"],
                       host(idx).astype(np.int32), host(gate), A[:, sl], inp["dt_bias"][:, sl],
                       inp["Dskip"][:, sl], h0=h0, zoh=zoh)


@pytest.mark.parametrize("E", [17, 32, 64])
@pytest.mark.parametrize("chunk", [0, 77, 256])
def test_many_experts_bf16_ragged(E, chunk):
    """k = 2, bf16 streams, several tiles and a ragged one (D = 200), ragged
    chunks, an initial state; fp32 y within 2e-3 and bf16 y faithful."""
    w, inp, t = case(B=2, L=700, D=200, E=E, k=2, dtype="bf16", seed=E + chunk, h0=True)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"])
    y, hf = swimba.scan(*args(t, idx, gate), h0=t["h0"], chunk=chunk, y_dtype=torch.float32)
    assert rel_err(host(y), ry) < TOL_BF16, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_BF16
    yb, hb = swimba.scan(*args(t, idx, gate), h0=t["h0"], chunk=chunk)
    assert_faithful_bf16(yb, ry, "y E=%d" % E)
    assert torch.equal(hb, hf)


@pytest.mark.parametrize("E,k", [(64, 1), (64, 3), (40, 5), (32, 1), (24, 3), (32, 4)])
@pytest.mark.parametrize("carry", ["fixup", "rewalk"])
def test_many_experts_k(E, k, carry):
    """top-1 and runtime k (3, 4, 5) with fp32 streams, both chunk joins;
    up to 32 experts the A rows come from LDS, beyond from memory."""
    w, inp, t = case(B=2, L=300, D=130, E=E, k=k, dtype="f32", seed=E * 7 + k)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    ry, rh = ref(inp, idx, gate)
    for chunk in (0, 64):
        y, hf = swimba.scan(*args(t, idx, gate), chunk=chunk, carry=carry)
        assert rel_err(host(y), ry) < TOL_F32, (chunk, rel_err(host(y), ry))
        assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("zoh", [False, True])
def test_many_experts_scalar_a(zoh):
    """One transition per (expert, channel) with 48 experts, both input terms."""
    w, inp, t = case(B=2, L=400, D=96, E=48, k=2, dtype="f32", seed=91 + zoh, h0=True,
                     scalar_a=True)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"], zoh=zoh)
    y, hf = swimba.scan(*args(t, idx, gate), h0=t["h0"], chunk=64, zoh=zoh)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_many_experts_zoh_diagonal():
    w, inp, t = case(B=1, L=500, D=128, E=32, k=2, dtype="f32", seed=97)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    ry, rh = ref(inp, idx, gate, zoh=True)
    y, hf = swimba.scan(*args(t, idx, gate), chunk=100, zoh=True)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_many_experts_noncontractive_falls_back():
    """A > 0 in one expert's entries: the per-tile check of A flags the tiles
    and the fix-up recomputes whole chunks, still matching the oracle."""
    w, inp, t = case(B=1, L=600, D=130, E=33, k=2, dtype="f32", seed=55)
    A = inp["A"].copy()
    A[20, :, 3] = 0.02
    inp["A"] = A
    t["A"] = torch.from_numpy(A).to(DEV)
    # route every token to experts 20 and 5 so the positive entry is used
    idx = torch.tensor([20, 5], dtype=torch.int32, device=DEV).repeat(1, 600, 1).contiguous()
    gate = torch.tensor([0.6, 0.4], dtype=torch.float32, device=DEV).repeat(1, 600, 1).contiguous()
    ry, rh = ref(inp, idx, gate)
    y, hf = swimba.scan(*args(t, idx, gate), chunk=64)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("scalar_a", [False, True])
@pytest.mark.parametrize("E", [24, 33, 64])
def test_many_experts_nonnegative_A_flags_its_tile(E, scalar_a):
    """One non-negative A entry (of an expert the routing never picks) in the
    third 64-channel tile: the per-tile check (while staging the A rows in
    LDS up to 32 experts, a pre-pass beyond) must flag that tile, whose
    chunks are then re-walked whole -- bit for bit the same y as an explicit
    full re-walk -- while every tile still matches the oracle."""
    w, inp, t = case(B=1, L=700, D=200, E=E, k=2, dtype="f32", seed=E + 60, scalar_a=scalar_a)
    A = inp["A"].copy()
    if scalar_a:
        A[E - 1, 150] = 0.0
    else:
        A[E - 1, 150, 7] = 0.0
    inp["A"] = A
    t["A"] = torch.from_numpy(A).to(DEV)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    idx = torch.where(idx == E - 1, torch.zeros_like(idx), idx)  # never expert E - 1
    ya, ha = swimba.scan(*args(t, idx, gate), chunk=96)
    yr, hr = swimba.scan(*args(t, idx, gate), chunk=96, carry="rewalk")
    assert torch.equal(ya[:, :, 128:192], yr[:, :, 128:192])
    assert torch.equal(ha, hr)
    ry, rh = ref(inp, idx, gate)
    assert rel_err(host(ya), ry) < TOL_F32 and rel_err(host(ha), rh) < TOL_F32


def test_many_experts_layer_sampled():
    """B = 2, L = 4096, D = 2048, E = 64, top-2, bf16 in the library's own
    chunking; 24 sampled channels against the oracle."""
    w, inp, t = case(B=2, L=4096, D=2048, E=64, k=2, dtype="bf16", seed=101)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    dsel = np.sort(np.random.default_rng(4).choice(w.D, 24, replace=False))
    ry, rh = ref(inp, idx, gate, dsel=dsel)
    y, hf = swimba.scan(*args(t, idx, gate), y_dtype=torch.float32)
    ys = y[:, :, torch.from_numpy(dsel).to(DEV)]
    assert rel_err(host(ys), ry) < TOL_BF16
    assert rel_err(host(hf)[:, dsel], rh) < TOL_BF16
    y2, h2 = swimba.scan(*args(t, idx, gate), y_dtype=torch.float32)
    assert torch.equal(y, y2) and torch.equal(hf, h2)   # deterministic


def test_many_experts_noalloc_matches():
    """The no-allocation entry point (its buffer also holds the per-tile A
    checks here) gives the same bits as the scan with a workspace."""
    w, inp, t = case(B=2, L=700, D=200, E=32, k=2, dtype="bf16", seed=7)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y1, h1 = swimba.scan(*args(t, idx, gate), chunk=100, y_dtype=torch.float32)
    y2, h2 = swimba.scan_noalloc(*args(t, idx, gate), chunk=100, y_dtype=torch.float32)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
