"""GPU parity of the per-slot separate trajectories (swimba_scan_slots: slot
j's state advances at every token with the expert routed to slot j; "Swimba:
Switch Mamba Model Scales State Space Models", Spanish "Distinción de
Diseños") against the oracle's ref_scan_slots on the same seeded inputs and
the GPU router's routing: every chunk join, k = 1..4, both transition forms,
both input terms, bf16 ragged shapes, sampled channels of the full-size
layer, the non-contractive fallback and the degenerate sizes."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, assert_faithful_bf16, dev_tensors, host, rel_err
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def case(B, L, D, E=4, k=2, dtype="f32", seed=0, h0=False, scalar=False, name=None):
    if name:
        w = workloads.BY_NAME[name]
    else:
        w = workloads.Workload("slots", B=B, L=L, D=D, N=16, E=E, k=k, dtype=dtype, seed=seed)
    inp = workloads.generate(w)
    if scalar:
        inp["A"] = np.ascontiguousarray(inp["A"][:, :, 0])
    if h0:
        inp["h0"] = np.random.default_rng(w.seed + 8).standard_normal(
            (w.B, w.k, w.D, 16)).astype(np.float32)
    return w, inp, dev_tensors(inp, w.dtype, DEV)


def diag_of(A):
    return A if A.ndim == 3 else np.ascontiguousarray(np.repeat(A[:, :, None], 16, axis=2))


def args(t, idx, gate):
    return (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"], t["Dskip"])


def ref(inp, idx, gate, h0=None, zoh=False, dsel=None):
    sl = slice(None) if dsel is None else dsel
    return oracle.scan_slots(inp["x"][:, :, sl], inp["dt_raw"][:, :, sl], inp["Bm"], inp["Cm"],
                             host(idx).astype(np.int32), host(gate), diag_of(inp["A"])[:, sl],
                             inp["dt_bias"][:, sl], inp["Dskip"][:, sl],
                             h0=None if h0 is None else h0[:, :, sl], zoh=zoh)


@pytest.mark.parametrize("carry", ["fixup", "rewalk"])
@pytest.mark.parametrize("chunk", [0, 16, 64, 100])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_slots_parity(k, chunk, carry):
    w, inp, t = case(B=2, L=300, D=130, E=5, k=k, seed=50 + k, h0=True)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    y, hf = swimba.scan_slots(*args(t, idx, gate), h0=t["h0"], chunk=chunk, carry=carry)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"])
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32, rel_err(host(hf), rh)


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("chunk", [0, 64])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_slots_forms(k, chunk, scalar, zoh):
    w, inp, t = case(B=2, L=260, D=96, E=4, k=k, seed=60 + k, h0=True, scalar=scalar)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    y, hf = swimba.scan_slots(*args(t, idx, gate), h0=t["h0"], chunk=chunk, zoh=zoh)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"], zoh=zoh)
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_slots_bf16_ragged(ydt):
    w, inp, t = case(B=2, L=700, D=200, E=8, k=2, dtype="bf16", seed=70)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    ydtype = torch.float32 if ydt == "f32" else torch.bfloat16
    y, hf = swimba.scan_slots(*args(t, idx, gate), chunk=77, y_dtype=ydtype)
    ry, rh = ref(inp, idx, gate)
    if ydt == "f32":
        assert rel_err(host(y), ry) < TOL_BF16
    else:
        assert_faithful_bf16(y, ry, "y")
    assert rel_err(host(hf), rh) < TOL_BF16


def test_slots_full_size_sampled():
    """The 130M-like layer (B=4, L=2048, D=1536, E=8, k=2, bf16) in the
    library's own chunking: 24 sampled channels against the oracle (each
    channel's slot recurrences are independent of the other channels)."""
    w, inp, t = case(0, 0, 0, name="mamba130m_layer")
    idx, gate = swimba.route(t["x"], t["Wr"], w.k)
    y, hf = swimba.scan_slots(*args(t, idx, gate))
    dsel = np.sort(np.random.default_rng(5).choice(w.D, 24, replace=False))
    ry, rh = ref(inp, idx, gate, dsel=dsel)
    assert_faithful_bf16(y[:, :, torch.from_numpy(dsel).to(DEV)], ry, "y")
    assert rel_err(host(hf)[:, :, dsel], rh) < TOL_BF16


def test_slots_many_chunks():
    """128 chunks of 64 tokens: the carry crosses every chunk boundary and
    the fix-up truncates on decayed slots."""
    w, inp, t = case(B=1, L=8192, D=64, E=4, k=2, seed=71, h0=True)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y, hf = swimba.scan_slots(*args(t, idx, gate), h0=t["h0"], chunk=64)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"])
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_slots_constant_routing_equals_separate():
    """Each slot keeps one expert for the whole sequence: the per-slot and
    per-expert trajectories coincide (GPU against GPU)."""
    w, inp, t = case(B=2, L=500, D=128, E=4, k=2, seed=72)
    idx = torch.tensor([3, 1], dtype=torch.int32, device=DEV).expand(2, 500, 2).contiguous()
    gate = torch.tensor([0.7, 0.3], device=DEV).expand(2, 500, 2).contiguous()
    ys, hs = swimba.scan_slots(*args(t, idx, gate), y_dtype=torch.float32)
    ye, he = swimba.scan_separate(*args(t, idx, gate), y_dtype=torch.float32)
    assert rel_err(host(ys), host(ye)) < 1e-5
    assert rel_err(host(hs[:, 0]), host(he[:, 3])) < 1e-5
    assert rel_err(host(hs[:, 1]), host(he[:, 1])) < 1e-5


def test_slots_noncontractive_fallback():
    """A positive A in one tile: its chunks are recomputed in full."""
    w, inp, t = case(B=1, L=600, D=64, E=4, k=2, seed=73)
    A = inp["A"].copy()
    A[1, 9] = 0.01
    inp["A"] = A
    t["A"] = torch.from_numpy(A).to(DEV)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y, hf = swimba.scan_slots(*args(t, idx, gate), chunk=64)
    ry, rh = ref(inp, idx, gate)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_slots_prepared_and_plan():
    w, inp, t = case(B=2, L=300, D=96, E=4, k=2, seed=74)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y0, h0 = swimba.scan_slots(*args(t, idx, gate), chunk=64)
    y = torch.empty_like(y0)
    hf = torch.empty_like(h0)
    call = swimba.PreparedScan(swimba.DESIGN_SLOTS, *args(t, idx, gate), y=y, h_final=hf,
                               chunk=64)
    call()
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(hf, h0)
    assert swimba.scan_plan(t["x"], t["A"], idx, separate=swimba.DESIGN_SLOTS, chunk=64) == (64, 5)


def test_slots_degenerate():
    # L = 0: h_final = h0
    w, inp, t = case(B=2, L=0, D=70, E=4, k=3, h0=True)
    idx = torch.zeros((2, 0, 3), dtype=torch.int32, device=DEV)
    gate = torch.zeros((2, 0, 3), dtype=torch.float32, device=DEV)
    y, hf = swimba.scan_slots(*args(t, idx, gate), h0=t["h0"])
    assert torch.equal(hf, t["h0"])
    # one token, one channel, tiny batch
    for (B, L, D, k) in ((1, 1, 64, 2), (3, 5, 1, 3), (2, 33, 65, 4)):
        w, inp, t = case(B=B, L=L, D=D, E=4, k=k, seed=B + L + D, h0=True)
        idx, gate = swimba.route(t["x"], t["Wr"], k)
        y, hf = swimba.scan_slots(*args(t, idx, gate), h0=t["h0"], chunk=16)
        ry, rh = ref(inp, idx, gate, h0=inp["h0"])
        assert rel_err(host(y), ry) < TOL_F32, (B, L, D, k)
        assert rel_err(host(hf), rh) < TOL_F32, (B, L, D, k)


@pytest.mark.parametrize("scalar,zoh", [(False, False), (True, False), (False, True)])
@pytest.mark.parametrize("chunk", [0, 96])
@pytest.mark.parametrize("E,k,dtype", [(24, 2, "f32"), (64, 1, "f32"), (40, 2, "bf16")])
def test_slots_many_experts(E, k, dtype, chunk, scalar, zoh):
    """More than 16 experts: each slot reads its expert's rows from memory
    every token (k <= 2), with h0 and a ragged last tile."""
    w, inp, t = case(B=2, L=420, D=136, E=E, k=k, dtype=dtype, seed=E + k, h0=True,
                     scalar=scalar)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    y, hf = swimba.scan_slots(*args(t, idx, gate), h0=t["h0"], chunk=chunk, zoh=zoh,
                              y_dtype=torch.float32)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"], zoh=zoh)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert rel_err(host(y), ry) < tol and rel_err(host(hf), rh) < tol


def test_slots_many_experts_nonnegative_A_flags_its_tile():
    """A non-negative A entry of an expert no slot uses, in the second tile:
    the per-tile check flags it, so that tile's chunks are re-walked whole
    (bit for bit the explicit full re-walk), and all of it matches the
    oracle."""
    w, inp, t = case(B=1, L=600, D=130, E=20, k=2, seed=77)
    A = inp["A"].copy()
    A[19, 100, 2] = 0.0
    inp["A"] = A
    t["A"] = torch.from_numpy(A).to(DEV)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    idx = torch.where(idx == 19, torch.zeros_like(idx), idx)
    ya, ha = swimba.scan_slots(*args(t, idx, gate), chunk=64)
    yr, hr = swimba.scan_slots(*args(t, idx, gate), chunk=64, carry="rewalk")
    assert torch.equal(ya[:, :, 64:128], yr[:, :, 64:128]) and torch.equal(ha, hr)
    ry, rh = ref(inp, idx, gate)
    assert rel_err(host(ya), ry) < TOL_F32 and rel_err(host(ha), rh) < TOL_F32
