"""GPU parity of the all-experts separate trajectories (swimba_scan_all_experts:
every expert's state advances at every token with its own parameters; the
routing only picks whose outputs are mixed; "Swimba: Switch Mamba Model Scales
State Space Models", Spanish "Distinción de Diseños") against the oracle's
ref_scan_all_experts on the same seeded inputs: every chunk join, k = 1..3,
both transition forms, both input terms, bf16 ragged shapes, sampled channels
of the full-size layer, the routing-independence of the states, the k = E
reduction to the per-expert design, and the degenerate sizes."""
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
        w = workloads.Workload("all_experts", B=B, L=L, D=D, N=16, E=E, k=k, dtype=dtype,
                               seed=seed)
    inp = workloads.generate(w)
    if scalar:
        inp["A"] = np.ascontiguousarray(inp["A"][:, :, 0])
    if h0:
        inp["h0"] = np.random.default_rng(w.seed + 9).standard_normal(
            (w.B, w.E, w.D, 16)).astype(np.float32)
    return w, inp, dev_tensors(inp, w.dtype, DEV)


def diag_of(A):
    return A if A.ndim == 3 else np.ascontiguousarray(np.repeat(A[:, :, None], 16, axis=2))


def args(t, idx, gate):
    return (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"], t["Dskip"])


def ref(inp, idx, gate, h0=None, zoh=False, dsel=None):
    sl = slice(None) if dsel is None else dsel
    return oracle.scan_all_experts(inp["x"][:, :, sl], inp["dt_raw"][:, :, sl], inp["Bm"],
                                   inp["Cm"], host(idx).astype(np.int32), host(gate),
                                   diag_of(inp["A"])[:, sl], inp["dt_bias"][:, sl],
                                   inp["Dskip"][:, sl],
                                   h0=None if h0 is None else h0[:, :, sl], zoh=zoh)


@pytest.mark.parametrize("carry", ["fixup", "rewalk"])
@pytest.mark.parametrize("chunk", [0, 64, 100])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_all_experts_parity(k, chunk, carry):
    w, inp, t = case(B=2, L=300, D=130, E=5, k=k, seed=80 + k, h0=True)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    y, hf = swimba.scan_all_experts(*args(t, idx, gate), h0=t["h0"], chunk=chunk, carry=carry)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"])
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32, rel_err(host(hf), rh)


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("chunk", [0, 64])
def test_all_experts_forms(chunk, scalar, zoh):
    w, inp, t = case(B=2, L=260, D=96, E=4, k=2, seed=90, h0=True, scalar=scalar)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y, hf = swimba.scan_all_experts(*args(t, idx, gate), h0=t["h0"], chunk=chunk, zoh=zoh)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"], zoh=zoh)
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_all_experts_bf16_ragged(ydt):
    w, inp, t = case(B=2, L=700, D=200, E=8, k=2, dtype="bf16", seed=91)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    ydtype = torch.float32 if ydt == "f32" else torch.bfloat16
    y, hf = swimba.scan_all_experts(*args(t, idx, gate), chunk=77, y_dtype=ydtype)
    ry, rh = ref(inp, idx, gate)
    if ydt == "f32":
        assert rel_err(host(y), ry) < TOL_BF16
    else:
        assert_faithful_bf16(y, ry, "y")
    assert rel_err(host(hf), rh) < TOL_BF16


def test_all_experts_full_size_sampled():
    """The 130M-like layer (B=4, L=2048, D=1536, E=8, k=2, bf16) in the
    library's own chunking: 24 sampled channels against the oracle."""
    w, inp, t = case(0, 0, 0, name="mamba130m_layer")
    idx, gate = swimba.route(t["x"], t["Wr"], w.k)
    y, hf = swimba.scan_all_experts(*args(t, idx, gate))
    dsel = np.sort(np.random.default_rng(6).choice(w.D, 24, replace=False))
    ry, rh = ref(inp, idx, gate, dsel=dsel)
    assert_faithful_bf16(y[:, :, torch.from_numpy(dsel).to(DEV)], ry, "y")
    assert rel_err(host(hf)[:, :, dsel], rh) < TOL_BF16


def test_all_experts_many_chunks_repeated_experts():
    """128 chunks of 64 tokens, forced routing with repeated experts."""
    w, inp, t = case(B=1, L=8192, D=64, E=4, k=2, seed=92, h0=True)
    rng = np.random.default_rng(93)
    ri = rng.integers(0, 4, (1, 8192, 2)).astype(np.int32)
    rg = rng.uniform(0.1, 1.0, (1, 8192, 2)).astype(np.float32)
    idx, gate = torch.from_numpy(ri).to(DEV), torch.from_numpy(rg).to(DEV)
    y, hf = swimba.scan_all_experts(*args(t, idx, gate), h0=t["h0"], chunk=64)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"])
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


def test_all_experts_states_ignore_routing():
    """Two unrelated routings: the same final states, bit for bit (GPU)."""
    w, inp, t = case(B=2, L=400, D=128, E=4, k=2, seed=94)
    idx1, gate1 = swimba.route(t["x"], t["Wr"], 2)
    rng = np.random.default_rng(95)
    idx2 = torch.from_numpy(rng.integers(0, 4, (2, 400, 2)).astype(np.int32)).to(DEV)
    gate2 = torch.from_numpy(rng.uniform(0.1, 1, (2, 400, 2)).astype(np.float32)).to(DEV)
    y1, h1 = swimba.scan_all_experts(*args(t, idx1, gate1), chunk=100)
    y2, h2 = swimba.scan_all_experts(*args(t, idx2, gate2), chunk=100)
    assert torch.equal(h1, h2)
    assert rel_err(host(y1), host(y2)) > 1e-3


def test_all_experts_full_routing_equals_separate():
    """k = E with every expert selected at every token: the per-expert design
    advances every expert at every token too (GPU against GPU)."""
    w, inp, t = case(B=2, L=300, D=96, E=3, k=3, seed=96, h0=True)
    rng = np.random.default_rng(97)
    ri = np.stack([np.stack([rng.permutation(3) for _ in range(300)]) for _ in range(2)])
    idx = torch.from_numpy(ri.astype(np.int32)).to(DEV)
    gate = torch.from_numpy(rng.uniform(0.1, 1, (2, 300, 3)).astype(np.float32)).to(DEV)
    ya, ha = swimba.scan_all_experts(*args(t, idx, gate), h0=t["h0"], chunk=64,
                                     y_dtype=torch.float32)
    ys, hs = swimba.scan_separate(*args(t, idx, gate), h0=t["h0"], chunk=64,
                                  y_dtype=torch.float32)
    assert rel_err(host(ya), host(ys)) < 1e-5
    assert rel_err(host(ha), host(hs)) < 1e-5


def test_all_experts_prepared_and_plan():
    w, inp, t = case(B=2, L=300, D=96, E=4, k=2, seed=98)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y0, h0 = swimba.scan_all_experts(*args(t, idx, gate), chunk=64)
    y = torch.empty_like(y0)
    hf = torch.empty_like(h0)
    call = swimba.PreparedScan(swimba.DESIGN_ALL_EXPERTS, *args(t, idx, gate), y=y, h_final=hf,
                               chunk=64)
    call()
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(hf, h0)
    assert swimba.scan_plan(t["x"], t["A"], idx, separate=swimba.DESIGN_ALL_EXPERTS,
                            chunk=64) == (64, 5)


def test_all_experts_degenerate():
    # L = 0: h_final = h0
    w, inp, t = case(B=2, L=0, D=70, E=4, k=3, h0=True)
    idx = torch.zeros((2, 0, 3), dtype=torch.int32, device=DEV)
    gate = torch.zeros((2, 0, 3), dtype=torch.float32, device=DEV)
    y, hf = swimba.scan_all_experts(*args(t, idx, gate), h0=t["h0"])
    assert torch.equal(hf, t["h0"])
    # one token, one channel, one expert, tiny batch
    for (B, L, D, E, k) in ((1, 1, 64, 2, 2), (3, 5, 1, 3, 3), (2, 33, 65, 4, 1), (1, 20, 8, 1, 1)):
        w, inp, t = case(B=B, L=L, D=D, E=E, k=k, seed=B + L + D, h0=True)
        idx, gate = swimba.route(t["x"], t["Wr"], k)
        y, hf = swimba.scan_all_experts(*args(t, idx, gate), h0=t["h0"], chunk=16)
        ry, rh = ref(inp, idx, gate, h0=inp["h0"])
        assert rel_err(host(y), ry) < TOL_F32, (B, L, D, E, k)
        assert rel_err(host(hf), rh) < TOL_F32, (B, L, D, E, k)


def test_all_experts_sixteen_experts_runtime_k():
    """E = 16 (the largest workgroup, one wave per expert) with k = 3 (the
    runtime-k slot loop), scalar transition and zero-order hold."""
    w, inp, t = case(B=1, L=200, D=70, E=16, k=3, seed=99, h0=True, scalar=True)
    idx, gate = swimba.route(t["x"], t["Wr"], 3)
    y, hf = swimba.scan_all_experts(*args(t, idx, gate), h0=t["h0"], chunk=64, zoh=True)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"], zoh=True)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("E,chunk", [(24, 0), (40, 128)])
def test_all_experts_many_experts(E, chunk):
    """More than 16 experts: 16 waves of two or four experts each, every
    expert advancing at every token."""
    w, inp, t = case(B=1, L=260, D=72, E=E, k=2, seed=E, h0=True)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y, hf = swimba.scan_all_experts(*args(t, idx, gate), h0=t["h0"], chunk=chunk)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"])
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32
