"""Seeded randomized GPU parity over the scan entry points: each case draws a
shape (B, L, D, E, k), the input and output dtypes, the chunk size and chunk
join, the transition form (diagonal or one scalar per channel), the input
term (Euler or zero-order hold), the design (mixed, separate per expert,
separate per routing slot), an initial state or none, and the routing (the
GPU router, or forced routing with random experts -- repeats allowed -- and
random positive gates).  Every case is compared with the oracle on the same
inputs at the bars of the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, assert_faithful_bf16, dev_tensors, host, rel_err
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
NCASES = 40


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    design = ("mixed", "separate", "slots")[seed % 3]
    E = int(rng.integers(1, 17))
    kmax = min(E, 4 if design == "slots" else 3)
    c = dict(
        seed=seed, design=design, E=E, k=int(rng.integers(1, kmax + 1)),
        B=int(rng.integers(1, 4)), L=int(rng.integers(1, 401)), D=int(rng.integers(1, 201)),
        dtype=("f32", "bf16")[int(rng.integers(0, 2))],
        scalar=bool(rng.integers(0, 2)), zoh=bool(rng.integers(0, 2)),
        h0=bool(rng.integers(0, 2)), routed=bool(rng.integers(0, 2)),
        carry=("fixup", "rewalk")[int(rng.integers(0, 2))])
    c["chunk"] = 0 if rng.integers(0, 3) == 0 else int(rng.integers(1, c["L"] + 1))
    c["ybf"] = c["dtype"] == "bf16" and bool(rng.integers(0, 2))
    return c


def label(c):
    return "%(seed)d-%(design)s-B%(B)dL%(L)dD%(D)dE%(E)dk%(k)d-%(dtype)s" % c


def draw_wide(seed):
    """17..64 experts (the per-slot design with k <= 2 there)."""
    c = draw(seed)
    rng = np.random.default_rng(5000 + seed)
    c["design"] = ("mixed", "separate", "slots")[seed % 3]
    c["E"] = int(rng.integers(17, 65))
    c["k"] = int(rng.integers(1, 3 if c["design"] == "slots" else 4))
    return c


CASES = [draw(s) for s in range(NCASES)] + [draw_wide(NCASES + s) for s in range(18)]


@pytest.mark.parametrize("c", CASES, ids=[label(c) for c in CASES])
def test_random_scan(c):
    B, L, D, E, k = c["B"], c["L"], c["D"], c["E"], c["k"]
    w = workloads.Workload("random", B=B, L=L, D=D, N=16, E=E, k=k, dtype=c["dtype"],
                           seed=2000 + c["seed"])
    inp = workloads.generate(w)
    rng = np.random.default_rng(3000 + c["seed"])
    if c["scalar"]:
        inp["A"] = np.ascontiguousarray(inp["A"][:, :, 0])
    trajectories = {"mixed": None, "separate": E, "slots": k}[c["design"]]
    shape = (B, D, 16) if trajectories is None else (B, trajectories, D, 16)
    if c["h0"]:
        inp["h0"] = rng.standard_normal(shape).astype(np.float32)
    t = dev_tensors(inp, c["dtype"], DEV)
    if c["routed"]:
        idx, gate = swimba.route(t["x"], t["Wr"], k)
    else:
        ri = rng.integers(0, E, (B, L, k)).astype(np.int32)
        rg = rng.uniform(0.05, 1.0, (B, L, k)).astype(np.float32)
        rg /= rg.sum(-1, keepdims=True)
        idx, gate = torch.from_numpy(ri).to(DEV), torch.from_numpy(rg).to(DEV)
    fn = {"mixed": swimba.scan, "separate": swimba.scan_separate,
          "slots": swimba.scan_slots}[c["design"]]
    ref = {"mixed": oracle.scan, "separate": oracle.scan_separate,
           "slots": oracle.scan_slots}[c["design"]]
    ydt = torch.bfloat16 if c["ybf"] else torch.float32
    y, hf = fn(t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"],
               t["Dskip"], h0=t.get("h0"), chunk=c["chunk"], carry=c["carry"], zoh=c["zoh"],
               y_dtype=ydt)
    A = inp["A"] if not c["scalar"] else np.repeat(inp["A"][:, :, None], 16, axis=2)
    ry, rh = ref(inp["x"], inp["dt_raw"], inp["Bm"], inp["Cm"], host(idx).astype(np.int32),
                 host(gate), A, inp["dt_bias"], inp["Dskip"], h0=inp.get("h0"), zoh=c["zoh"])
    tol = TOL_F32 if c["dtype"] == "f32" else TOL_BF16
    if c["ybf"]:
        assert_faithful_bf16(y, ry, "y")
    else:
        assert rel_err(host(y), ry) < tol, ("y", rel_err(host(y), ry), c)
    assert rel_err(host(hf), rh) < tol, ("h_final", rel_err(host(hf), rh), c)


def draw_streams(seed):
    rng = np.random.default_rng(5000 + seed)
    c = dict(seed=seed, B=int(rng.integers(1, 4)), L=int(rng.integers(1, 301)),
             D=int(rng.integers(1, 201)), k=int(rng.integers(1, 5)),
             dtype=("f32", "bf16")[int(rng.integers(0, 2))], h0=bool(rng.integers(0, 2)),
             carry=("fixup", "rewalk")[int(rng.integers(0, 2))])
    c["chunk"] = 0 if rng.integers(0, 3) == 0 else int(rng.integers(1, c["L"] + 1))
    return c


SCASES = [draw_streams(s) for s in range(16)]


@pytest.mark.parametrize("c", SCASES, ids=["%(seed)d-B%(B)dL%(L)dD%(D)dk%(k)d-%(dtype)s" % c
                                           for c in SCASES])
def test_random_streams(c):
    B, L, D, k = c["B"], c["L"], c["D"], c["k"]
    w = workloads.Workload("random_streams", B=B, L=L, D=D, N=16, E=max(k, 1), k=k,
                           dtype=c["dtype"], seed=6000 + c["seed"])
    inp = workloads.generate_streams(w, k=k, B=B, L=L, D=D)
    h0 = None
    if c["h0"]:
        h0 = np.random.default_rng(7000 + c["seed"]).standard_normal((B, D, 16)).astype(np.float32)
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    t = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to(dt).to(DEV)
         for n in ("X", "dt_raw", "Bs", "Cs")}
    y, hf = swimba.scan_streams(t["X"], t["dt_raw"], t["Bs"], t["Cs"],
                                torch.from_numpy(inp["gate"]).to(DEV),
                                torch.from_numpy(inp["A"]).to(DEV),
                                torch.from_numpy(inp["dt_bias"]).to(DEV),
                                h0=None if h0 is None else torch.from_numpy(h0).to(DEV),
                                chunk=c["chunk"], carry=c["carry"], y_dtype=torch.float32)
    ry, rh = oracle.scan_streams(inp["X"], inp["dt_raw"], inp["Bs"], inp["Cs"], inp["gate"],
                                 inp["A"], inp["dt_bias"], h0=h0)
    tol = TOL_F32 if c["dtype"] == "f32" else TOL_BF16
    assert rel_err(host(y), ry) < tol, ("y", rel_err(host(y), ry), c)
    assert rel_err(host(hf), rh) < tol, ("h_final", rel_err(host(hf), rh), c)


def draw_step(seed):
    rng = np.random.default_rng(8000 + seed)
    E = int(rng.integers(1, 17))
    return dict(seed=seed, B=int(rng.integers(1, 41)), D=int(rng.integers(1, 301)), E=E,
                k=int(rng.integers(1, min(E, 3) + 1)),
                dtype=("f32", "bf16")[int(rng.integers(0, 2))], scalar=bool(rng.integers(0, 2)),
                zoh=bool(rng.integers(0, 2)), routed=bool(rng.integers(0, 2)))


PCASES = [draw_step(s) for s in range(16)]


@pytest.mark.parametrize("c", PCASES, ids=["%(seed)d-B%(B)dD%(D)dE%(E)dk%(k)d-%(dtype)s" % c
                                           for c in PCASES])
def test_random_step(c):
    """Three consecutive decode steps on a persistent state."""
    B, D, E, k, S = c["B"], c["D"], c["E"], c["k"], 3
    w = workloads.Workload("random_step", B=B, L=S, D=D, N=16, E=E, k=k, dtype=c["dtype"],
                           seed=9000 + c["seed"])
    inp = workloads.generate(w)
    rng = np.random.default_rng(9500 + c["seed"])
    if c["scalar"]:
        inp["A"] = np.ascontiguousarray(inp["A"][:, :, 0])
    t = dev_tensors(inp, c["dtype"], DEV)
    A = inp["A"] if not c["scalar"] else np.repeat(inp["A"][:, :, None], 16, axis=2)
    s0 = rng.standard_normal((B, D, 16)).astype(np.float32)
    state = torch.from_numpy(s0).to(DEV)
    rstate = s0.astype(np.float64)
    for s in range(S):
        xs, rs = t["x"][:, s].contiguous(), t["dt_raw"][:, s].contiguous()
        Bs, Cs = t["Bm"][:, s].contiguous(), t["Cm"][:, s].contiguous()
        if c["routed"]:
            io = torch.empty((B, k), dtype=torch.int32, device=DEV)
            go = torch.empty((B, k), dtype=torch.float32, device=DEV)
            y = swimba.step(xs, rs, Bs, Cs, t["A"], t["dt_bias"], t["Dskip"], state, Wr=t["Wr"],
                            k=k, idx_out=io, gate_out=go, y_dtype=torch.float32, zoh=c["zoh"])
        else:
            ri = rng.integers(0, E, (B, k)).astype(np.int32)
            rg = rng.uniform(0.05, 1.0, (B, k)).astype(np.float32)
            rg /= rg.sum(-1, keepdims=True)
            io, go = torch.from_numpy(ri).to(DEV), torch.from_numpy(rg).to(DEV)
            y = swimba.step(xs, rs, Bs, Cs, t["A"], t["dt_bias"], t["Dskip"], state, idx=io,
                            gate=go, y_dtype=torch.float32, zoh=c["zoh"])
        ry, _, _ = oracle.step(inp["x"][:, s], inp["dt_raw"][:, s], inp["Bm"][:, s],
                               inp["Cm"][:, s], A, inp["dt_bias"], inp["Dskip"], rstate,
                               idx=host(io).astype(np.int32), gate=host(go), zoh=c["zoh"])
        assert rel_err(host(y), ry) < TOL_F32, (s, rel_err(host(y), ry), c)
    assert rel_err(host(state), rstate) < TOL_F32, c
