"""GPU studies and variants built from the library's entry points:

* Theorem 4 of "Swimba: Switch Mamba Model Scales State Space Models"
  (French summary, "Fondements Théoriques"): the one-trajectory (mixed) and
  per-expert (separate) designs coincide under constant top-1 routing and
  drift apart as routing varies over time -- measured as the relative
  difference of their outputs against the switching rate;
* the separate-design reading in which all E experts advance at every token
  (gates zero for the unselected), run as swimba_scan_separate with k = E and
  dense routing, against the oracle with the same dense routing;
* a decode loop captured once in a HIP graph and replayed, against the same
  steps run eagerly."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL_BF16, TOL_F32, check_route, dev_tensors, host, rel_err,
                         route_tolerance)
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def inputs(B, L, D, E, seed, dtype="f32"):
    w = workloads.Workload("study", B=B, L=L, D=D, N=16, E=E, k=1, dtype=dtype, seed=seed)
    inp = workloads.generate(w)
    return w, inp, dev_tensors(inp, dtype, DEV)


def divergence(t, idx, gate):
    a = (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"], t["Dskip"])
    ym, _ = swimba.scan(*a, y_dtype=torch.float32)
    ys, _ = swimba.scan_separate(*a, y_dtype=torch.float32)
    return float(torch.linalg.vector_norm(ym - ys) / torch.linalg.vector_norm(ys))


def test_theorem4_designs_diverge_with_switching():
    B, L, D, E = 2, 1024, 256, 8
    w, inp, t = inputs(B, L, D, E, seed=61)
    d = {}
    for p in (0.0, 0.01, 0.1, 0.5):
        i, g = workloads.switching_routing(B, L, E, p, seed=62)
        d[p] = divergence(t, torch.from_numpy(i).to(DEV), torch.from_numpy(g).to(DEV))
    # constant top-1 routing: one expert runs alone in both designs
    assert d[0.0] < 1e-5, d
    assert d[0.01] > 1e-3 and d[0.01] < d[0.1] < d[0.5], d


def test_theorem4_divergence_matches_oracle():
    """The divergence itself, on a small case, from the oracle's two designs."""
    B, L, D, E = 1, 300, 64, 4
    w, inp, t = inputs(B, L, D, E, seed=63)
    i, g = workloads.switching_routing(B, L, E, 0.2, seed=64)
    got = divergence(t, torch.from_numpy(i).to(DEV), torch.from_numpy(g).to(DEV))
    args = (inp["x"], inp["dt_raw"], inp["Bm"], inp["Cm"], i, g.astype(np.float64), inp["A"],
            inp["dt_bias"], inp["Dskip"])
    ym, _ = oracle.scan(*args)
    ys, _ = oracle.scan_separate(*args)
    want = np.linalg.norm(ym - ys) / np.linalg.norm(ys)
    assert abs(got - want) < 1e-4 * want + 1e-6, (got, want)


@pytest.mark.parametrize("chunk", [0, 64])
def test_separate_all_experts_advance(chunk):
    """Every expert advances at every token, weighted by its gate (zero when
    not selected): k = E with dense routing."""
    B, L, D, E, k = 2, 300, 96, 4, 2
    w, inp, t = inputs(B, L, D, E, seed=65)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    gi, gg = host(idx).astype(np.int64), host(gate)
    dense = np.zeros((B, L, E))
    np.put_along_axis(dense, gi, gg, axis=2)
    didx = np.broadcast_to(np.arange(E, dtype=np.int32), (B, L, E)).copy()
    a = (t["x"], t["dt_raw"], t["Bm"], t["Cm"], torch.from_numpy(didx).to(DEV),
         torch.from_numpy(dense.astype(np.float32)).to(DEV), t["A"], t["dt_bias"], t["Dskip"])
    y, hf = swimba.scan_separate(*a, chunk=chunk)
    ry, rh = oracle.scan_separate(inp["x"], inp["dt_raw"], inp["Bm"], inp["Cm"], didx, dense,
                                  inp["A"], inp["dt_bias"], inp["Dskip"])
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32
    # differs from the design that advances only the selected experts
    ys, _ = swimba.scan_separate(t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"],
                                 t["dt_bias"], t["Dskip"], chunk=chunk)
    assert rel_err(host(ys), host(y)) > 1e-2


def test_decode_graph_replay_matches_eager():
    """16 routed decode steps captured in one graph; three replays, each from
    the same initial state with eager work in between, against the eager run."""
    B, D, E, k, S = 64, 512, 8, 2, 16
    w = workloads.Workload("decode_graph", B=B, L=1, D=D, N=16, E=E, k=k, dtype="bf16", seed=66)
    p, steps = workloads.decode_steps(w, steps=S)
    P = {n: torch.from_numpy(v).to(DEV) for n, v in p.items()}
    X = [{n: torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(DEV)
          for n, v in s_.items()} for s_ in steps]
    s0 = torch.randn((B, D, 16), device=DEV)
    # eager reference
    st = s0.clone()
    ys = []
    for s_ in X:
        ys.append(swimba.step(s_["x"], s_["dt_raw"], s_["Bm"], s_["Cm"], P["A"], P["dt_bias"],
                              P["Dskip"], st, Wr=P["Wr"], k=k).clone())
    st_eager = st.clone()
    # capture
    state = s0.clone()
    yg = [torch.empty((B, D), dtype=torch.bfloat16, device=DEV) for _ in range(S)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls = [swimba.PreparedStep(s_["x"], s_["dt_raw"], s_["Bm"], s_["Cm"], P["A"],
                                     P["dt_bias"], P["Dskip"], state, Wr=P["Wr"], k=k, y=yg[i],
                                     stream=side) for i, s_ in enumerate(X)]
        for c in calls:      # warm-up on the capture stream
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for c in calls:
            c()
    for r in range(3):
        state.copy_(s0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, st_eager), r
        for i in range(S):
            assert torch.equal(yg[i], ys[i]), (r, i)
        _ = (s0 * 2).sum().item()   # eager work between replays


def test_decode_graph_replay_matches_oracle_full_shape():
    """The decode workload's shape (B 256, D 5120, E 8, top-2): 16 routed steps
    captured in one HIP graph, replayed three times (eager work in between).
    Every replayed step's routing is checked against the oracle's router,
    and its y and state against the oracle's step fed with that routing."""
    w = workloads.BY_NAME["decode"]
    S = 16
    p, steps = workloads.decode_steps(w, steps=S)
    steps = list(steps)
    P = {n: torch.from_numpy(v).to(DEV) for n, v in p.items()}
    X = [{n: torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(DEV)
          for n, v in s_.items()} for s_ in steps]
    B, D, k = w.B, w.D, w.k
    state = torch.zeros((B, D, 16), dtype=torch.float32, device=DEV)
    yg = [torch.empty((B, D), dtype=torch.float32, device=DEV) for _ in range(S)]
    ig = [torch.empty((B, k), dtype=torch.int32, device=DEV) for _ in range(S)]
    gg = [torch.empty((B, k), dtype=torch.float32, device=DEV) for _ in range(S)]
    snaps = [torch.empty((B, D, 16), dtype=torch.float32, device=DEV) for _ in range(S)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls = [swimba.PreparedStep(s_["x"], s_["dt_raw"], s_["Bm"], s_["Cm"], P["A"],
                                     P["dt_bias"], P["Dskip"], state, Wr=P["Wr"], k=k, y=yg[i],
                                     idx_out=ig[i], gate_out=gg[i], stream=side)
                 for i, s_ in enumerate(X)]
        for c in calls:      # warm-up on the capture stream
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i, c in enumerate(calls):
            c()
            torch.mul(state, 1.0, out=snaps[i])   # the state after step i (a kernel)
    first = None
    for r in range(3):
        state.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [(host(yg[i]), ig[i].cpu().numpy(), host(gg[i]), host(snaps[i])) for i in range(S)]
        if first is None:
            # the oracle, step by step, driven by the replay's routing
            rstate = np.zeros((B, D, 16))
            for i, s_ in enumerate(steps):
                gy, gi, ga, gs = got[i]
                _, _, logits, absdot = oracle.route(s_["x"], p["Wr"], k)
                check_route(gi, logits, route_tolerance(absdot, D), k)
                ry, _, _ = oracle.step(s_["x"], s_["dt_raw"], s_["Bm"], s_["Cm"], p["A"],
                                       p["dt_bias"], p["Dskip"], rstate, idx=gi, gate=ga)
                assert rel_err(gy, ry) < TOL_BF16, (r, i)
                assert rel_err(gs, rstate) < TOL_BF16, (r, i)
            first = got
        else:
            for i in range(S):
                for a_, b_ in zip(got[i], first[i]):
                    assert np.array_equal(a_, b_), (r, i)
        _ = (state * 2).sum().item()   # eager work between replays


def test_step_slices_agree_at_near_tie():
    """Two rows of D = 1024 (each row split over several workgroups) whose
    two experts' logits tie in exact arithmetic: Wr[:, 1] = Wr[:, 0] + v with
    v orthogonal to both rows' x.  Every workgroup of a row must route the
    row the same way: every channel's y and state equal the oracle's step
    driven by the reported routing (top-1, so a split row would mix two
    experts' parameters)."""
    B, D, E, k = 2, 1024, 2, 1
    w = workloads.Workload("tie", B=B, L=1, D=D, N=16, E=E, k=k, dtype="f32", seed=808)
    inp = workloads.generate(w)
    x = inp["x"][:, 0].astype(np.float64)
    rng = np.random.default_rng(809)
    v = rng.standard_normal(D)
    for r in range(B):   # Gram-Schmidt: v orthogonal to both rows
        q = x[r] - sum((x[r] @ x[j]) / (x[j] @ x[j]) * x[j] for j in range(r))
        v -= (v @ q) / (q @ q) * q
    Wr = inp["Wr"].copy()
    Wr[:, 1] = (Wr[:, 0].astype(np.float64) + 0.3 * v / np.linalg.norm(v)).astype(np.float32)
    inp["Wr"] = Wr
    t = dev_tensors(inp, "f32", DEV)
    h0 = np.random.default_rng(810).standard_normal((B, D, 16)).astype(np.float32)
    state = torch.from_numpy(h0).to(DEV)
    idx_out = torch.empty((B, k), dtype=torch.int32, device=DEV)
    gate_out = torch.empty((B, k), dtype=torch.float32, device=DEV)
    y = swimba.step(t["x"][:, 0].contiguous(), t["dt_raw"][:, 0].contiguous(),
                    t["Bm"][:, 0].contiguous(), t["Cm"][:, 0].contiguous(), t["A"], t["dt_bias"],
                    t["Dskip"], state, Wr=t["Wr"], k=k, idx_out=idx_out, gate_out=gate_out,
                    y_dtype=torch.float32)
    _, _, logits, absdot = oracle.route(inp["x"][:, 0], Wr, k)
    check_route(idx_out.cpu().numpy(), logits, route_tolerance(absdot, D), k)
    rstate = h0.astype(np.float64)
    ry, _, _ = oracle.step(inp["x"][:, 0], inp["dt_raw"][:, 0], inp["Bm"][:, 0], inp["Cm"][:, 0],
                           inp["A"], inp["dt_bias"], inp["Dskip"], rstate,
                           idx=idx_out.cpu().numpy(), gate=host(gate_out))
    assert rel_err(host(y), ry) < TOL_F32
    assert rel_err(host(state), rstate) < TOL_F32
