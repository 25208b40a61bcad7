"""GPU parity of the scalar-transition form (one A per expert and channel,
shared by its 16 states: the Mamba-2 form A_t = a_t I) for the mixed scan,
the separate design and the decode step.

The oracle needs no new function: a scalar A is the diagonal A with the same
value in every state entry, so the expected values come from the oracle's
diagonal scans on the broadcast A.  Inputs: the seeded workloads, with the
scalar A of (e, d) taken as the n = 0 entry of that workload's A draw."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL_BF16, TOL_F32, assert_faithful_bf16, dev_tensors, host, rel_err)
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def case(B, L, D, E=4, k=2, dtype="f32", seed=0, h0=False, name=None):
    if name:
        w = workloads.BY_NAME[name]
    else:
        w = workloads.Workload("scalar_a", B=B, L=L, D=D, N=16, E=E, k=k, dtype=dtype, seed=seed)
    inp = workloads.generate(w)
    inp["A"] = np.ascontiguousarray(inp["A"][:, :, 0])          # [E, D]
    if h0:
        inp["h0"] = np.random.default_rng(seed + 3).standard_normal(
            (w.B, w.D, 16)).astype(np.float32)
    return w, inp, dev_tensors(inp, w.dtype, DEV)


def diag(A):
    """The same transition as a diagonal A: every state entry equal."""
    return np.ascontiguousarray(np.repeat(A[:, :, None], 16, axis=2))


def args(t, idx, gate, A=None):
    return (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"] if A is None else A,
            t["dt_bias"], t["Dskip"])


def ref(inp, idx, gate, h0=None, dsel=None, separate=False):
    sl = slice(None) if dsel is None else dsel
    fn = oracle.scan_separate if separate else oracle.scan
    return fn(inp["x"][:, :, sl], inp["dt_raw"][:, :, sl], inp["Bm"], inp["Cm"],
              host(idx).astype(np.int32), host(gate), diag(inp["A"])[:, sl],
              inp["dt_bias"][:, sl], inp["Dskip"][:, sl], h0=h0)


@pytest.mark.parametrize("carry", ["fixup", "rewalk"])
@pytest.mark.parametrize("chunk", [0, 16, 100, 256])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_scalar_a_mixed(chunk, carry, k):
    w, inp, t = case(B=2, L=300, D=130, E=5, k=k, seed=20 + k, h0=True)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    y, hf = swimba.scan(*args(t, idx, gate), h0=t["h0"], chunk=chunk, carry=carry)
    ry, rh = ref(inp, idx, gate, h0=inp["h0"])
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_scalar_a_bf16_ragged(ydt):
    w, inp, t = case(B=2, L=700, D=200, E=8, k=2, dtype="bf16", seed=5)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    ydtype = torch.float32 if ydt == "f32" else torch.bfloat16
    y, hf = swimba.scan(*args(t, idx, gate), chunk=77, y_dtype=ydtype)
    ry, rh = ref(inp, idx, gate)
    if ydt == "f32":
        assert rel_err(host(y), ry) < TOL_BF16
    else:
        assert_faithful_bf16(y, ry, "y")
    assert rel_err(host(hf), rh) < TOL_BF16


def test_scalar_a_equals_broadcast_diagonal_on_gpu():
    """The scalar form computes the same mixed exponent, decay and chunk
    decay as the diagonal kernels given the broadcast A."""
    w, inp, t = case(B=2, L=1000, D=192, E=8, k=2, dtype="bf16", seed=6)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    Ad = torch.from_numpy(diag(inp["A"])).to(DEV)
    for chunk in (0, 128):
        y1, h1 = swimba.scan(*args(t, idx, gate), chunk=chunk, y_dtype=torch.float32)
        y2, h2 = swimba.scan(*args(t, idx, gate, A=Ad), chunk=chunk, y_dtype=torch.float32)
        assert rel_err(host(y1), host(y2)) < 1e-6
        assert rel_err(host(h1), host(h2)) < 1e-6


def test_scalar_a_full_size_sampled():
    w, inp, t = case(0, 0, 0, name="mamba130m_layer")
    idx, gate = swimba.route(t["x"], t["Wr"], w.k)
    dsel = np.sort(np.random.default_rng(4).choice(w.D, 24, replace=False))
    ry, rh = ref(inp, idx, gate, dsel=dsel)
    y, hf = swimba.scan(*args(t, idx, gate))
    assert_faithful_bf16(y[:, :, torch.from_numpy(dsel).to(DEV)], ry, "y")
    assert rel_err(host(hf)[:, dsel], rh) < TOL_BF16


def test_scalar_a_noncontractive_fallback():
    w, inp, t = case(B=1, L=600, D=64, E=4, k=2, seed=7)
    A = inp["A"].copy()
    A[1, 9] = 0.01
    inp["A"] = A
    t["A"] = torch.from_numpy(A).to(DEV)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    y, hf = swimba.scan(*args(t, idx, gate), chunk=64)
    ry, rh = ref(inp, idx, gate)
    assert rel_err(host(y), ry) < TOL_F32 and rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("chunk", [0, 64])
@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (4, 3), (16, 2), (24, 2), (40, 3)])
def test_scalar_a_separate(chunk, E, k):
    """4 experts (one per wave), 16 (prefetched rounds), 24 and 40 (two and
    four experts per wave)."""
    w, inp, t = case(B=2, L=300, D=100, E=E, k=k, seed=30 + k + E)
    idx, gate = swimba.route(t["x"], t["Wr"], k)
    h0 = np.random.default_rng(9).standard_normal((2, E, 100, 16)).astype(np.float32)
    y, hf = swimba.scan_separate(*args(t, idx, gate), h0=torch.from_numpy(h0).to(DEV),
                                 chunk=chunk)
    ry, rh = ref(inp, idx, gate, h0=h0, separate=True)
    assert rel_err(host(y), ry) < TOL_F32, rel_err(host(y), ry)
    assert rel_err(host(hf), rh) < TOL_F32


@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("routed", [True, False])
def test_scalar_a_step(routed, k):
    w, inp, t = case(B=8, L=6, D=300, E=6, k=k, seed=11)
    state = torch.zeros((8, 300, 16), dtype=torch.float32, device=DEV)
    rstate = np.zeros((8, 300, 16))
    Ad = diag(inp["A"])
    for s in range(6):
        xs, rs = t["x"][:, s].contiguous(), t["dt_raw"][:, s].contiguous()
        Bs, Cs = t["Bm"][:, s].contiguous(), t["Cm"][:, s].contiguous()
        if routed:
            # the scan part is compared on the routing the GPU chose
            io = torch.empty((8, k), dtype=torch.int32, device=DEV)
            go = torch.empty((8, k), dtype=torch.float32, device=DEV)
            y = swimba.step(xs, rs, Bs, Cs, t["A"], t["dt_bias"], t["Dskip"], state, Wr=t["Wr"],
                            k=k, idx_out=io, gate_out=go)
            ry, _, _ = oracle.step(inp["x"][:, s], inp["dt_raw"][:, s], inp["Bm"][:, s],
                                   inp["Cm"][:, s], Ad, inp["dt_bias"], inp["Dskip"], rstate,
                                   idx=host(io).astype(np.int32), gate=host(go))
        else:
            idx = torch.from_numpy(np.array([[s % 6, (s + 1) % 6][:k]] * 8, np.int32)).to(DEV)
            gate = torch.from_numpy(np.array([[0.6, 0.4][:k]] * 8, np.float32)).to(DEV)
            y = swimba.step(xs, rs, Bs, Cs, t["A"], t["dt_bias"], t["Dskip"], state, idx=idx,
                            gate=gate)
            ry, _, _ = oracle.step(inp["x"][:, s], inp["dt_raw"][:, s], inp["Bm"][:, s],
                                   inp["Cm"][:, s], Ad, inp["dt_bias"], inp["Dskip"], rstate,
                                   idx=host(idx).astype(np.int32), gate=host(gate))
        assert rel_err(host(y), ry) < TOL_F32, (s, rel_err(host(y), ry))
    assert rel_err(host(state), rstate) < TOL_F32
