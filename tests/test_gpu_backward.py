"""GPU parity of the mixed scan's backward (swimba_scan_backward) against the
fp64 oracle's gradients (ref_scan_backward, itself pinned by finite
differences of the forward oracle), on the same seeded inputs and the GPU
router's routing.

Bars: rel 1e-4 for fp32 inputs and 2e-3 for bf16 inputs (fp32 arithmetic),
with the error measured against max(|ref|, rms(ref)) as in the forward tests.
Sums over channels (dB, dC, dgate) and over tokens (dA, dbias, dDskip) add
many terms in fp32; their error stays far inside these bars at the sizes
used here."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, dev_tensors, host, rel_err
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAMES = ("dx", "ddt_raw", "dBm", "dCm", "dgate", "dA", "ddt_bias", "dDskip", "dh0")
ORACLE = {"ddt_bias": "dbias"}


def case(B, L, D, E=4, k=2, dtype="f32", seed=0, dy_dtype=None):
    w = workloads.Workload("bwd", B=B, L=L, D=D, N=16, E=E, k=k, dtype=dtype, seed=seed)
    inp = workloads.generate(w)
    rng = np.random.default_rng(seed + 77)
    inp["h0"] = rng.standard_normal((B, D, 16)).astype(np.float32)
    inp["dhf"] = rng.standard_normal((B, D, 16)).astype(np.float32)
    dy = rng.standard_normal((B, L, D)).astype(np.float32)
    dyd = dy_dtype or dtype
    if dyd == "bf16":
        dy = workloads.bf16_round(dy)
    inp["dy"] = dy
    t = dev_tensors(inp, dtype, DEV)
    t["dy"] = torch.from_numpy(dy).to(torch.bfloat16 if dyd == "bf16" else torch.float32).to(DEV)
    return w, inp, t


def run(t, w, chunk=0, with_h0=True, with_dhf=True):
    idx, gate = swimba.route(t["x"], t["Wr"], w.k)
    g = swimba.scan_backward(t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"],
                             t["dt_bias"], t["Dskip"], t["dy"],
                             h0=t["h0"] if with_h0 else None,
                             dh_final=t["dhf"] if with_dhf else None, chunk=chunk)
    return idx, gate, g


def reference(inp, idx, gate, with_h0=True, with_dhf=True):
    return oracle.scan_backward(inp["x"], inp["dt_raw"], inp["Bm"], inp["Cm"],
                                host(idx).astype(np.int32), host(gate), inp["A"],
                                inp["dt_bias"], inp["Dskip"], inp["dy"],
                                h0=inp["h0"] if with_h0 else None,
                                dh_final=inp["dhf"] if with_dhf else None)


def check(g, ref, tol, names=NAMES):
    for n in names:
        err = rel_err(host(g[n]), ref[ORACLE.get(n, n)])
        assert err < tol, (n, err)


@pytest.mark.parametrize("chunk", [0, 16, 64, 256])
@pytest.mark.parametrize("k", [1, 2])
def test_backward_tiny(chunk, k):
    w, inp, t = case(B=1, L=256, D=64, E=4, k=k, seed=1 + k)
    idx, gate, g = run(t, w, chunk=chunk)
    check(g, reference(inp, idx, gate), TOL_F32)


@pytest.mark.parametrize("with_h0,with_dhf", [(False, False), (True, False), (False, True)])
def test_backward_optional_state_gradients(with_h0, with_dhf):
    w, inp, t = case(B=2, L=200, D=64, E=4, k=2, seed=5)
    idx, gate, g = run(t, w, chunk=32, with_h0=with_h0, with_dhf=with_dhf)
    check(g, reference(inp, idx, gate, with_h0, with_dhf), TOL_F32)


@pytest.mark.parametrize("chunk", [0, 64])
@pytest.mark.parametrize("E,k", [(5, 3), (8, 2), (16, 2), (3, 1)])
def test_backward_ragged_and_expert_counts(chunk, E, k):
    """A ragged channel tile (D = 130), the runtime-k path (k = 3), the
    4-wave chunk and state workgroups and 16-expert accumulators for
    E = 16, a length that is not a
    whole number of chunks or staging blocks."""
    w, inp, t = case(B=2, L=301, D=130, E=E, k=k, seed=10 * E + k)
    idx, gate, g = run(t, w, chunk=chunk)
    check(g, reference(inp, idx, gate), TOL_F32)


@pytest.mark.parametrize("dy_dtype", ["f32", "bf16"])
def test_backward_bf16_inputs(dy_dtype):
    w, inp, t = case(B=2, L=700, D=200, E=8, k=2, dtype="bf16", seed=7, dy_dtype=dy_dtype)
    idx, gate, g = run(t, w, chunk=0)
    check(g, reference(inp, idx, gate), TOL_BF16)


def test_backward_moderate_size():
    """Several chunks per sequence, tiles and workgroups: every output,
    including the sums over channels, against the oracle."""
    w, inp, t = case(B=2, L=1024, D=512, E=8, k=2, dtype="bf16", seed=9)
    idx, gate, g = run(t, w)
    check(g, reference(inp, idx, gate), TOL_BF16)


def test_backward_full_size_sampled_channels():
    """The 130M-like layer (B=4, L=2048, D=1536, E=8, k=2, bf16): per-channel
    gradients of 24 sampled channels (each channel's recurrence is
    independent, so the oracle runs on that subset)."""
    w0 = workloads.BY_NAME["mamba130m_layer"]
    w, inp, t = case(B=w0.B, L=w0.L, D=w0.D, E=w0.E, k=w0.k, dtype="bf16", seed=w0.seed)
    idx, gate, g = run(t, w)
    dsel = np.sort(np.random.default_rng(3).choice(w.D, 24, replace=False))
    ref = oracle.scan_backward(inp["x"][:, :, dsel], inp["dt_raw"][:, :, dsel], inp["Bm"],
                               inp["Cm"], host(idx).astype(np.int32), host(gate),
                               inp["A"][:, dsel], inp["dt_bias"][:, dsel],
                               inp["Dskip"][:, dsel], inp["dy"][:, :, dsel],
                               h0=inp["h0"][:, dsel], dh_final=inp["dhf"][:, dsel])
    sel = torch.from_numpy(dsel).to(DEV)
    for n, axis in (("dx", 2), ("ddt_raw", 2), ("dA", 1), ("ddt_bias", 1), ("dDskip", 1),
                    ("dh0", 1)):
        got = host(g[n].index_select(axis, sel))
        err = rel_err(got, ref[ORACLE.get(n, n)])
        assert err < TOL_BF16, (n, err)


def test_backward_1p4b_layer_sampled():
    """The 1.4B-like layer (B=8, L=4096, D=4096, E=8, k=2, bf16) in the
    library's own chunking: per-channel gradients of 16 sampled channels
    against the oracle on that subset; dC at three early tokens of every
    sequence against dy_t h_t with the oracle's states h_t (the forward over
    all channels up to t); finite, deterministic sums over channels."""
    w0 = workloads.BY_NAME["mamba1p4b_layer"]
    w, inp, t = case(B=w0.B, L=w0.L, D=w0.D, E=w0.E, k=w0.k, dtype="bf16", seed=w0.seed)
    idx, gate, g = run(t, w)
    gi, gg = host(idx).astype(np.int32), host(gate)
    dsel = np.sort(np.random.default_rng(5).choice(w.D, 16, replace=False))
    ref = oracle.scan_backward(inp["x"][:, :, dsel], inp["dt_raw"][:, :, dsel], inp["Bm"],
                               inp["Cm"], gi, gg, inp["A"][:, dsel], inp["dt_bias"][:, dsel],
                               inp["Dskip"][:, dsel], inp["dy"][:, :, dsel],
                               h0=inp["h0"][:, dsel], dh_final=inp["dhf"][:, dsel])
    sel = torch.from_numpy(dsel).to(DEV)
    for n, axis in (("dx", 2), ("ddt_raw", 2), ("dA", 1), ("ddt_bias", 1), ("dDskip", 1),
                    ("dh0", 1)):
        got = host(g[n].index_select(axis, sel))
        err = rel_err(got, ref[ORACLE.get(n, n)])
        assert err < TOL_BF16, (n, err)
    dC = host(g["dCm"])
    for tt in (0, 37, 200):
        sl = slice(0, tt + 1)
        _, ht = oracle.scan(inp["x"][:, sl], inp["dt_raw"][:, sl], inp["Bm"][:, sl],
                            inp["Cm"][:, sl], gi[:, sl], gg[:, sl], inp["A"], inp["dt_bias"],
                            inp["Dskip"], h0=inp["h0"])
        want = np.einsum("bd,bdn->bn", inp["dy"][:, tt].astype(np.float64), ht)
        assert rel_err(dC[:, tt], want) < TOL_BF16, (tt, rel_err(dC[:, tt], want))
    for n in ("dBm", "dCm", "dgate"):
        assert torch.isfinite(g[n]).all(), n
    _, _, g2 = run(t, w)
    for n in NAMES:
        assert torch.equal(g[n], g2[n]), n


def test_backward_chunking_agrees_and_is_deterministic():
    w, inp, t = case(B=1, L=2048, D=128, E=8, k=2, dtype="bf16", seed=11)
    _, _, g0 = run(t, w, chunk=0)
    _, _, g1 = run(t, w, chunk=0)
    for n in NAMES:
        assert torch.equal(g0[n], g1[n]), n
    _, _, g2 = run(t, w, chunk=96)
    for n in NAMES:
        assert rel_err(host(g2[n]), host(g0[n])) < 1e-4, n


def test_backward_degenerate():
    # L = 0: zero parameter gradients, dh0 = dh_final
    w, inp, t = case(B=2, L=0, D=70, E=4, k=2)
    idx = torch.zeros((2, 0, 2), dtype=torch.int32, device=DEV)
    gate = torch.zeros((2, 0, 2), dtype=torch.float32, device=DEV)
    g = swimba.scan_backward(t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"],
                             t["dt_bias"], t["Dskip"], t["dy"], dh_final=t["dhf"])
    assert torch.equal(g["dh0"], t["dhf"])
    assert torch.count_nonzero(g["dA"]) == 0 and torch.count_nonzero(g["ddt_bias"]) == 0
    # one token, one channel
    for (B, L, D) in ((1, 1, 64), (3, 5, 1)):
        w, inp, t = case(B=B, L=L, D=D, E=3, k=2, seed=B + L + D)
        idx, gate, g = run(t, w)
        check(g, reference(inp, idx, gate), TOL_F32)


def test_prepared_backward():
    w, inp, t = case(B=2, L=300, D=96, E=4, k=2, seed=13)
    idx, gate, g = run(t, w)
    out = {n: torch.empty_like(g[n]) for n in NAMES}
    call = swimba.PreparedBackward(t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"],
                                   t["dt_bias"], t["Dskip"], t["dy"], out, h0=t["h0"],
                                   dh_final=t["dhf"])
    call()
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(out[n], g[n]), n
