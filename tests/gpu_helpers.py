"""Shared helpers of the GPU parity tests: device copies of the seeded
workloads, the error metric, and the router comparison with certified
near-ties.  Nothing here computes the method; the expected values come from
the oracle."""
from __future__ import annotations

import math

import numpy as np
import torch

U32 = 2.0 ** -24

# Parity bars.  fp32 inputs: 1e-4; bf16 inputs with fp32 accumulation: 2e-3.
# bf16 outputs are checked for faithful rounding (within one bf16 ulp of the
# correctly rounded reference) instead, because bf16's own unit round-off
# (2^-8) exceeds the bf16-input bar.
TOL_F32 = 1e-4
TOL_BF16 = 2e-3


def dev_tensors(inp: dict, dtype: str, device="cuda"):
    """numpy workload arrays -> device tensors; streams in the workload dtype,
    parameters fp32."""
    out = {}
    for k, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k in ("x", "dt_raw", "Bm", "Cm") and dtype == "bf16":
            t = t.to(torch.bfloat16)  # values are already bf16-representable
        out[k] = t.to(device)
    return out


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    """max_i |got_i - ref_i| / max(|ref_i|, rms(ref))."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    e = np.abs(got - ref) / den
    if np.any(np.isnan(got) != np.isnan(ref)):
        return float("inf")
    return float(np.nanmax(e))


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(v).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def bf16_rne(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(v, np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.float().numpy().astype(np.float64)


def assert_faithful_bf16(got_bf16: torch.Tensor, ref: np.ndarray, what="", tol=TOL_F32):
    """bf16 outputs are faithful roundings of values within the fp32 bar of
    the reference: |got - ref| <= ulp_bf16 + tol * max(|ref|, rms(ref)).  The
    second term is the fp32 arithmetic's own error, which scales with the
    signal (rms), not with an output that happens to lie near zero."""
    got = host(got_bf16)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref))) if ref.size else 1.0
    allow = bf16_ulp(np.maximum(np.abs(got), np.abs(ref))) + \
        tol * np.maximum(np.abs(ref), rms)
    err = np.abs(got - ref)
    bad = ~(err <= allow)
    if bad.any():
        i = np.argsort((err / allow).ravel())[::-1][:5]
        raise AssertionError("%s: %d bf16 outputs outside the bar; worst (got, ref): %s" % (
            what, int(bad.sum()), list(zip(got.ravel()[i].tolist(), ref.ravel()[i].tolist()))))


def route_tolerance(absdot: np.ndarray, D: int) -> np.ndarray:
    """Bound on |fp32 logit - exact logit| for the routers' summations: each
    lane sums at most ceil(D/64) products in order and the partial sums are
    combined in at most 8 more levels (gamma_m * sum_d |x_d Wr[d,e]|,
    m = ceil(D/64) + 8)."""
    m = -(-D // 64) + 8
    gamma = m * U32 / (1 - m * U32)
    return gamma * absdot


def check_route(idx_gpu, logits, tol, k) -> int:
    """idx must match the oracle's top-k wherever the ranking is certain; at
    certified near-ties any order consistent with the tolerance is accepted.
    Returns the number of near-tie tokens."""
    T, E = logits.shape
    ties = 0
    order = np.lexsort((np.tile(np.arange(E), (T, 1)), -logits), axis=1)
    for t in range(T):
        o = order[t]
        top = o[:k]
        look = o[:min(k + 1, E)]
        amb = any(logits[t, a] - logits[t, b] <= tol[t, a] + tol[t, b]
                  for a, b in zip(look[:-1], look[1:]))
        gi = idx_gpu[t]
        if not amb:
            assert list(gi) == list(top), (t, list(gi), list(top), logits[t])
            continue
        ties += 1
        assert len(set(gi.tolist())) == k and all(0 <= e < E for e in gi)
        sel = set(gi.tolist())
        for s_ in sel:        # every selected expert could be in the top k
            for u in set(range(E)) - sel:
                assert logits[t, s_] + tol[t, s_] >= logits[t, u] - tol[t, u], (t, s_, u)
        for a, b in zip(gi[:-1], gi[1:]):  # and the slot order is possible
            assert logits[t, a] + tol[t, a] >= logits[t, b] - tol[t, b], (t, a, b)
    return ties


def gate_bound(idx, tol):
    """Bound on |gate error| given logit errors within `tol`: a softmax output
    moves by at most half the largest logit error (|d g_j / d l| sums to
    2 g_j (1 - g_j) <= 1/2), plus a few fp32 roundings of exp and divide."""
    sel_tol = np.take_along_axis(tol, idx.astype(np.int64), axis=1)
    return 3e-7 + 0.5 * sel_tol.max(axis=1, keepdims=True)


class HipEvents:
    """Timing events through the HIP runtime's C API (for the scans'
    phase_events argument, which takes raw hipEvent_t handles)."""

    def __init__(self, n):
        import ctypes
        self._ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e)
        self.array = (ctypes.c_void_p * n)(*[e.value for e in self.ev])

    @property
    def address(self):
        return self._ct.addressof(self.array)

    def ms(self, i, j):
        v = self._ct.c_float()
        rc = self.lib.hipEventElapsedTime(self._ct.byref(v), self.ev[i], self.ev[j])
        assert rc == 0, rc
        return float(v.value)

    def close(self):
        for e in self.ev:
            self.lib.hipEventDestroy(e)
