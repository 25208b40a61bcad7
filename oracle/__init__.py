"""fp64 CPU oracle for the Swimba parameter-space-MoE selective scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``parameter_space_moe_amd``) never imports it, and the two share no code:
the arithmetic lives in ``swimba_oracle.c`` (plain C, fp64, OpenMP over
independent channels), this module only marshals numpy arrays.

Each function cites, in ``swimba_oracle.c``, the passage of the pages it
follows: "Swimba: Switch Mamba Model Scales State Space Models" (the Dutch
summary's "Kernmechanisme van Swimba" for the mixed recurrence; the French
summary's "Fondements Théoriques" for Theorems 1-4) and "Mamba y las SSMs: el
retorno del estado persistente" (sections "SSMs" and "Mamba", Figure 2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swimba_oracle.c")
_SO = os.path.join(_HERE, "libswimba_oracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _SO) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load the oracle library (building it first only when nothing is built)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    so = path or _SO
    if not os.path.exists(so):
        build(force=True)
    lib = ctypes.CDLL(so)
    i64, ci = ctypes.c_int64, ctypes.c_int
    lib.ref_route.argtypes = [i64, ci, ci, ci, _f64p, _f64p, _i32p, _f64p, _f64p, _f64p]
    lib.ref_scan.argtypes = [ci] * 6 + [_f64p] * 4 + [_i32p] + [_f64p] * 7 + [ci]
    lib.ref_scan_separate.argtypes = [ci] * 6 + [_f64p] * 4 + [_i32p] + [_f64p] * 7 + [ci]
    lib.ref_scan_slots.argtypes = [ci] * 6 + [_f64p] * 4 + [_i32p] + [_f64p] * 7 + [ci]
    lib.ref_scan_all_experts.argtypes = [ci] * 6 + [_f64p] * 4 + [_i32p] + [_f64p] * 7 + [ci]
    lib.ref_mamba_scan.argtypes = [ci] * 4 + [_f64p] * 10 + [ci]
    lib.ref_scan_streams.argtypes = [ci] * 5 + [_f64p] * 10
    lib.ref_scan_backward.argtypes = [ci] * 6 + [_f64p] * 4 + [_i32p] + [_f64p] * 16
    lib.ref_step.argtypes = [ci] * 5 + [_f64p] * 5 + [_i32p] + [_f64p] * 6 + [_i32p, _f64p, ci]
    lib.ref_num_threads.restype = ci
    for f in (lib.ref_route, lib.ref_scan, lib.ref_scan_separate, lib.ref_scan_slots,
              lib.ref_scan_all_experts, lib.ref_mamba_scan,
              lib.ref_scan_streams, lib.ref_scan_backward, lib.ref_step):
        f.restype = None
    if path is None:
        _lib = lib
    return lib


def _d(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    if a is None:
        return None
    if a.dtype == np.int32:
        return a.ctypes.data_as(_i32p)
    return a.ctypes.data_as(_f64p)


def num_threads(lib=None) -> int:
    return int((lib or load()).ref_num_threads())


def route(x, Wr, k, lib=None):
    """Top-k router.  x [T, D], Wr [D, E] -> idx [T,k] int32, gate [T,k],
    logits [T,E], absdot [T,E] (sum_d |x_d Wr[d,e]|), all fp64."""
    lib = lib or load()
    x, Wr = _d(x), _d(Wr)
    T, D = x.shape
    E = Wr.shape[1]
    assert Wr.shape[0] == D and 1 <= k <= E
    idx = np.zeros((T, k), np.int32)
    gate = np.zeros((T, k))
    logits = np.zeros((T, E))
    absdot = np.zeros((T, E))
    lib.ref_route(T, D, E, k, _p(x), _p(Wr), _p(idx), _p(gate), _p(logits), _p(absdot))
    return idx, gate, logits, absdot


def _scan_common(fn, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, state_shape, zoh):
    x, dt_raw, Bm, Cm = _d(x), _d(dt_raw), _d(Bm), _d(Cm)
    idx, gate = _i(idx), _d(gate)
    A, dt_bias, Dskip = _d(A), _d(dt_bias), _d(Dskip)
    B, L, D = x.shape
    N = Bm.shape[2]
    E = A.shape[0]
    k = idx.shape[2]
    assert dt_raw.shape == x.shape and Bm.shape == (B, L, N) and Cm.shape == (B, L, N)
    assert idx.shape == (B, L, k) and gate.shape == (B, L, k)
    assert A.shape == (E, D, N) and dt_bias.shape == (E, D) and Dskip.shape == (E, D)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < E)
    shape = state_shape(B, E, D, N)
    h0 = None if h0 is None else _d(h0)
    if h0 is not None:
        assert h0.shape == shape
    y = np.zeros((B, L, D))
    hf = np.zeros(shape)
    fn(B, L, D, N, E, k, _p(x), _p(dt_raw), _p(Bm), _p(Cm), _p(idx), _p(gate), _p(A),
       _p(dt_bias), _p(Dskip), _p(h0), _p(y), _p(hf), 1 if zoh else 0)
    return y, hf


def scan(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, lib=None, zoh=False):
    """Mixed (parameter-space) scan.  Shapes: x, dt_raw [B,L,D]; Bm, Cm [B,L,N];
    idx, gate [B,L,k]; A [E,D,N]; dt_bias, Dskip [E,D]; h0 [B,D,N] or None.
    zoh: zero-order-hold input term instead of Euler.
    Returns y [B,L,D], h_final [B,D,N] (fp64)."""
    lib = lib or load()
    return _scan_common(lib.ref_scan, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0,
                        lambda B, E, D, N: (B, D, N), zoh)


def scan_separate(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, lib=None,
                  zoh=False):
    """Separate design: one state per expert.  h0, h_final [B,E,D,N]."""
    lib = lib or load()
    return _scan_common(lib.ref_scan_separate, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias,
                        Dskip, h0, lambda B, E, D, N: (B, E, D, N), zoh)


def scan_slots(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, lib=None, zoh=False):
    """Separate trajectories per routing slot: slot j's state advances at every
    token with the expert selected in slot j.  h0, h_final [B,k,D,N]."""
    lib = lib or load()
    k = np.shape(idx)[2]
    return _scan_common(lib.ref_scan_slots, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias,
                        Dskip, h0, lambda B, E, D, N: (B, k, D, N), zoh)


def scan_all_experts(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, lib=None,
                     zoh=False):
    """Separate trajectories where every expert advances at every token; the
    routing picks whose outputs are mixed.  h0, h_final [B,E,D,N]."""
    lib = lib or load()
    return _scan_common(lib.ref_scan_all_experts, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias,
                        Dskip, h0, lambda B, E, D, N: (B, E, D, N), zoh)


def scan_backward(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, dy, h0=None, dh_final=None,
                  lib=None):
    """Gradients of the mixed scan.  Inputs as ``scan`` plus dy [B,L,D] and
    dh_final [B,D,N] (None = 0).  Returns a dict of fp64 arrays: dx, ddt_raw
    [B,L,D]; dBm, dCm [B,L,N]; dgate [B,L,k]; dA [E,D,N]; dbias, dDskip [E,D];
    dh0 [B,D,N]."""
    lib = lib or load()
    x, dt_raw, Bm, Cm = _d(x), _d(dt_raw), _d(Bm), _d(Cm)
    idx, gate = _i(idx), _d(gate)
    A, dt_bias, Dskip, dy = _d(A), _d(dt_bias), _d(Dskip), _d(dy)
    B, L, D = x.shape
    N = Bm.shape[2]
    E = A.shape[0]
    k = idx.shape[2]
    assert dy.shape == x.shape and A.shape == (E, D, N) and idx.shape == (B, L, k)
    h0 = None if h0 is None else _d(h0)
    dh_final = None if dh_final is None else _d(dh_final)
    out = dict(dx=np.zeros((B, L, D)), ddt_raw=np.zeros((B, L, D)), dBm=np.zeros((B, L, N)),
               dCm=np.zeros((B, L, N)), dgate=np.zeros((B, L, k)), dA=np.zeros((E, D, N)),
               dbias=np.zeros((E, D)), dDskip=np.zeros((E, D)), dh0=np.zeros((B, D, N)))
    lib.ref_scan_backward(B, L, D, N, E, k, _p(x), _p(dt_raw), _p(Bm), _p(Cm), _p(idx),
                          _p(gate), _p(A), _p(dt_bias), _p(Dskip), _p(h0), _p(dy),
                          _p(dh_final), *[_p(out[n]) for n in ("dx", "ddt_raw", "dBm", "dCm",
                                                                 "dgate", "dA", "dbias",
                                                                 "dDskip", "dh0")])
    return out


def mamba_scan(x, dt_raw, Bm, Cm, A, dt_bias, Dskip, h0=None, lib=None, zoh=False):
    """Plain single-expert selective scan.  A [D,N], dt_bias, Dskip [D]."""
    lib = lib or load()
    x, dt_raw, Bm, Cm = _d(x), _d(dt_raw), _d(Bm), _d(Cm)
    A, dt_bias, Dskip = _d(A), _d(dt_bias), _d(Dskip)
    B, L, D = x.shape
    N = Bm.shape[2]
    assert A.shape == (D, N) and dt_bias.shape == (D,) and Dskip.shape == (D,)
    h0 = None if h0 is None else _d(h0)
    y = np.zeros((B, L, D))
    hf = np.zeros((B, D, N))
    lib.ref_mamba_scan(B, L, D, N, _p(x), _p(dt_raw), _p(Bm), _p(Cm), _p(A), _p(dt_bias),
                       _p(Dskip), _p(h0), _p(y), _p(hf), 1 if zoh else 0)
    return y, hf


def scan_streams(X, dt_raw, Bs, Cs, gate, A, dt_bias, h0=None, lib=None):
    """Stream-mixed scan (shared A; mixed B X injection and C readout).
    Shapes: X [B,L,k,D]; dt_raw [B,L,D]; Bs, Cs [B,L,k,N]; gate [B,L,k];
    A [D,N]; dt_bias [D]; h0 [B,D,N] or None.  Returns y [B,L,D], h_final
    [B,D,N] (fp64)."""
    lib = lib or load()
    X, dt_raw, Bs, Cs, gate = _d(X), _d(dt_raw), _d(Bs), _d(Cs), _d(gate)
    A, dt_bias = _d(A), _d(dt_bias)
    B, L, k, D = X.shape
    N = Bs.shape[3]
    assert dt_raw.shape == (B, L, D) and Bs.shape == (B, L, k, N) and Cs.shape == (B, L, k, N)
    assert gate.shape == (B, L, k) and A.shape == (D, N) and dt_bias.shape == (D,)
    h0 = None if h0 is None else _d(h0)
    if h0 is not None:
        assert h0.shape == (B, D, N)
    y = np.zeros((B, L, D))
    hf = np.zeros((B, D, N))
    lib.ref_scan_streams(B, L, D, N, k, _p(X), _p(dt_raw), _p(Bs), _p(Cs), _p(gate), _p(A),
                         _p(dt_bias), _p(h0), _p(y), _p(hf))
    return y, hf


def step(x, dt_raw, Bm, Cm, A, dt_bias, Dskip, state, Wr=None, k=None, idx=None, gate=None,
         lib=None, zoh=False):
    """One decode step.  x, dt_raw [B,D]; Bm, Cm [B,N]; state [B,D,N] fp64,
    updated IN PLACE.  Routing from Wr [D,E] with top-k, or forced idx/gate
    [B,k].  Returns y [B,D], idx [B,k], gate [B,k]."""
    lib = lib or load()
    assert isinstance(state, np.ndarray) and state.dtype == np.float64 and state.flags.c_contiguous
    x, dt_raw, Bm, Cm = _d(x), _d(dt_raw), _d(Bm), _d(Cm)
    A, dt_bias, Dskip = _d(A), _d(dt_bias), _d(Dskip)
    B, D = x.shape
    N = Bm.shape[1]
    E = A.shape[0]
    if idx is not None:
        idx, gate = _i(idx), _d(gate)
        k = idx.shape[1]
        Wr_p = None
    else:
        Wr = _d(Wr)
        Wr_p = _p(Wr)
    assert state.shape == (B, D, N) and 1 <= k <= E
    y = np.zeros((B, D))
    idx_out = np.zeros((B, k), np.int32)
    gate_out = np.zeros((B, k))
    lib.ref_step(B, D, N, E, k, _p(x), _p(dt_raw), _p(Bm), _p(Cm), Wr_p, _p(idx), _p(gate),
                 _p(A), _p(dt_bias), _p(Dskip), _p(state), _p(y), _p(idx_out), _p(gate_out),
                 1 if zoh else 0)
    return y, idx_out, gate_out
