"""Python binding of libswimba.so: the same entry points as include/swimba.h,
taking torch tensors.  Argument marshalling only -- every step of the
computation runs in the HIP kernels; torch provides device memory and the
current stream.  There is no fallback: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswimba.so")

F32, BF16 = 0, 1
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5
# fixed chunk-workspace buffer of swimba_scan_noalloc (SWIMBA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20
CARRY = {"auto": 0, "rewalk": 1, "fixup": 2}
A_DIAGONAL, A_SCALAR = 0, 1  # A [E, D, N] or [E, D] (one transition per channel)
DISC_EULER, DISC_ZOH = 0, 1  # input term Delta B x, or zero-order hold
N_STATE = 16

_vp = ctypes.c_void_p
_ci = ctypes.c_int


class ScanArgs(ctypes.Structure):
    _fields_ = [("B", _ci), ("L", _ci), ("D", _ci), ("N", _ci), ("E", _ci), ("k", _ci),
                ("in_dtype", _ci), ("y_dtype", _ci),
                ("x", _vp), ("dt_raw", _vp), ("Bm", _vp), ("Cm", _vp),
                ("idx", _vp), ("gate", _vp), ("A", _vp), ("dt_bias", _vp), ("Dskip", _vp),
                ("h0", _vp), ("y", _vp), ("h_final", _vp),
                ("chunk", _ci), ("carry", _ci), ("phase_events", _vp), ("a_form", _ci),
                ("disc", _ci)]


class StepArgs(ctypes.Structure):
    _fields_ = [("B", _ci), ("D", _ci), ("N", _ci), ("E", _ci), ("k", _ci),
                ("in_dtype", _ci), ("y_dtype", _ci),
                ("x", _vp), ("dt_raw", _vp), ("Bm", _vp), ("Cm", _vp),
                ("Wr", _vp), ("idx", _vp), ("gate", _vp), ("idx_out", _vp), ("gate_out", _vp),
                ("A", _vp), ("dt_bias", _vp), ("Dskip", _vp), ("state", _vp), ("y", _vp),
                ("a_form", _ci), ("disc", _ci)]


class GradArgs(ctypes.Structure):
    _fields_ = [("fwd", ScanArgs), ("dy", _vp), ("dy_dtype", _ci), ("dh_final", _vp),
                ("dx", _vp), ("ddt_raw", _vp), ("dBm", _vp), ("dCm", _vp), ("dgate", _vp),
                ("dA", _vp), ("ddt_bias", _vp), ("dDskip", _vp), ("dh0", _vp)]


class StreamArgs(ctypes.Structure):
    _fields_ = [("B", _ci), ("L", _ci), ("D", _ci), ("N", _ci), ("k", _ci),
                ("in_dtype", _ci), ("y_dtype", _ci),
                ("X", _vp), ("dt_raw", _vp), ("Bs", _vp), ("Cs", _vp), ("gate", _vp),
                ("A", _vp), ("dt_bias", _vp), ("h0", _vp), ("y", _vp), ("h_final", _vp),
                ("chunk", _ci), ("carry", _ci), ("phase_events", _vp)]


class SwimbaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))
        self.status = status


_lib = None


def load(path: str | None = None):
    """Load libswimba.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    so = path or LIB_PATH
    if not os.path.exists(so):
        raise ImportError("libswimba.so is not built (%s); run __graft_entry__.build() or "
                          "python parameter_space_moe_amd/build.py" % so)
    lib = ctypes.CDLL(so)
    lib.swimba_route.argtypes = [_vp, _ci, _vp, ctypes.c_int64, _ci, _ci, _ci, _vp, _vp, _vp]
    lib.swimba_route.restype = _ci
    lib.swimba_scan_workspace_size.argtypes = [ctypes.POINTER(ScanArgs), _ci]
    lib.swimba_scan_workspace_size.restype = ctypes.c_size_t
    for fn in (lib.swimba_scan, lib.swimba_scan_separate, lib.swimba_scan_slots,
               lib.swimba_scan_all_experts):
        fn.argtypes = [ctypes.POINTER(ScanArgs), _vp, ctypes.c_size_t, _vp]
        fn.restype = _ci
    lib.swimba_scan_noalloc.argtypes = [ctypes.POINTER(ScanArgs), _vp]
    lib.swimba_scan_noalloc.restype = _ci
    lib.swimba_scan_plan.argtypes = [ctypes.POINTER(ScanArgs), _ci, ctypes.POINTER(_ci),
                                     ctypes.POINTER(_ci)]
    lib.swimba_scan_plan.restype = _ci
    lib.swimba_scan_streams_workspace_size.argtypes = [ctypes.POINTER(StreamArgs)]
    lib.swimba_scan_streams_workspace_size.restype = ctypes.c_size_t
    lib.swimba_scan_streams_plan.argtypes = [ctypes.POINTER(StreamArgs), ctypes.POINTER(_ci),
                                             ctypes.POINTER(_ci)]
    lib.swimba_scan_streams_plan.restype = _ci
    lib.swimba_scan_streams.argtypes = [ctypes.POINTER(StreamArgs), _vp, ctypes.c_size_t, _vp]
    lib.swimba_scan_streams.restype = _ci
    lib.swimba_scan_backward_workspace_size.argtypes = [ctypes.POINTER(GradArgs)]
    lib.swimba_scan_backward_workspace_size.restype = ctypes.c_size_t
    lib.swimba_scan_backward.argtypes = [ctypes.POINTER(GradArgs), _vp, ctypes.c_size_t, _vp]
    lib.swimba_scan_backward.restype = _ci
    lib.swimba_step.argtypes = [ctypes.POINTER(StepArgs), _vp]
    lib.swimba_step.restype = _ci
    lib.swimba_status_string.argtypes = [_ci]
    lib.swimba_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().swimba_status_string(status).decode()


def _check(fn, rc):
    if rc != OK:
        raise SwimbaError(fn, rc)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, shape=None, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _hold(stream, *tensors):
    """Temporaries allocated here for a call on the caller's stream: the
    caching allocator must not hand them out again before that stream's
    work has run (allocation is ordered on the current stream only)."""
    if stream is not None:
        for t in tensors:
            t.record_stream(stream)


def route(x: torch.Tensor, Wr: torch.Tensor, k: int, idx=None, gate=None, stream=None):
    """Top-k router: x [..., D] (f32/bf16), Wr [D, E] f32 -> idx [..., k] int32,
    gate [..., k] f32 (include/swimba.h: swimba_route)."""
    _need(x, "x")
    D = x.shape[-1]
    E = Wr.shape[1] if Wr.dim() == 2 else -1
    _need(Wr, "Wr", (D, E), torch.float32, x.device)
    T = x.numel() // D if D else 0
    lead = tuple(x.shape[:-1])
    if idx is None:
        idx = torch.empty(lead + (k,), dtype=torch.int32, device=x.device)
    if gate is None:
        gate = torch.empty(lead + (k,), dtype=torch.float32, device=x.device)
    _need(idx, "idx", lead + (k,), torch.int32, x.device)
    _need(gate, "gate", lead + (k,), torch.float32, x.device)
    rc = load().swimba_route(_ptr(x), _dt(x), _ptr(Wr), T, D, E, k, _ptr(idx), _ptr(gate),
                             _stream(stream))
    _check("swimba_route", rc)
    return idx, gate


def _scan_args(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, y, h_final, chunk, carry,
               design, phase_events, need_y=True, zoh=False):
    _need(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [B, L, D]")
    B, L, D = x.shape
    E = A.shape[0]
    N = Bm.shape[2] if Bm.dim() == 3 else -1
    k = idx.shape[2] if idx.dim() == 3 else -1
    dev = x.device
    _need(dt_raw, "dt_raw", (B, L, D), x.dtype, dev)
    _need(Bm, "Bm", (B, L, N), x.dtype, dev)
    _need(Cm, "Cm", (B, L, N), x.dtype, dev)
    _need(idx, "idx", (B, L, k), torch.int32, dev)
    _need(gate, "gate", (B, L, k), torch.float32, dev)
    scalar_a = A.dim() == 2
    _need(A, "A", (E, D) if scalar_a else (E, D, N), torch.float32, dev)
    _need(dt_bias, "dt_bias", (E, D), torch.float32, dev)
    _need(Dskip, "Dskip", (E, D), torch.float32, dev)
    sshape = _state_shape(design, B, E, k, D, N)
    if h0 is not None:
        _need(h0, "h0", sshape, torch.float32, dev)
    if need_y:
        _need(y, "y", (B, L, D), None, dev)
    if h_final is not None:
        _need(h_final, "h_final", sshape, torch.float32, dev)
    a = ScanArgs()
    a.B, a.L, a.D, a.N, a.E, a.k = B, L, D, N, E, k
    a.in_dtype, a.y_dtype = _dt(x), (_dt(y) if y is not None else _dt(x))
    a.x, a.dt_raw, a.Bm, a.Cm = _ptr(x), _ptr(dt_raw), _ptr(Bm), _ptr(Cm)
    a.idx, a.gate, a.A, a.dt_bias, a.Dskip = _ptr(idx), _ptr(gate), _ptr(A), _ptr(dt_bias), \
        _ptr(Dskip)
    a.h0, a.y, a.h_final = _ptr(h0), _ptr(y), _ptr(h_final)
    a.chunk = int(chunk)
    a.carry = CARRY[carry] if isinstance(carry, str) else int(carry)
    a.phase_events = phase_events
    a.a_form = A_SCALAR if scalar_a else A_DIAGONAL
    a.disc = DISC_ZOH if zoh else DISC_EULER
    return a


# Which scan (SWIMBA_DESIGN_* in include/swimba.h); a bool `separate` reads as
# MIXED (False) or SEPARATE (True).
DESIGN_MIXED, DESIGN_SEPARATE, DESIGN_SLOTS, DESIGN_ALL_EXPERTS = 0, 1, 2, 3
_SCAN_FN = {DESIGN_MIXED: "swimba_scan", DESIGN_SEPARATE: "swimba_scan_separate",
            DESIGN_SLOTS: "swimba_scan_slots", DESIGN_ALL_EXPERTS: "swimba_scan_all_experts"}


def _state_shape(design, B, E, k, D, N=N_STATE):
    """h0 / h_final shape: one state per (b, d), per (b, expert, d) or per
    (b, slot, d)."""
    design = int(design)
    if design in (DESIGN_SEPARATE, DESIGN_ALL_EXPERTS):
        return (B, E, D, N)
    if design == DESIGN_SLOTS:
        return (B, k, D, N)
    return (B, D, N)


def workspace_size(args: ScanArgs, design) -> int:
    return int(load().swimba_scan_workspace_size(ctypes.byref(args), int(design)))


def _scan(design, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, y=None,
          h_final=None, y_dtype=None, want_state=True, chunk=0, carry="auto", workspace=None,
          stream=None, phase_events=None, zoh=False):
    design = int(design)
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    if h_final is None and want_state:
        shape = _state_shape(design, x.shape[0], A.shape[0], idx.shape[-1], x.shape[2])
        h_final = torch.empty(shape, dtype=torch.float32, device=x.device)
    a = _scan_args(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, y, h_final, chunk, carry,
                   design, phase_events, zoh=zoh)
    lib = load()
    need = workspace_size(a, design)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
        _hold(stream, workspace)
    name = _SCAN_FN[design]
    rc = getattr(lib, name)(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(name, rc)
    return y, h_final


def scan(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, **kw):
    """Parameter-space-mixed scan (include/swimba.h: swimba_scan).  A is
    [E,D,16], or [E,D] for one transition per channel (the scalar form).
    Returns (y [B,L,D], h_final [B,D,16] or None)."""
    return _scan(False, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, **kw)


def scan_noalloc(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, y=None,
                 h_final=None, y_dtype=None, want_state=True, chunk=0, carry="auto",
                 stream=None, zoh=False):
    """The mixed scan with its chunk workspace in the library's fixed buffer
    (include/swimba.h: swimba_scan_noalloc): no workspace is allocated for
    the call.  Outputs y and h_final are allocated here unless given.
    Returns (y [B,L,D], h_final [B,D,16] or None)."""
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    if h_final is None and want_state:
        h_final = torch.empty((x.shape[0], x.shape[2], N_STATE), dtype=torch.float32,
                              device=x.device)
    a = _scan_args(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, y, h_final, chunk, carry,
                   DESIGN_MIXED, None, zoh=zoh)
    rc = load().swimba_scan_noalloc(ctypes.byref(a), _stream(stream))
    _check("swimba_scan_noalloc", rc)
    return y, h_final


def scan_separate(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, **kw):
    """Separate design (include/swimba.h: swimba_scan_separate).  Returns
    (y [B,L,D], h_final [B,E,D,16] or None)."""
    return _scan(DESIGN_SEPARATE, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, **kw)


def scan_slots(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, **kw):
    """Separate trajectories per routing slot (include/swimba.h:
    swimba_scan_slots).  Returns (y [B,L,D], h_final [B,k,D,16] or None)."""
    return _scan(DESIGN_SLOTS, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, **kw)


def scan_all_experts(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None, **kw):
    """Separate trajectories where every expert advances at every token
    (include/swimba.h: swimba_scan_all_experts).  Returns (y [B,L,D],
    h_final [B,E,D,16] or None)."""
    return _scan(DESIGN_ALL_EXPERTS, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, **kw)


def _grad_args(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, dy, h0, dh_final, chunk,
               out):
    a = _scan_args(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, None, None, chunk,
                   "auto", False, None, need_y=False)
    B, L, D = x.shape
    E, k = A.shape[0], idx.shape[2]
    N = Bm.shape[2]
    dev = x.device
    _need(dy, "dy", (B, L, D), None, dev)
    if dh_final is not None:
        _need(dh_final, "dh_final", (B, D, N), torch.float32, dev)
    shapes = {"dx": (B, L, D), "ddt_raw": (B, L, D), "dBm": (B, L, N), "dCm": (B, L, N),
              "dgate": (B, L, k), "dA": tuple(A.shape), "ddt_bias": (E, D), "dDskip": (E, D),
              "dh0": (B, D, N)}
    for name, shape in shapes.items():
        if out.get(name) is not None:
            _need(out[name], name, shape, torch.float32, dev)
    g = GradArgs()
    g.fwd = a
    g.dy, g.dy_dtype, g.dh_final = _ptr(dy), _dt(dy), _ptr(dh_final)
    for name in shapes:
        setattr(g, name, _ptr(out.get(name)))
    return g


def scan_backward(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, dy, h0=None, dh_final=None,
                  chunk=0, want_dh0=True, out=None, workspace=None, stream=None):
    """Gradients of the mixed scan (include/swimba.h: swimba_scan_backward) for
    dL/dy = dy (and dL/dh_final).  Returns a dict of fp32 tensors: dx,
    ddt_raw [B,L,D]; dBm, dCm [B,L,16]; dgate [B,L,k]; dA [E,D,16]; ddt_bias,
    dDskip [E,D]; dh0 [B,D,16] (when want_dh0)."""
    B, L, D = x.shape
    E, k, N = A.shape[0], idx.shape[2], N_STATE
    dev = x.device
    out = dict(out or {})
    shapes = {"dx": (B, L, D), "ddt_raw": (B, L, D), "dBm": (B, L, N), "dCm": (B, L, N),
              "dgate": (B, L, k), "dA": tuple(A.shape), "ddt_bias": (E, D), "dDskip": (E, D)}
    if want_dh0:
        shapes["dh0"] = (B, D, N)
    for name, shape in shapes.items():
        if out.get(name) is None:
            out[name] = torch.empty(shape, dtype=torch.float32, device=dev)
    g = _grad_args(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, dy, h0, dh_final, chunk, out)
    lib = load()
    need = int(lib.swimba_scan_backward_workspace_size(ctypes.byref(g)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _hold(stream, workspace)
    rc = lib.swimba_scan_backward(ctypes.byref(g), _ptr(workspace), workspace.numel(),
                                  _stream(stream))
    _check("swimba_scan_backward", rc)
    return out


class PreparedBackward:
    """swimba_scan_backward marshalled once (see PreparedScan)."""

    def __init__(self, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, dy, out, h0=None,
                 dh_final=None, chunk=0, workspace=None, stream=None):
        self.args = _grad_args(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, dy, h0, dh_final,
                               chunk, out)
        lib = load()
        need = int(lib.swimba_scan_backward_workspace_size(ctypes.byref(self.args)))
        self.workspace = workspace if workspace is not None else torch.empty(
            max(need, 1), dtype=torch.uint8, device=x.device)
        self._keep = (x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, dy, h0, dh_final, out)
        self._fn = lib.swimba_scan_backward
        self._ref = ctypes.byref(self.args)
        self._ws = self.workspace.data_ptr()
        self._wsn = self.workspace.numel()
        self.stream = _stream(stream)

    def __call__(self):
        rc = self._fn(self._ref, self._ws, self._wsn, self.stream)
        if rc != OK:
            raise SwimbaError("swimba_scan_backward", rc)


def _shape_args(x, A, idx, chunk, y_dtype):
    B, L, D = x.shape
    a = ScanArgs()
    a.B, a.L, a.D, a.N, a.E, a.k = B, L, D, N_STATE, A.shape[0], idx.shape[2]
    a.a_form = A_SCALAR if A.dim() == 2 else A_DIAGONAL
    a.in_dtype = _dt(x)
    a.y_dtype = a.in_dtype if y_dtype is None else (BF16 if y_dtype == torch.bfloat16 else F32)
    a.chunk = chunk
    return a


def scan_workspace_bytes(x, A, idx, separate=False, chunk=0, y_dtype=None):
    """Workspace bytes the scan named by `separate` (a DESIGN_* value, or a
    bool for mixed / separate) needs for these shapes."""
    return workspace_size(_shape_args(x, A, idx, chunk, y_dtype), separate)


def scan_plan(x, A, idx, separate=False, chunk=0):
    """(tokens per chunk, number of chunks) the scan will use (swimba_scan_plan);
    `separate` as in scan_workspace_bytes."""
    c, n = _ci(), _ci()
    rc = load().swimba_scan_plan(ctypes.byref(_shape_args(x, A, idx, chunk, None)),
                                 int(separate), ctypes.byref(c), ctypes.byref(n))
    _check("swimba_scan_plan", rc)
    return c.value, n.value


class PreparedScan:
    """A scan call marshalled once (argument struct, workspace) for callers
    that issue the same call repeatedly; __call__ goes straight to the C ABI."""

    def __init__(self, separate, x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0=None,
                 y=None, h_final=None, chunk=0, carry="auto", workspace=None, stream=None,
                 zoh=False):
        # separate: a DESIGN_* value, or a bool for mixed / separate
        design = int(separate)
        self.args = _scan_args(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, y, h_final,
                               chunk, carry, design, None, zoh=zoh)
        need = workspace_size(self.args, design)
        self.workspace = workspace if workspace is not None else torch.empty(
            max(need, 1), dtype=torch.uint8, device=x.device)
        self._keep = (x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, y, h_final)
        lib = load()
        self._name = _SCAN_FN[design]
        self._fn = getattr(lib, self._name)
        self._ref = ctypes.byref(self.args)
        self._ws = self.workspace.data_ptr()
        self._wsn = self.workspace.numel()
        self.stream = _stream(stream)

    def __call__(self, phase_events=None):
        self.args.phase_events = phase_events
        rc = self._fn(self._ref, self._ws, self._wsn, self.stream)
        if rc != OK:
            raise SwimbaError(self._name, rc)


def _stream_args(X, dt_raw, Bs, Cs, gate, A, dt_bias, h0, y, h_final, chunk, carry,
                 phase_events):
    _need(X, "X")
    if X.dim() != 4:
        raise ValueError("X must be [B, L, k, D]")
    B, L, k, D = X.shape
    N = A.shape[1] if A.dim() == 2 else -1
    dev = X.device
    _need(dt_raw, "dt_raw", (B, L, D), X.dtype, dev)
    _need(Bs, "Bs", (B, L, k, N), X.dtype, dev)
    _need(Cs, "Cs", (B, L, k, N), X.dtype, dev)
    _need(gate, "gate", (B, L, k), torch.float32, dev)
    _need(A, "A", (D, N), torch.float32, dev)
    _need(dt_bias, "dt_bias", (D,), torch.float32, dev)
    if h0 is not None:
        _need(h0, "h0", (B, D, N), torch.float32, dev)
    _need(y, "y", (B, L, D), None, dev)
    if h_final is not None:
        _need(h_final, "h_final", (B, D, N), torch.float32, dev)
    a = StreamArgs()
    a.B, a.L, a.D, a.N, a.k = B, L, D, N, k
    a.in_dtype, a.y_dtype = _dt(X), _dt(y)
    a.X, a.dt_raw, a.Bs, a.Cs, a.gate = _ptr(X), _ptr(dt_raw), _ptr(Bs), _ptr(Cs), _ptr(gate)
    a.A, a.dt_bias, a.h0, a.y, a.h_final = _ptr(A), _ptr(dt_bias), _ptr(h0), _ptr(y), \
        _ptr(h_final)
    a.chunk = int(chunk)
    a.carry = CARRY[carry] if isinstance(carry, str) else int(carry)
    a.phase_events = phase_events
    return a


def scan_streams(X, dt_raw, Bs, Cs, gate, A, dt_bias, h0=None, y=None, h_final=None,
                 y_dtype=None, want_state=True, chunk=0, carry="auto", workspace=None,
                 stream=None, phase_events=None):
    """Stream-mixed scan (include/swimba.h: swimba_scan_streams).  X [B,L,k,D];
    dt_raw [B,L,D]; Bs, Cs [B,L,k,16]; gate [B,L,k] f32; A [D,16], dt_bias [D]
    f32.  Returns (y [B,L,D], h_final [B,D,16] or None)."""
    B, L, k, D = X.shape
    if y is None:
        y = torch.empty((B, L, D), dtype=y_dtype or X.dtype, device=X.device)
    if h_final is None and want_state:
        h_final = torch.empty((B, D, N_STATE), dtype=torch.float32, device=X.device)
    a = _stream_args(X, dt_raw, Bs, Cs, gate, A, dt_bias, h0, y, h_final, chunk, carry,
                     phase_events)
    lib = load()
    need = int(lib.swimba_scan_streams_workspace_size(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
        _hold(stream, workspace)
    rc = lib.swimba_scan_streams(ctypes.byref(a), _ptr(workspace), workspace.numel(),
                                 _stream(stream))
    _check("swimba_scan_streams", rc)
    return y, h_final


def scan_streams_plan(X, chunk=0):
    """(tokens per chunk, number of chunks) of swimba_scan_streams for X [B,L,k,D]."""
    a = StreamArgs()
    a.B, a.L, a.k, a.D = X.shape
    a.N = N_STATE
    a.in_dtype = a.y_dtype = _dt(X)
    a.chunk = chunk
    c, n = _ci(), _ci()
    rc = load().swimba_scan_streams_plan(ctypes.byref(a), ctypes.byref(c), ctypes.byref(n))
    _check("swimba_scan_streams_plan", rc)
    return c.value, n.value


class PreparedStreams:
    """swimba_scan_streams marshalled once (see PreparedScan)."""

    def __init__(self, X, dt_raw, Bs, Cs, gate, A, dt_bias, h0=None, y=None, h_final=None,
                 chunk=0, carry="auto", workspace=None, stream=None):
        self.args = _stream_args(X, dt_raw, Bs, Cs, gate, A, dt_bias, h0, y, h_final, chunk,
                                 carry, None)
        lib = load()
        need = int(lib.swimba_scan_streams_workspace_size(ctypes.byref(self.args)))
        self.workspace = workspace if workspace is not None else torch.empty(
            max(need, 1), dtype=torch.uint8, device=X.device)
        self._keep = (X, dt_raw, Bs, Cs, gate, A, dt_bias, h0, y, h_final)
        self._fn = lib.swimba_scan_streams
        self._ref = ctypes.byref(self.args)
        self._ws = self.workspace.data_ptr()
        self._wsn = self.workspace.numel()
        self.stream = _stream(stream)

    def __call__(self, phase_events=None):
        self.args.phase_events = phase_events
        rc = self._fn(self._ref, self._ws, self._wsn, self.stream)
        if rc != OK:
            raise SwimbaError("swimba_scan_streams", rc)


class PreparedRoute:
    """swimba_route marshalled once (see PreparedScan)."""

    def __init__(self, x, Wr, k, idx, gate, stream=None):
        _need(x, "x")
        D = x.shape[-1]
        E = Wr.shape[1]
        _need(Wr, "Wr", (D, E), torch.float32, x.device)
        lead = tuple(x.shape[:-1])
        _need(idx, "idx", lead + (k,), torch.int32, x.device)
        _need(gate, "gate", lead + (k,), torch.float32, x.device)
        self._keep = (x, Wr, idx, gate)
        self._a = (x.data_ptr(), _dt(x), Wr.data_ptr(), x.numel() // D, D, E, k, idx.data_ptr(),
                   gate.data_ptr(), _stream(stream))
        self._fn = load().swimba_route

    def __call__(self):
        rc = self._fn(*self._a)
        if rc != OK:
            raise SwimbaError("swimba_route", rc)


def _step_args(x, dt_raw, Bm, Cm, A, dt_bias, Dskip, state, Wr, k, idx, gate, y, idx_out,
               gate_out, y_dtype, zoh=False):
    _need(x, "x")
    B, D = x.shape
    E = A.shape[0]
    N = Bm.shape[1] if Bm.dim() == 2 else -1
    dev = x.device
    _need(dt_raw, "dt_raw", (B, D), x.dtype, dev)
    _need(Bm, "Bm", (B, N), x.dtype, dev)
    _need(Cm, "Cm", (B, N), x.dtype, dev)
    scalar_a = A.dim() == 2
    _need(A, "A", (E, D) if scalar_a else (E, D, N), torch.float32, dev)
    _need(dt_bias, "dt_bias", (E, D), torch.float32, dev)
    _need(Dskip, "Dskip", (E, D), torch.float32, dev)
    _need(state, "state", (B, D, N), torch.float32, dev)
    if idx is not None:
        k = idx.shape[1]
        _need(idx, "idx", (B, k), torch.int32, dev)
        _need(gate, "gate", (B, k), torch.float32, dev)
    else:
        if Wr is None or k is None:
            raise ValueError("step needs Wr and k, or idx and gate")
        _need(Wr, "Wr", (D, E), torch.float32, dev)
    if y is None:
        y = torch.empty((B, D), dtype=y_dtype or x.dtype, device=dev)
    _need(y, "y", (B, D), None, dev)
    if idx_out is not None:
        _need(idx_out, "idx_out", (B, k), torch.int32, dev)
    if gate_out is not None:
        _need(gate_out, "gate_out", (B, k), torch.float32, dev)
    a = StepArgs()
    a.B, a.D, a.N, a.E, a.k = B, D, N, E, k
    a.in_dtype, a.y_dtype = _dt(x), _dt(y)
    a.x, a.dt_raw, a.Bm, a.Cm = _ptr(x), _ptr(dt_raw), _ptr(Bm), _ptr(Cm)
    a.Wr, a.idx, a.gate = _ptr(Wr), _ptr(idx), _ptr(gate)
    a.idx_out, a.gate_out = _ptr(idx_out), _ptr(gate_out)
    a.A, a.dt_bias, a.Dskip, a.state, a.y = _ptr(A), _ptr(dt_bias), _ptr(Dskip), _ptr(state), \
        _ptr(y)
    a.a_form = A_SCALAR if scalar_a else A_DIAGONAL
    a.disc = DISC_ZOH if zoh else DISC_EULER
    return a, y


def step(x, dt_raw, Bm, Cm, A, dt_bias, Dskip, state, Wr=None, k=None, idx=None, gate=None,
         y=None, idx_out=None, gate_out=None, y_dtype=None, stream=None, zoh=False):
    """One decode step (include/swimba.h: swimba_step).  x, dt_raw [B,D];
    Bm, Cm [B,16]; state [B,D,16] f32 updated in place.  Routing from Wr [D,E]
    with top-k, or forced idx/gate [B,k].  Returns y [B,D]."""
    a, y = _step_args(x, dt_raw, Bm, Cm, A, dt_bias, Dskip, state, Wr, k, idx, gate, y, idx_out,
                      gate_out, y_dtype, zoh)
    rc = load().swimba_step(ctypes.byref(a), _stream(stream))
    _check("swimba_step", rc)
    return y


class PreparedStep:
    """swimba_step marshalled once for fixed tensors (a decode loop that keeps
    its buffers calls the C ABI directly, without per-call checks)."""

    def __init__(self, x, dt_raw, Bm, Cm, A, dt_bias, Dskip, state, Wr=None, k=None, idx=None,
                 gate=None, y=None, idx_out=None, gate_out=None, y_dtype=None, stream=None,
                 zoh=False):
        self.args, self.y = _step_args(x, dt_raw, Bm, Cm, A, dt_bias, Dskip, state, Wr, k, idx,
                                       gate, y, idx_out, gate_out, y_dtype, zoh)
        self._keep = (x, dt_raw, Bm, Cm, A, dt_bias, Dskip, state, Wr, idx, gate, idx_out,
                      gate_out)
        self._ref = ctypes.byref(self.args)
        self._fn = load().swimba_step
        self.stream = _stream(stream)

    def __call__(self):
        rc = self._fn(self._ref, self.stream)
        if rc != OK:
            raise SwimbaError("swimba_step", rc)
        return self.y
