"""Benchmark of the Swimba hot path on one MI355X.

One step = one pass of the path over one batch of the workload: the router
(logits, top-k, gates) and the parameter-space-mixed scan with its chunk carry,
inputs resident in HBM.  Printed as one JSON line (rank 0):
  value    = tokens x channels per second of the whole step (G tc/s)
  roofline = the dominant kernel (the scan's chunk pass) against the VALU issue
             ceiling that bounds it, with its HBM rate against 8 TB/s beside it
  modes    = the separate design (per expert, per routing slot, and every
             expert advancing at every token), the
             dense single-expert scan (E = 1), the
             scan alone, and the decode step, for the "mixed vs separate" and
             "mixed vs dense" ratios; the stream-mixed form (shared A, mixed
             B X injection and C readout), the scalar-transition (Mamba-2)
             form of the mixed scan and the mixed scan's backward at the same
             shape
  cpu_baseline = the fp64 oracle timed on this host on the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, public peak
# VALU ceiling: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz issue slots per second;
# a slot is one fp32 FMA (2 flops).  The kernels use no packed fp32, so the
# non-packed FMA rate is the ceiling: 78.6 TFLOP/s.
VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2.4e9 * 2 / 1e12
N_STATE = 16


def slots_per_tc(k: int) -> float:
    """Minimum VALU issue slots per token x channel of the mixed scan on this
    ISA (v_exp_f32 and v_log_f32 issue at half rate: 2 slots each).
    Per state entry: k for the mixed exponent, 2 for exp2, 1 for Delta*x*B,
    1 for the state update, 1 for the readout.  Per (token, channel): softplus
    (2 transcendentals = 4 slots, 5 VALU), beta and delta (2k), Delta*g_j (k),
    Delta*x, the D term, and x/dt_raw/y conversions (3)."""
    return N_STATE * (k + 5) + (4 + 5 + 3 * k + 2 + 3)


def scalar_a_slots_per_tc(k: int) -> float:
    """Minimum VALU issue slots per token x channel of the mixed scan with one
    transition per channel (the Mamba-2 form): per state entry Delta*x*B,
    the update and the readout (3); per (token, channel) softplus (4 + 5),
    beta, delta and the mixed exponent (3k), Delta*g_j (k), one exp2 (2),
    Delta*x, the D term and the x/dt_raw/y conversions (5)."""
    return N_STATE * 3 + (9 + 4 * k + 2 + 5)


def stream_slots_per_tc(k: int) -> float:
    """Minimum VALU issue slots per token x channel of the stream-mixed scan
    (shared A).  Per state entry: Delta*A (1), exp2 (2), the k-slot injection
    (k), the update (1), the readout (1).  Per (token, channel): softplus
    (4 + 5), Delta*X_j (k), and the X, dt_raw and y conversions (k + 2)."""
    return N_STATE * (k + 5) + (9 + 2 * k + 2)


# --------------------------------------------------------------- HIP events
class Hip:
    """HIP events through the runtime's C API (timing on a given stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        v = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(v), a, b) == 0
        return float(v.value)


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# everything the chunk-pass kernel and its launch are built from
SCAN_SOURCES = ["parameter_space_moe_amd/csrc/scan_mixed.hpp",
                "parameter_space_moe_amd/csrc/scan_common.hpp",
                "parameter_space_moe_amd/csrc/swimba_device.hpp",
                "parameter_space_moe_amd/csrc/swimba_api.hip",
                "parameter_space_moe_amd/build.py"]


def load_traffic(workload):
    """HBM bytes per chunk-pass launch measured by rocprofv3 counters, if the
    committed measurement was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "scan_chunk_%s_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest(SCAN_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, inp):
    """The fp64 oracle on this host: router + mixed scan over the same workload."""
    import numpy as np

    import oracle
    T = w.B * w.L
    x = inp["x"].astype(np.float64)
    reps = []
    t_end = time.perf_counter() + 10.0
    while True:
        t0 = time.perf_counter()
        idx, gate, _, _ = oracle.route(x.reshape(T, w.D), inp["Wr"], w.k)
        oracle.scan(x, inp["dt_raw"], inp["Bm"], inp["Cm"], idx.reshape(w.B, w.L, w.k),
                    gate.reshape(w.B, w.L, w.k), inp["A"], inp["dt_bias"], inp["Dskip"])
        reps.append(time.perf_counter() - t0)
        # about 10 s of CPU work (at least 5 runs), so that the median is stable
        if (time.perf_counter() > t_end and len(reps) >= 5) or len(reps) >= 500:
            break
    best = sorted(reps)[len(reps) // 2]
    return {"value": round(w.tc / best / 1e9, 5), "unit": "G token*channel/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "whole workload (router + mixed scan, %d x %d x %d), median of %d runs"
                      % (w.B, w.L, w.D, len(reps))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mamba130m_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-modes", action="store_true",
                    help="time only the step (for profiler runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from parameter_space_moe_amd import swimba, workloads

    w = workloads.BY_NAME[args.workload]
    assert w.steps == 0, "decode workload is reported under modes"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = workloads.generate(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to(name, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(inp[name]))
        return t.to(dtype).to(dev) if dtype is not None else t.to(dev)

    x, dtr, Bm, Cm = to("x", dt), to("dt_raw", dt), to("Bm", dt), to("Cm", dt)
    Wr, A, bias, Dsk = to("Wr"), to("A"), to("dt_bias"), to("Dskip")
    B, L, D, E, k = w.B, w.L, w.D, w.E, w.k
    idx = torch.empty((B, L, k), dtype=torch.int32, device=dev)
    gate = torch.empty((B, L, k), dtype=torch.float32, device=dev)
    y = torch.empty((B, L, D), dtype=dt, device=dev)
    hf = torch.empty((B, D, N_STATE), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()
    K, W = args.steps, args.warmup
    # marshalled once; the timed loop goes straight to the C ABI
    route_call = swimba.PreparedRoute(x, Wr, k, idx, gate)
    scan_call = swimba.PreparedScan(False, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y=y,
                                    h_final=hf, chunk=w.chunk)
    chunk_len, plan_chunks = swimba.scan_plan(x, A, idx, chunk=w.chunk)

    # ------------------------------------------------------- the timed step
    def step():
        route_call()
        scan_call()

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K

    # ------------------------------------------- per-kernel durations
    # A second run of K steps in which the scan's passes are timed by events
    # that the kernels' own dispatches stamp (start and end of each pass).  The
    # runtime adds a few microseconds of stream work per stamped event, so these
    # steps are kept out of the timed region above.
    ev = [[hip.event() for _ in range(6)] for _ in range(K)]
    ev_arrays = [(ctypes.c_void_p * 6)(*[x_.value for x_ in e]) for e in ev]
    t1 = time.perf_counter()
    for i in range(K):
        route_call()
        scan_call(ctypes.addressof(ev_arrays[i]))
    torch.cuda.synchronize()
    ms_per_step_evented = (time.perf_counter() - t1) * 1e3 / K
    chunk_ms = sum(hip.ms(e[0], e[1]) for e in ev) / K
    carry_ms = sum(hip.ms(e[2], e[3]) for e in ev) / K
    fixup_ms = sum(hip.ms(e[4], e[5]) for e in ev) / K
    # the router on its own, back to back, after the timed region
    r0, r1 = hip.event(), hip.event()
    hip.record(r0, stream)
    for _ in range(K):
        route_call()
    hip.record(r1, stream)
    torch.cuda.synchronize()
    route_ms = hip.ms(r0, r1) / K
    scan_ms = chunk_ms + carry_ms + fixup_ms
    tc = w.tc
    value = tc / (ms_per_step * 1e-3) / 1e9

    # dominant kernel: the chunk pass.  Algorithmic bytes per launch: x, dt_raw
    # read and y written once (2 B each in bf16), B_t, C_t, idx, gate per token,
    # and the chunk records (decay and end state, fp32 x 16 per chunk/channel).
    esz = 2 if w.dtype == "bf16" else 4
    chunk_bytes = tc * 3 * esz + B * L * (2 * N_STATE * esz + 2 * k * 4)
    if plan_chunks > 1:
        chunk_bytes += 2 * B * plan_chunks * N_STATE * D * 4
    achieved_gbs = chunk_bytes / (chunk_ms * 1e-3) / 1e9
    flops = tc * slots_per_tc(k) * 2
    achieved_tf = flops / (chunk_ms * 1e-3) / 1e12
    traffic = load_traffic(w.name)

    out = {
        "metric": "scan throughput (G token*channel/s) + % of HBM roofline, mixed vs separate",
        "value": round(value, 3), "unit": "G token*channel/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": B, "L": L, "D": D, "N": N_STATE, "E": E, "k": k,
                   "chunk": chunk_len, "chunks": plan_chunks, "parallelism": "single-gpu"},
        "roofline": {"bound": "alu", "kernel": "mix_chunk_kernel",
                     "achieved": round(achieved_tf, 3), "peak": round(VALU_PEAK_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(achieved_tf / VALU_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "note": "VALU issue slots as FMA-equivalent flops, %d slots/tc"
                             % slots_per_tc(k)},
        "roofline_hbm": {"bound": "hbm", "kernel": "mix_chunk_kernel",
                         "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                         "step_frac": round(tc * 3 * esz / (ms_per_step * 1e-3) / 1e9
                                            / HBM_PEAK_GBS, 4)},
        "kernels_ms": {"route": round(route_ms, 4), "chunk_pass": round(chunk_ms, 4),
                       "carry": round(carry_ms, 4), "fixup": round(fixup_ms, 4),
                       "ms_per_step_with_events": round(ms_per_step_evented, 4)},
    }

    if not args.no_modes:
        out["modes"] = modes(args, w, swimba, workloads, x, dtr, Bm, Cm, Wr, A, bias, Dsk, idx,
                             gate, y, hf)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


def _time(fn, reps, warm=2):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / reps


def expert_sweep(swimba, dev, reps):
    """Router + mixed scan at the Mamba-1.4B-like layer shape (B=8, L=4096,
    D=4096, top-2) for E = 2, 4, 8, 16 experts: the active experts, not the
    total, set the cost ("Fondements Théoriques", Theorem 2).  Inputs are
    seeded normal draws made on the GPU; E = 32 is beyond the scans' 16."""
    import torch
    B, L, D, k = 8, 4096, 4096, 2
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    bf = torch.bfloat16
    x = torch.randn((B, L, D), generator=g, device=dev).to(bf)
    dtr = torch.randn((B, L, D), generator=g, device=dev).to(bf)
    Bm = torch.randn((B, L, N_STATE), generator=g, device=dev).to(bf)
    Cm = torch.randn((B, L, N_STATE), generator=g, device=dev).to(bf)
    y = torch.empty((B, L, D), dtype=bf, device=dev)
    hf = torch.empty((B, D, N_STATE), dtype=torch.float32, device=dev)
    idx = torch.empty((B, L, k), dtype=torch.int32, device=dev)
    gate = torch.empty((B, L, k), dtype=torch.float32, device=dev)
    out = {"shape": "B=%d L=%d D=%d k=%d bf16" % (B, L, D, k)}
    base = None
    for E in (2, 4, 8, 16):
        Wr = torch.randn((D, E), generator=g, device=dev) / D ** 0.5
        A = -torch.exp(torch.rand((E, D, N_STATE), generator=g, device=dev) * math.log(16.0))
        bias = torch.randn((E, D), generator=g, device=dev) * 0.1 ** 0.5
        Dsk = torch.randn((E, D), generator=g, device=dev)
        route = swimba.PreparedRoute(x, Wr, k, idx, gate)
        scan = swimba.PreparedScan(False, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y=y,
                                   h_final=hf)

        def step():
            route()
            scan()

        ms = _time(step, reps)
        base = base or ms
        out["E%d" % E] = {"ms": round(ms, 4), "G_tc_per_s": round(B * L * D / ms / 1e6, 3),
                          "over_E2": round(ms / base, 3)}
    return out


def theorem4_mode(swimba, workloads, w, x, dtr, Bm, Cm, A, bias, Dsk):
    """Theorem 4 ("Fondements Théoriques"): relative difference between the
    mixed and separate designs' outputs under top-1 routing that switches
    expert with probability p per token (p = 0: constant routing, where they
    coincide)."""
    import torch
    dev = x.device
    out = {"shape": "B=%d L=%d D=%d E=%d top-1" % (w.B, w.L, w.D, w.E)}
    for p in (0.0, 0.01, 0.1, 0.5, 1.0):
        i, g = workloads.switching_routing(w.B, w.L, w.E, p, seed=7)
        idx = torch.from_numpy(i).to(dev)
        gate = torch.from_numpy(g).to(dev)
        a = (x, dtr, Bm, Cm, idx, gate, A, bias, Dsk)
        ym, _ = swimba.scan(*a, y_dtype=torch.float32, want_state=False)
        ys, _ = swimba.scan_separate(*a, y_dtype=torch.float32, want_state=False)
        d = torch.linalg.vector_norm(ym - ys) / torch.linalg.vector_norm(ys)
        out["p%g" % p] = round(float(d), 5)
    return out


def backward_mode(swimba, w, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, reps, ms_mixed):
    """Gradients of the mixed scan for a seeded dL/dy at the same shape (the
    whole backward call: forward recompute with the chunk records, the two
    carries, the gradient pass and the reductions), against the forward scan."""
    import torch
    dev = x.device
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    dy = torch.randn(x.shape, generator=g, device=dev).to(x.dtype)
    B, L, D, E, k = w.B, w.L, w.D, w.E, w.k
    f32 = torch.float32
    out = {"dx": torch.empty((B, L, D), dtype=f32, device=dev),
           "ddt_raw": torch.empty((B, L, D), dtype=f32, device=dev),
           "dBm": torch.empty((B, L, N_STATE), dtype=f32, device=dev),
           "dCm": torch.empty((B, L, N_STATE), dtype=f32, device=dev),
           "dgate": torch.empty((B, L, k), dtype=f32, device=dev),
           "dA": torch.empty_like(A), "ddt_bias": torch.empty_like(bias),
           "dDskip": torch.empty_like(Dsk),
           "dh0": torch.empty((B, D, N_STATE), dtype=f32, device=dev)}
    call = swimba.PreparedBackward(x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, dy, out)
    ms = _time(call, reps)
    return {"ms": round(ms, 4), "G_tc_per_s": round(w.tc / ms / 1e6, 3),
            "over_forward_scan": round(ms / ms_mixed, 3),
            "workspace_MB": round(call.workspace.numel() / 1e6, 1),
            "note": "fp32 gradients of x, dt_raw, B, C, gates, A, dt_bias, Dskip, h0"}


def scalar_a_mode(swimba, w, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y, hf, reps, ms_mixed):
    """The mixed scan with one transition per (expert, channel), the Mamba-2
    form A_t = a_t I, on the same inputs (A[e, d] = the n = 0 entry of the
    diagonal draw): one exponential per (token, channel) instead of 16.  The
    scan alone, and its chunk pass against the VALU ceiling and 8 TB/s."""
    import torch
    As = A[:, :, 0].contiguous()
    scan = swimba.PreparedScan(False, x, dtr, Bm, Cm, idx, gate, As, bias, Dsk, y=y,
                               h_final=hf, chunk=w.chunk)
    ms = _time(scan, reps)
    hip = Hip()
    ev = [[hip.event() for _ in range(6)] for _ in range(reps)]
    arrs = [(ctypes.c_void_p * 6)(*[e_.value for e_ in e]) for e in ev]
    for a in arrs:
        scan(ctypes.addressof(a))
    torch.cuda.synchronize()
    chunk_ms = sum(hip.ms(e[0], e[1]) for e in ev) / reps
    fixup_ms = sum(hip.ms(e[4], e[5]) for e in ev) / reps
    tc, k = w.tc, w.k
    esz = 2 if w.dtype == "bf16" else 4
    _, nchunks = swimba.scan_plan(x, As, idx, chunk=w.chunk)
    chunk_bytes = tc * 3 * esz + w.B * w.L * (2 * N_STATE * esz + 2 * k * 4)
    if nchunks > 1:
        chunk_bytes += 2 * w.B * nchunks * N_STATE * w.D * 4
    tf = tc * scalar_a_slots_per_tc(k) * 2 / (chunk_ms * 1e-3) / 1e12
    gbs = chunk_bytes / (chunk_ms * 1e-3) / 1e9
    return {"scan_ms": round(ms, 4), "G_tc_per_s": round(tc / ms / 1e6, 3),
            "over_diagonal": round(ms / ms_mixed, 3),
            "chunk_pass_ms": round(chunk_ms, 4), "fixup_ms": round(fixup_ms, 4),
            "valu_frac": round(tf / VALU_PEAK_TFLOPS, 4),
            "valu_note": "%d slots/tc as FMA-equivalent flops" % scalar_a_slots_per_tc(k),
            "hbm_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def stream_mode(swimba, workloads, w, x, Wr, idx, gate, reps):
    """The pages' stream-mixed form at the same layer shape: shared A, each of
    the k slots carries its expert's X, B and C streams, the injection and the
    readout are mixed by the gates ("Kernmechanisme van Swimba").  Times the
    router on the layer's x plus the stream scan, and the scan's chunk pass
    alone (dispatch-stamped events) against the VALU ceiling and 8 TB/s."""
    import numpy as np
    import torch
    dev = x.device
    inp = workloads.generate_streams(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T = {}
    for name, v in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        T[name] = (t.to(dt) if name in ("X", "dt_raw", "Bs", "Cs") else t).to(dev)
    y = torch.empty((w.B, w.L, w.D), dtype=dt, device=dev)
    hf = torch.empty((w.B, w.D, N_STATE), dtype=torch.float32, device=dev)
    scan = swimba.PreparedStreams(T["X"], T["dt_raw"], T["Bs"], T["Cs"], T["gate"], T["A"],
                                  T["dt_bias"], y=y, h_final=hf)
    route = swimba.PreparedRoute(x, Wr, w.k, idx, gate)
    chunk_len, nchunks = swimba.scan_streams_plan(T["X"])
    ms_scan = _time(scan, reps)

    def step():
        route()
        scan()

    ms_step = _time(step, reps)
    hip = Hip()
    ev = [[hip.event() for _ in range(6)] for _ in range(reps)]
    arrs = [(ctypes.c_void_p * 6)(*[e_.value for e_ in e]) for e in ev]
    for a in arrs:
        scan(ctypes.addressof(a))
    torch.cuda.synchronize()
    chunk_ms = sum(hip.ms(e[0], e[1]) for e in ev) / reps
    carry_ms = sum(hip.ms(e[2], e[3]) for e in ev) / reps
    fixup_ms = sum(hip.ms(e[4], e[5]) for e in ev) / reps
    tc, k = w.tc, w.k
    esz = 2 if w.dtype == "bf16" else 4
    # X (k slots) and dt_raw read, y written; per token the k B and C streams
    # and gates; per chunk and channel the decay and end state
    chunk_bytes = tc * (k + 2) * esz + w.B * w.L * k * (2 * N_STATE * esz + 4)
    if nchunks > 1:
        chunk_bytes += 2 * w.B * nchunks * N_STATE * w.D * 4
    tf = tc * stream_slots_per_tc(k) * 2 / (chunk_ms * 1e-3) / 1e12
    gbs = chunk_bytes / (chunk_ms * 1e-3) / 1e9
    return {"shape": "B=%d L=%d D=%d k=%d %s, chunk %d x %d" % (w.B, w.L, w.D, k, w.dtype,
                                                              chunk_len, nchunks),
            "scan_ms": round(ms_scan, 4), "G_tc_per_s": round(tc / ms_scan / 1e6, 3),
            "route_plus_scan_ms": round(ms_step, 4),
            "chunk_pass_ms": round(chunk_ms, 4), "carry_ms": round(carry_ms, 4),
            "fixup_ms": round(fixup_ms, 4),
            "valu_frac": round(tf / VALU_PEAK_TFLOPS, 4),
            "valu_note": "%d slots/tc as FMA-equivalent flops" % stream_slots_per_tc(k),
            "hbm_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def modes(args, w, swimba, workloads, x, dtr, Bm, Cm, Wr, A, bias, Dsk, idx, gate, y, hf):
    import numpy as np
    import torch
    dev = x.device
    reps = max(5, args.steps // 2)
    tc = w.tc
    res = {}
    # mixed scan alone (routing precomputed)
    mixed = swimba.PreparedScan(False, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y=y, h_final=hf,
                                chunk=w.chunk)
    ms_mixed = _time(mixed, reps)
    res["mixed_scan"] = {"ms": round(ms_mixed, 4), "G_tc_per_s": round(tc / ms_mixed / 1e6, 3)}
    # separate design: route + per-expert scans
    hfs = torch.empty((w.B, w.E, w.D, N_STATE), dtype=torch.float32, device=dev)
    sep = swimba.PreparedScan(True, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y=y, h_final=hfs,
                              chunk=w.chunk)
    ms_sep = _time(sep, reps)
    res["separate_scan"] = {"ms": round(ms_sep, 4), "G_tc_per_s": round(tc / ms_sep / 1e6, 3),
                            "separate_over_mixed": round(ms_sep / ms_mixed, 3)}
    del hfs, sep
    # separate trajectories per routing slot: k states per (b, d), each slot
    # advancing at every token with its own expert (library's chunking)
    hfk = torch.empty((w.B, w.k, w.D, N_STATE), dtype=torch.float32, device=dev)
    slots = swimba.PreparedScan(swimba.DESIGN_SLOTS, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk,
                                y=y, h_final=hfk)
    ms_slots = _time(slots, reps)
    res["slots_scan"] = {"ms": round(ms_slots, 4), "G_tc_per_s": round(tc / ms_slots / 1e6, 3),
                         "slots_over_mixed": round(ms_slots / ms_mixed, 3)}
    del hfk, slots
    # separate trajectories where every expert advances at every token (E
    # updates per token; the routing only picks the outputs)
    hfa = torch.empty((w.B, w.E, w.D, N_STATE), dtype=torch.float32, device=dev)
    alle = swimba.PreparedScan(swimba.DESIGN_ALL_EXPERTS, x, dtr, Bm, Cm, idx, gate, A, bias,
                               Dsk, y=y, h_final=hfa)
    ms_all = _time(alle, reps)
    res["all_experts_scan"] = {"ms": round(ms_all, 4), "G_tc_per_s": round(tc / ms_all / 1e6, 3),
                               "all_experts_over_mixed": round(ms_all / ms_mixed, 3)}
    del hfa, alle
    # dense single-expert scan (E = 1): the plain Mamba scan on the same shapes
    idx1 = torch.zeros((w.B, w.L, 1), dtype=torch.int32, device=dev)
    gate1 = torch.ones((w.B, w.L, 1), dtype=torch.float32, device=dev)
    A1, b1, D1 = A[:1].contiguous(), bias[:1].contiguous(), Dsk[:1].contiguous()
    dense = swimba.PreparedScan(False, x, dtr, Bm, Cm, idx1, gate1, A1, b1, D1, y=y, h_final=hf,
                                chunk=w.chunk)
    ms_dense = _time(dense, reps)
    res["dense_scan"] = {"ms": round(ms_dense, 4), "G_tc_per_s": round(tc / ms_dense / 1e6, 3),
                         "mixed_over_dense": round(ms_mixed / ms_dense, 3)}
    # the timed step again, one step at a time, each after writing 512 MB so
    # that the 256 MB Infinity Cache holds none of its inputs (this workload's
    # inputs fit in it, so back-to-back steps read them from the cache)
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    route = swimba.PreparedRoute(x, Wr, w.k, idx, gate)
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    evs = [(hip.event(), hip.event()) for _ in range(reps)]
    for e0, e1 in evs:
        flush.fill_(1.0)
        hip.record(e0, stream)
        route()
        mixed()
        hip.record(e1, stream)
    torch.cuda.synchronize()
    ms_cold = sum(hip.ms(e0, e1) for e0, e1 in evs) / reps
    res["step_mall_flushed"] = {"ms": round(ms_cold, 4), "G_tc_per_s": round(tc / ms_cold / 1e6, 3),
                                "note": "route + mixed scan after a 512 MB write, HIP events"}
    del flush
    res["expert_sweep"] = expert_sweep(swimba, dev, reps)
    res["stream_mixed"] = stream_mode(swimba, workloads, w, x, Wr, idx, gate, reps)
    zoh = swimba.PreparedScan(False, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y=y, h_final=hf,
                              chunk=w.chunk, zoh=True)
    ms_zoh = _time(zoh, reps)
    res["zoh_scan"] = {"ms": round(ms_zoh, 4), "G_tc_per_s": round(tc / ms_zoh / 1e6, 3),
                       "over_euler": round(ms_zoh / ms_mixed, 3),
                       "note": "zero-order-hold input term, B_bar = A^-1 (exp(Delta A) - I) B"}
    res["theorem4"] = theorem4_mode(swimba, workloads, w, x, dtr, Bm, Cm, A, bias, Dsk)
    res["backward"] = backward_mode(swimba, w, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, reps,
                                    ms_mixed)
    res["scalar_a"] = scalar_a_mode(swimba, w, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y, hf,
                                    reps, ms_mixed)
    # decode workload: 128 routed steps on a persistent fp32 state
    wd = workloads.BY_NAME["decode"]
    p, steps = workloads.decode_steps(wd)
    dd = torch.bfloat16 if wd.dtype == "bf16" else torch.float32
    P = {kk: torch.from_numpy(v).to(dev) for kk, v in p.items()}
    S = [{kk: torch.from_numpy(np.ascontiguousarray(v)).to(dd).to(dev) for kk, v in s.items()}
         for s in steps]
    state = torch.zeros((wd.B, wd.D, N_STATE), dtype=torch.float32, device=dev)
    yd = torch.empty((wd.B, wd.D), dtype=dd, device=dev)

    # marshalled once per step's inputs; the loop calls the C ABI directly
    calls = [swimba.PreparedStep(s["x"], s["dt_raw"], s["Bm"], s["Cm"], P["A"], P["dt_bias"],
                                 P["Dskip"], state, Wr=P["Wr"], k=wd.k, y=yd) for s in S]

    def run_decode():
        for c in calls:
            c()

    ms_dec = _time(run_decode, 2, warm=1)
    # the same 128 steps captured once in a HIP graph and replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gcalls = [swimba.PreparedStep(s["x"], s["dt_raw"], s["Bm"], s["Cm"], P["A"],
                                      P["dt_bias"], P["Dskip"], state, Wr=P["Wr"], k=wd.k, y=yd,
                                      stream=side) for s in S]
        for c in gcalls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for c in gcalls:
            c()
    ms_graph = _time(graph.replay, 3, warm=1)
    esz = 2 if wd.dtype == "bf16" else 4
    per_step_bytes = wd.B * wd.D * (2 * N_STATE * 4 + 3 * esz)
    gbs = per_step_bytes * len(S) / (ms_dec * 1e-3) / 1e9
    res["decode"] = {"workload": wd.name, "steps": len(S), "ms": round(ms_dec, 4),
                     "us_per_step": round(ms_dec * 1e3 / len(S), 2),
                     "G_channel_steps_per_s": round(wd.B * wd.D * len(S) / ms_dec / 1e6, 3),
                     "hbm_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "graph_us_per_step": round(ms_graph * 1e3 / len(S), 2),
                     "note": "state (84 MB) fits the 256 MB Infinity Cache in steady state; "
                             "graph = the 128 steps captured once and replayed"}
    return res


if __name__ == "__main__":
    main()
