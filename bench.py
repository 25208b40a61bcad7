"""Benchmark of the Swimba hot path on one MI355X.

One step = one pass of the path over one batch of the workload: the router
(logits, top-k, gates) and the parameter-space-mixed scan with its chunk
carry, inputs resident in HBM.  The default workload is the long-context one
(B = 1, L = 65536, D = 2560, E = 16, top-2, bf16, chunk 256): the largest
single-GPU shape, whose 1 GB of streams does not fit the 256 MB Infinity
Cache.  Printed as one JSON line:
  value        = tokens x channels per second of the step (G tc/s), from the
                 median of K steps each timed with HIP events on the stream
                 the kernels run on, after 0.1 s of untimed steps (the GPU
                 clock settles after ~30 ms of load) and W warm-up steps
  roofline     = the dominant kernel (the scan's chunk pass) against 8 TB/s,
                 with 6 algorithmic bytes per token x channel (bf16 x and
                 dt_raw read, y written); `valu` beside it gives the same
                 kernel against the VALU issue ceiling that bounds it
  modes        = the scan alone, the dense single-expert scan (E = 1), the
                 separate design ("mixed vs separate") and the scalar-transition
                 (Mamba-2) form at the same shape; the same and the step on the
                 Mamba-1.4B-like layer; an
                 expert-count sweep; the Mamba-130M-like layer (steady and
                 cache-flushed) with the stream-mixed, scalar-transition,
                 zero-order-hold, per-slot and all-experts forms, the
                 backward and the Theorem 4 study; the decode step (steady
                 and cache-flushed, eager and graph-captured)
  cpu_baseline = the fp64 oracle on this host's cores, on the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, public peak
# VALU ceiling: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz issue slots per second;
# a slot is one fp32 FMA (2 flops).  The kernels use no packed fp32, so the
# non-packed FMA rate is the ceiling: 78.6 TFLOP/s.
VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2.4e9 * 2 / 1e12
# Clock the scan kernels ran at, fitted from GRBM_GUI_ACTIVE against traced
# dispatch durations (profiles/clock_mamba130m_layer.md).
MEASURED_CLOCK_GHZ = 2.17
N_STATE = 16
FLUSH_BYTES = 512 * 2**20       # twice the 256 MB Infinity Cache


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


def algorithmic_bytes_per_tc(dtype: str) -> int:
    """x and dt_raw read and y written once: 6 B per token x channel in bf16,
    12 in fp32 (B_t and C_t add 4N/D bytes, under 0.03 B at these widths)."""
    return 3 * (2 if dtype == "bf16" else 4)


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


HIP = None


def hip():
    global HIP
    if HIP is None:
        HIP = Hip()
    return HIP


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


# ------------------------------------------------------------- timing helpers
def stream_of_torch():
    import torch
    return torch.cuda.current_stream().cuda_stream


def time_events(fn, reps, warm=2, flush=None):
    """Median over `reps` calls of fn, each bracketed by HIP events on the
    current stream; `flush()` (untimed) runs before each call."""
    import torch
    h = hip()
    st = stream_of_torch()
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = [(h.event(), h.event()) for _ in range(reps)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        h.record(e0, st)
        fn()
        h.record(e1, st)
    torch.cuda.synchronize()
    return statistics.median(h.ms(e0, e1) for e0, e1 in evs)


PREWARM_S = 0.1


def prewarm(lay, seconds=PREWARM_S):
    """Untimed steps in batches of 10 until `seconds` of wall time have
    passed with the GPU busy; returns how many ran."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            lay.step()
        torch.cuda.synchronize()
        n += 10
    return n


class Flusher:
    """Writes 512 MB (twice the Infinity Cache) so that a following call
    finds none of its inputs cached."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.fill_(1.0)


# ----------------------------------------------------------------- workloads
class Layer:
    """Device copies of a workload's inputs and prepared router/scan calls."""

    def __init__(self, w, dev):
        import numpy as np
        import torch

        from parameter_space_moe_amd import swimba, workloads
        self.w = w
        self.inp = workloads.generate(w)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.dt = dt

        def to(name, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(self.inp[name]))
            return t.to(dtype).to(dev) if dtype is not None else t.to(dev)

        self.x, self.dtr, self.Bm, self.Cm = (to("x", dt), to("dt_raw", dt), to("Bm", dt),
                                              to("Cm", dt))
        self.Wr, self.A, self.bias, self.Dsk = to("Wr"), to("A"), to("dt_bias"), to("Dskip")
        B, L, D, k = w.B, w.L, w.D, w.k
        self.idx = torch.empty((B, L, k), dtype=torch.int32, device=dev)
        self.gate = torch.empty((B, L, k), dtype=torch.float32, device=dev)
        self.y = torch.empty((B, L, D), dtype=dt, device=dev)
        self.hf = torch.empty((B, D, N_STATE), dtype=torch.float32, device=dev)
        self.route = swimba.PreparedRoute(self.x, self.Wr, k, self.idx, self.gate)
        self.scan = swimba.PreparedScan(False, self.x, self.dtr, self.Bm, self.Cm, self.idx,
                                        self.gate, self.A, self.bias, self.Dsk, y=self.y,
                                        h_final=self.hf, chunk=w.chunk)
        self.chunk, self.nchunks = swimba.scan_plan(self.x, self.A, self.idx, chunk=w.chunk)
        self.route()

    def step(self):
        self.route()
        self.scan()

    def timed_steps(self, K, W, phases=True):
        """K steps, each bracketed by HIP events; with `phases` the scan's
        passes are also stamped by their own dispatches (hipExtLaunchKernelGGL
        events, which add a little stream work inside the step). Returns
        per-step (and per-pass) durations (ms) and the wall time."""
        import torch
        h = hip()
        st = stream_of_torch()
        for _ in range(W):
            self.step()
        torch.cuda.synchronize()
        s0 = [h.event() for _ in range(K)]
        s1 = [h.event() for _ in range(K)]
        ph = [[h.event() for _ in range(6)] for _ in range(K)]
        arrs = [(ctypes.c_void_p * 6)(*[e.value for e in p]) for p in ph]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            h.record(s0[i], st)
            self.route()
            self.scan(ctypes.addressof(arrs[i]) if phases else None)
            h.record(s1[i], st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step = [h.ms(s0[i], s1[i]) for i in range(K)]
        if not phases:
            return dict(step=step, wall=wall)
        route = [h.ms(s0[i], ph[i][0]) for i in range(K)]
        chunk = [h.ms(ph[i][0], ph[i][1]) for i in range(K)]
        carry = [h.ms(ph[i][2], ph[i][3]) for i in range(K)]
        fix = [h.ms(ph[i][4], ph[i][5]) for i in range(K)]
        return dict(step=step, route=route, chunk=chunk, carry=carry, fixup=fix, wall=wall)


def chunk_roofline(w, chunk_ms, traffic=None):
    """The chunk pass against 8 TB/s with 6 (bf16) or 12 (fp32) algorithmic
    bytes per token x channel."""
    bpt = algorithmic_bytes_per_tc(w.dtype)
    achieved = w.tc * bpt / (chunk_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": "mix_chunk_kernel", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_tc": bpt, "units_per_launch": w.tc,
            "note": "achieved = %d B/tc x %d tc per launch / mean chunk-pass duration "
                    "(dispatch-stamped HIP events in the timed steps)" % (bpt, w.tc)}


def chunk_valu(w, chunk_ms):
    slots = slots_per_tc(w.k)
    tf = w.tc * slots * 2 / (chunk_ms * 1e-3) / 1e12
    at_clock = VALU_PEAK_TFLOPS * MEASURED_CLOCK_GHZ / 2.4
    return {"bound": "alu", "kernel": "mix_chunk_kernel", "achieved": round(tf, 2),
            "peak": round(VALU_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
            "frac": round(tf / VALU_PEAK_TFLOPS, 4),
            "frac_at_measured_clock": round(tf / at_clock, 4),
            "measured_clock_GHz": MEASURED_CLOCK_GHZ, "slots_per_tc": slots,
            "note": "VALU issue slots (an FMA slot = 2 flops, a transcendental 2 slots) at "
                    "256 CUs x 64 lanes x 2.4 GHz, packed fp32 not used"}


# --------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the clock settles after about 30 ms of sustained load (the chunk pass of
    # the long-context step runs ~15% slower over its first ~30 dispatches)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="long_context")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--designs-only", action="store_true",
                    help="time only the mixed, separate, dense and scalar-transition "
                         "scans at the workload's shape (for profiler runs of their "
                         "kernels)")
    ap.add_argument("--no-modes", action="store_true",
                    help="time only the step (for profiler runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from parameter_space_moe_amd import swimba, workloads

    w = workloads.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.steps:
        # the decode workload alone (it is also reported under the default
        # run's modes): for profiler runs of the step kernel
        print(json.dumps({"decode": decode_mode(swimba, workloads, dev, Flusher(dev))}), flush=True)
        return
    print("bench: %s, generating inputs" % w.name, file=sys.stderr, flush=True)
    lay = Layer(w, dev)
    if args.designs_only:
        # the three designs alone on the router's routing (they are also
        # reported under the default run's modes)
        lay.route()
        res, ms_mixed = ratios_at(lay, swimba, dev, args.steps)
        res["scalar_a"] = scalar_a_mode(swimba, w, lay, args.steps, ms_mixed)
        print(json.dumps({"designs": res}), flush=True)
        return
    K, W = args.steps, args.warmup
    # The GPU clock settles only after ~30 ms of sustained load: untimed steps
    # for PREWARM_S first (reported), then the W warm-up steps, then K timed.
    n_pre = prewarm(lay)
    print("bench: timing %d steps" % K, file=sys.stderr, flush=True)
    r = lay.timed_steps(K, W, phases=False)
    ms_step = statistics.median(r["step"])
    # the passes' durations from a second run whose dispatches stamp events
    rp = lay.timed_steps(K, 1)
    chunk_ms = statistics.mean(rp["chunk"])
    value = w.tc / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "scan throughput (G token*channel/s) + % of HBM roofline, mixed vs separate",
        "value": round(value, 3), "unit": "G token*channel/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "D": w.D, "N": N_STATE, "E": w.E,
                   "k": w.k, "chunk": lay.chunk, "chunks": lay.nchunks,
                   "parallelism": "single-gpu"},
        "roofline": chunk_roofline(w, chunk_ms, load_traffic(w.name)),
        "valu": chunk_valu(w, chunk_ms),
        "step_hbm_frac": round(w.tc * algorithmic_bytes_per_tc(w.dtype) / (ms_step * 1e-3)
                               / 1e9 / HBM_PEAK_GBS, 4),
        "timing": {"ms_per_step_median": round(ms_step, 4),
                   "ms_per_step_min": round(min(r["step"]), 4),
                   "ms_per_step_max": round(max(r["step"]), 4),
                   "ms_per_step_wall_mean": round(r["wall"] * 1e3 / K, 4),
                   "prewarm_steps": n_pre,
                   "prewarm_note": "untimed steps for %.1f s before the W warm-up steps "
                                   "(the clock settles after ~30 ms of load)" % PREWARM_S,
                   "method": "HIP events on the library stream around each of K steps; "
                             "median"},
        "kernels_ms": {"route": round(statistics.mean(rp["route"]), 4),
                       "chunk_pass": round(chunk_ms, 4),
                       "carry": round(statistics.mean(rp["carry"]), 4),
                       "fixup": round(statistics.mean(rp["fixup"]), 4),
                       "note": "from a second run of K steps whose scan passes stamp "
                               "dispatch events; the timed run has only the step events"},
    }
    if not args.no_modes:
        out["modes"] = modes(args, lay, swimba, workloads, dev)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, lay.inp)
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------- cpu baseline
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp):
    """The fp64 oracle on this host: router + mixed scan.  At the OpenMP
    thread count the environment gives (all of this host's CPU share) over
    the whole workload, and on one thread over the first L/16 tokens of
    every sequence; each repeated for about 10 s, median."""
    import numpy as np

    import oracle

    def run(L, reps_s):
        x = np.ascontiguousarray(inp["x"][:, :L], dtype=np.float64)
        dtr = np.ascontiguousarray(inp["dt_raw"][:, :L])
        Bm = np.ascontiguousarray(inp["Bm"][:, :L])
        Cm = np.ascontiguousarray(inp["Cm"][:, :L])
        times = []
        t_end = time.perf_counter() + reps_s
        while True:
            t0 = time.perf_counter()
            idx, gate, _, _ = oracle.route(x.reshape(w.B * L, w.D), inp["Wr"], w.k)
            oracle.scan(x, dtr, Bm, Cm, idx.reshape(w.B, L, w.k), gate.reshape(w.B, L, w.k),
                        inp["A"], inp["dt_bias"], inp["Dskip"])
            times.append(time.perf_counter() - t0)
            if (time.perf_counter() > t_end and len(times) >= 3) or len(times) >= 200:
                break
        return w.B * L * w.D / statistics.median(times) / 1e9, len(times)

    threads = oracle.num_threads()
    v_all, n_all = run(w.L, 10.0)
    # one thread: the OpenMP runtime the oracle runs on, set from here
    gomp = ctypes.CDLL("libgomp.so.1")
    L1 = max(1, w.L // 16)
    gomp.omp_set_num_threads(1)
    try:
        v_one, n_one = run(L1, 10.0)
    finally:
        gomp.omp_set_num_threads(threads)
    return {"value": round(v_all, 5), "unit": "G token*channel/s", "cores": threads,
            "kind": "oracle",
            "sample": "whole workload (router + mixed scan, %d x %d x %d), median of %d runs"
                      % (w.B, w.L, w.D, n_all),
            "one_thread": {"value": round(v_one, 5), "cores": 1,
                           "sample": "first %d tokens of each sequence, median of %d runs"
                                     % (L1, n_one)},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "note": "threads = OMP_NUM_THREADS of the environment (the host's CPU share)"}


# -------------------------------------------------------------------- modes
def ratios_at(lay, swimba, dev, reps, flush=None):
    """The mixed scan alone, the dense single-expert scan (E = 1: the plain
    Mamba scan on the same streams) and the separate design (one state per
    expert), each with the routing precomputed."""
    import torch
    w = lay.w
    res = {}
    ms_mixed = time_events(lay.scan, reps, flush=flush)
    res["mixed_scan"] = {"ms": round(ms_mixed, 4), "G_tc_per_s": round(w.tc / ms_mixed / 1e6, 3)}
    hfs = torch.empty((w.B, w.E, w.D, N_STATE), dtype=torch.float32, device=dev)
    # the separate design at its own chunking (chunks are an implementation
    # detail of each design: its fix-up stops after a number of selections
    # per expert, so it takes a few long chunks)
    sep = swimba.PreparedScan(True, lay.x, lay.dtr, lay.Bm, lay.Cm, lay.idx, lay.gate, lay.A,
                              lay.bias, lay.Dsk, y=lay.y, h_final=hfs, chunk=0)
    ms_sep = time_events(sep, reps, flush=flush)
    sc, sn = swimba.scan_plan(lay.x, lay.A, lay.idx, separate=True)
    res["separate_scan"] = {"ms": round(ms_sep, 4), "G_tc_per_s": round(w.tc / ms_sep / 1e6, 3),
                            "separate_over_mixed": round(ms_sep / ms_mixed, 3),
                            "chunk": sc, "chunks": sn,
                            "workspace_MB": round(sep.workspace.numel() / 1e6, 1)}
    del sep, hfs
    idx1 = torch.zeros((w.B, w.L, 1), dtype=torch.int32, device=dev)
    gate1 = torch.ones((w.B, w.L, 1), dtype=torch.float32, device=dev)
    A1, b1, D1 = lay.A[:1].contiguous(), lay.bias[:1].contiguous(), lay.Dsk[:1].contiguous()
    dense = swimba.PreparedScan(False, lay.x, lay.dtr, lay.Bm, lay.Cm, idx1, gate1, A1, b1, D1,
                                y=lay.y, h_final=lay.hf, chunk=w.chunk)
    ms_dense = time_events(dense, reps, flush=flush)
    res["dense_scan"] = {"ms": round(ms_dense, 4), "G_tc_per_s": round(w.tc / ms_dense / 1e6, 3),
                         "mixed_over_dense": round(ms_mixed / ms_dense, 3)}
    return res, ms_mixed


def layer_mode(lay, swimba, dev, reps, flush):
    """A second workload: its timed step (router + mixed scan, events), the
    chunk pass against 8 TB/s and the VALU ceiling, and the mixed / dense /
    separate ratios."""
    w = lay.w
    ms_step = statistics.median(lay.timed_steps(reps, 2, phases=False)["step"])
    r = lay.timed_steps(reps, 1)
    chunk_ms = statistics.mean(r["chunk"])
    res = {"shape": "B=%d L=%d D=%d E=%d k=%d %s, chunk %d x %d" % (
        w.B, w.L, w.D, w.E, w.k, w.dtype, lay.chunk, lay.nchunks),
        "step_ms": round(ms_step, 4), "G_tc_per_s": round(w.tc / ms_step / 1e6, 3),
        "kernels_ms": {"route": round(statistics.mean(r["route"]), 4),
                       "chunk_pass": round(chunk_ms, 4),
                       "carry": round(statistics.mean(r["carry"]), 4),
                       "fixup": round(statistics.mean(r["fixup"]), 4)},
        "chunk_hbm": chunk_roofline(w, chunk_ms, load_traffic(w.name)),
        "chunk_valu_frac": chunk_valu(w, chunk_ms)["frac"]}
    ms_flushed = time_events(lay.step, reps, flush=flush)
    res["step_flushed_ms"] = round(ms_flushed, 4)
    rat, ms_mixed = ratios_at(lay, swimba, dev, reps)
    res.update(rat)
    res["scalar_a"] = scalar_a_mode(swimba, w, lay, reps, ms_mixed)
    return res


def modes(args, lay, swimba, workloads, dev):
    import torch
    reps = 10
    flush = Flusher(dev)
    res = {}
    # at the headline shape: the step after a cache-flushing write, and the
    # mixed / dense / separate scans
    ms_fl = time_events(lay.step, reps, flush=flush)
    res["step_flushed"] = {"ms": round(ms_fl, 4), "G_tc_per_s": round(lay.w.tc / ms_fl / 1e6, 3),
                           "note": "route + mixed scan after a 512 MB write, HIP events, median"}
    print("bench: modes at %s" % lay.w.name, file=sys.stderr, flush=True)
    rat, ms_mixed = ratios_at(lay, swimba, dev, reps)
    res.update(rat)
    # the Mamba-2 form (one transition per expert and channel) at this shape
    res["scalar_a"] = scalar_a_mode(swimba, lay.w, lay, reps, ms_mixed)
    for name in ("mamba1p4b_layer", "long_context"):
        if name == lay.w.name:
            continue
        print("bench: modes at %s" % name, file=sys.stderr, flush=True)
        other = Layer(workloads.BY_NAME[name], dev)
        res[name] = layer_mode(other, swimba, dev, reps, flush)
        del other
        torch.cuda.empty_cache()
    print("bench: expert sweep", file=sys.stderr, flush=True)
    res["expert_sweep"] = expert_sweep(swimba, dev, reps)
    print("bench: 130M-like layer forms", file=sys.stderr, flush=True)
    res["mamba130m_layer"] = small_layer_modes(swimba, workloads, dev, reps, flush)
    print("bench: decode", file=sys.stderr, flush=True)
    res["decode"] = decode_mode(swimba, workloads, dev, flush)
    return res


def expert_sweep(swimba, dev, reps):
    """Router + mixed scan at the Mamba-1.4B-like layer shape (B=8, L=4096,
    D=4096, top-2) for E = 2 .. 64 experts: the active experts, not the
    total, set the cost ("Fondements Théoriques", Theorem 2); beside it the
    mixed scan alone and the separate design on the same routing.  Inputs are
    seeded normal draws made on the GPU; an expert count the scans do not
    take is reported as such."""
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
    for E in (2, 4, 8, 16, 32, 64):
        Wr = torch.randn((D, E), generator=g, device=dev) / D ** 0.5
        A = -torch.exp(torch.rand((E, D, N_STATE), generator=g, device=dev) * math.log(16.0))
        bias = torch.randn((E, D), generator=g, device=dev) * 0.1 ** 0.5
        Dsk = torch.randn((E, D), generator=g, device=dev)
        route = swimba.PreparedRoute(x, Wr, k, idx, gate)
        try:
            scan = swimba.PreparedScan(False, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y=y,
                                       h_final=hf)
            route()
            scan()
        except swimba.SwimbaError as e:
            out["E%d" % E] = {"unsupported": str(e)}
            continue

        def step():
            route()
            scan()

        ms = time_events(step, reps)
        ms_route = time_events(route, reps)
        ms_scan = time_events(scan, reps)
        # the separate design on the same routing (its own chunking)
        hfs = torch.empty((B, E, D, N_STATE), dtype=torch.float32, device=dev)
        sep = swimba.PreparedScan(True, x, dtr, Bm, Cm, idx, gate, A, bias, Dsk, y=y,
                                  h_final=hfs)
        ms_sep = time_events(sep, reps)
        del sep, hfs
        base = base or ms
        out["E%d" % E] = {"ms": round(ms, 4), "route_ms": round(ms_route, 4),
                          "G_tc_per_s": round(B * L * D / ms / 1e6, 3),
                          "over_E2": round(ms / base, 3),
                          "scan_ms": round(ms_scan, 4), "separate_ms": round(ms_sep, 4),
                          "separate_over_mixed": round(ms_sep / ms_scan, 3)}
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
    whole backward call: forward recompute with the chunk records, the
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
    ms = time_events(call, reps)
    return {"ms": round(ms, 4), "G_tc_per_s": round(w.tc / ms / 1e6, 3),
            "over_forward_scan": round(ms / ms_mixed, 3),
            "workspace_MB": round(call.workspace.numel() / 1e6, 1),
            "note": "fp32 gradients of x, dt_raw, B, C, gates, A, dt_bias, Dskip, h0"}


def phase_ms(call, reps):
    """Mean chunk / carry / fix-up durations of `reps` calls of a prepared
    scan, from events its kernels' dispatches stamp."""
    import torch
    h = hip()
    ev = [[h.event() for _ in range(6)] for _ in range(reps)]
    arrs = [(ctypes.c_void_p * 6)(*[e_.value for e_ in e]) for e in ev]
    for a in arrs:
        call(ctypes.addressof(a))
    torch.cuda.synchronize()
    return [sum(h.ms(e[2 * i], e[2 * i + 1]) for e in ev) / reps for i in range(3)]


def scalar_a_mode(swimba, w, lay, reps, ms_mixed):
    """The mixed scan with one transition per (expert, channel), the Mamba-2
    form A_t = a_t I, on the same inputs (A[e, d] = the n = 0 entry of the
    diagonal draw): one exponential per (token, channel) instead of 16.  The
    scan alone, and its chunk pass against the VALU ceiling and 8 TB/s."""
    As = lay.A[:, :, 0].contiguous()
    scan = swimba.PreparedScan(False, lay.x, lay.dtr, lay.Bm, lay.Cm, lay.idx, lay.gate, As,
                               lay.bias, lay.Dsk, y=lay.y, h_final=lay.hf, chunk=w.chunk)
    ms = time_events(scan, reps)
    chunk_ms, _, fixup_ms = phase_ms(scan, reps)
    tc = w.tc
    tf = tc * scalar_a_slots_per_tc(w.k) * 2 / (chunk_ms * 1e-3) / 1e12
    gbs = tc * algorithmic_bytes_per_tc(w.dtype) / (chunk_ms * 1e-3) / 1e9
    return {"scan_ms": round(ms, 4), "G_tc_per_s": round(tc / ms / 1e6, 3),
            "over_diagonal": round(ms / ms_mixed, 3),
            "chunk_pass_ms": round(chunk_ms, 4), "fixup_ms": round(fixup_ms, 4),
            "valu_frac": round(tf / VALU_PEAK_TFLOPS, 4),
            "valu_note": "%d slots/tc as FMA-equivalent flops" % scalar_a_slots_per_tc(w.k),
            "hbm_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def stream_mode(swimba, workloads, w, lay, reps):
    """The pages' stream-mixed form at the same layer shape: shared A, each of
    the k slots carries its expert's X, B and C streams, the injection and the
    readout are mixed by the gates ("Kernmechanisme van Swimba").  Times the
    router on the layer's x plus the stream scan, and the scan's chunk pass
    alone (dispatch-stamped events) against the VALU ceiling and 8 TB/s."""
    import numpy as np
    import torch
    dev = lay.x.device
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
    chunk_len, nchunks = swimba.scan_streams_plan(T["X"])
    ms_scan = time_events(scan, reps)

    def step():
        lay.route()
        scan()

    ms_step = time_events(step, reps)
    chunk_ms, carry_ms, fixup_ms = phase_ms(scan, reps)
    tc, k = w.tc, w.k
    esz = 2 if w.dtype == "bf16" else 4
    tf = tc * stream_slots_per_tc(k) * 2 / (chunk_ms * 1e-3) / 1e12
    # X (k slots) and dt_raw read, y written
    gbs = tc * (k + 2) * esz / (chunk_ms * 1e-3) / 1e9
    return {"shape": "B=%d L=%d D=%d k=%d %s, chunk %d x %d" % (w.B, w.L, w.D, k, w.dtype,
                                                              chunk_len, nchunks),
            "scan_ms": round(ms_scan, 4), "G_tc_per_s": round(tc / ms_scan / 1e6, 3),
            "route_plus_scan_ms": round(ms_step, 4),
            "chunk_pass_ms": round(chunk_ms, 4), "carry_ms": round(carry_ms, 4),
            "fixup_ms": round(fixup_ms, 4),
            "valu_frac": round(tf / VALU_PEAK_TFLOPS, 4),
            "valu_note": "%d slots/tc as FMA-equivalent flops" % stream_slots_per_tc(k),
            "hbm_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def small_layer_modes(swimba, workloads, dev, reps, flush):
    """The Mamba-130M-like layer (77 MB of streams, inside the 256 MB
    Infinity Cache): the step steady-state and after a cache-flushing write,
    and the other forms of the scan at this shape."""
    import torch
    w = workloads.BY_NAME["mamba130m_layer"]
    lay = Layer(w, dev)
    res = {"shape": "B=%d L=%d D=%d E=%d k=%d %s, chunk %d x %d" % (
        w.B, w.L, w.D, w.E, w.k, w.dtype, lay.chunk, lay.nchunks)}
    ms_step = statistics.median(lay.timed_steps(reps, 2, phases=False)["step"])
    r = lay.timed_steps(reps, 1)
    res["step_ms"] = round(ms_step, 4)
    res["kernels_ms"] = {"route": round(statistics.mean(r["route"]), 4),
                         "chunk_pass": round(statistics.mean(r["chunk"]), 4),
                         "carry": round(statistics.mean(r["carry"]), 4),
                         "fixup": round(statistics.mean(r["fixup"]), 4)}
    ms_fl = time_events(lay.step, reps, flush=flush)
    res["step_flushed_ms"] = round(ms_fl, 4)
    res["step_flushed_G_tc_per_s"] = round(w.tc / ms_fl / 1e6, 3)
    rat, ms_mixed = ratios_at(lay, swimba, dev, reps)
    res.update(rat)
    hfk = torch.empty((w.B, w.k, w.D, N_STATE), dtype=torch.float32, device=dev)
    slots = swimba.PreparedScan(swimba.DESIGN_SLOTS, lay.x, lay.dtr, lay.Bm, lay.Cm, lay.idx,
                                lay.gate, lay.A, lay.bias, lay.Dsk, y=lay.y, h_final=hfk)
    ms_slots = time_events(slots, reps)
    res["slots_scan"] = {"ms": round(ms_slots, 4), "G_tc_per_s": round(w.tc / ms_slots / 1e6, 3),
                         "slots_over_mixed": round(ms_slots / ms_mixed, 3)}
    del hfk, slots
    hfa = torch.empty((w.B, w.E, w.D, N_STATE), dtype=torch.float32, device=dev)
    alle = swimba.PreparedScan(swimba.DESIGN_ALL_EXPERTS, lay.x, lay.dtr, lay.Bm, lay.Cm,
                               lay.idx, lay.gate, lay.A, lay.bias, lay.Dsk, y=lay.y, h_final=hfa)
    ms_all = time_events(alle, reps)
    res["all_experts_scan"] = {"ms": round(ms_all, 4), "G_tc_per_s": round(w.tc / ms_all / 1e6, 3),
                               "all_experts_over_mixed": round(ms_all / ms_mixed, 3)}
    del hfa, alle
    res["stream_mixed"] = stream_mode(swimba, workloads, w, lay, reps)
    zoh = swimba.PreparedScan(False, lay.x, lay.dtr, lay.Bm, lay.Cm, lay.idx, lay.gate, lay.A,
                              lay.bias, lay.Dsk, y=lay.y, h_final=lay.hf, chunk=w.chunk, zoh=True)
    ms_zoh = time_events(zoh, reps)
    res["zoh_scan"] = {"ms": round(ms_zoh, 4), "G_tc_per_s": round(w.tc / ms_zoh / 1e6, 3),
                       "over_euler": round(ms_zoh / ms_mixed, 3),
                       "note": "zero-order-hold input term, B_bar = A^-1 (exp(Delta A) - I) B"}
    res["theorem4"] = theorem4_mode(swimba, workloads, w, lay.x, lay.dtr, lay.Bm, lay.Cm, lay.A,
                                    lay.bias, lay.Dsk)
    res["backward"] = backward_mode(swimba, w, lay.x, lay.dtr, lay.Bm, lay.Cm, lay.idx, lay.gate,
                                    lay.A, lay.bias, lay.Dsk, reps, ms_mixed)
    res["scalar_a"] = scalar_a_mode(swimba, w, lay, reps, ms_mixed)
    return res


def decode_mode(swimba, workloads, dev, flush):
    """The decode workload: 128 routed steps on a persistent fp32 state
    (B = 256, D = 5120, E = 8, top-2).  Steady-state (the 84 MB state stays
    in the Infinity Cache between steps), after a cache-flushing write before
    every step, and the 128 steps captured once in a HIP graph."""
    import numpy as np
    import torch
    wd = workloads.BY_NAME["decode"]
    p, steps = workloads.decode_steps(wd)
    dd = torch.bfloat16 if wd.dtype == "bf16" else torch.float32
    P = {kk: torch.from_numpy(v).to(dev) for kk, v in p.items()}
    S = [{kk: torch.from_numpy(np.ascontiguousarray(v)).to(dd).to(dev) for kk, v in s.items()}
         for s in steps]
    state = torch.zeros((wd.B, wd.D, N_STATE), dtype=torch.float32, device=dev)
    yd = torch.empty((wd.B, wd.D), dtype=dd, device=dev)
    calls = [swimba.PreparedStep(s["x"], s["dt_raw"], s["Bm"], s["Cm"], P["A"], P["dt_bias"],
                                 P["Dskip"], state, Wr=P["Wr"], k=wd.k, y=yd) for s in S]
    n = len(calls)
    h = hip()
    st = stream_of_torch()

    def per_step(flushing, seq=None):
        seq = seq or calls
        evs = [(h.event(), h.event()) for _ in range(n)]
        # three full passes first: the first steps after a pause run slower
        for _ in range(3):
            for c in seq:
                c()
        for c, (e0, e1) in zip(seq, evs):
            if flushing:
                flush()
            h.record(e0, st)
            c()
            h.record(e1, st)
        torch.cuda.synchronize()
        return statistics.median(h.ms(e0, e1) for e0, e1 in evs)

    us_steady = per_step(False) * 1e3
    us_flushed = per_step(True) * 1e3
    # the same steps with the routing given (the router's cost is the gap)
    idx = torch.empty((wd.B, wd.k), dtype=torch.int32, device=dev)
    gate = torch.empty((wd.B, wd.k), dtype=torch.float32, device=dev)
    swimba.PreparedStep(S[0]["x"], S[0]["dt_raw"], S[0]["Bm"], S[0]["Cm"], P["A"],
                        P["dt_bias"], P["Dskip"], state, Wr=P["Wr"], k=wd.k, y=yd,
                        idx_out=idx, gate_out=gate)()
    given = [swimba.PreparedStep(s["x"], s["dt_raw"], s["Bm"], s["Cm"], P["A"], P["dt_bias"],
                                 P["Dskip"], state, idx=idx, gate=gate, y=yd) for s in S]
    us_given = per_step(False, given) * 1e3

    def run_all():
        for c in calls:
            c()

    ms_all = time_events(run_all, 3, warm=1)
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
    ms_graph = time_events(graph.replay, 3, warm=1)
    esz = 2 if wd.dtype == "bf16" else 4
    # state read and written (fp32), x and dt_raw read and y written per channel
    per_step_bytes = wd.B * wd.D * (2 * N_STATE * 4 + 3 * esz)
    gbs = per_step_bytes / (us_steady * 1e-6) / 1e9
    gbs_fl = per_step_bytes / (us_flushed * 1e-6) / 1e9
    return {"workload": wd.name, "steps": n,
            "us_per_step": round(us_steady, 2),
            "G_channel_steps_per_s": round(wd.B * wd.D / us_steady / 1e3, 3),
            "hbm_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "us_per_step_flushed": round(us_flushed, 2),
            "hbm_frac_flushed": round(gbs_fl / HBM_PEAK_GBS, 4),
            "us_per_step_routing_given": round(us_given, 2),
            "us_per_step_back_to_back": round(ms_all * 1e3 / n, 2),
            "graph_us_per_step": round(ms_graph * 1e3 / n, 2),
            "bytes_per_step": per_step_bytes,
            "note": "per-step HIP events, median over the 128 steps; the 84 MB state stays in "
                    "the 256 MB Infinity Cache in steady state; flushed = a 512 MB write "
                    "before each step; routing given = idx/gate passed in, no fused router; "
                    "graph = the 128 steps captured once and replayed"}


if __name__ == "__main__":
    main()
