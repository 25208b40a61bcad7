"""Calls on a caller's stream: the binding allocates the workspace on the
current stream and records it on the caller's, so a side-stream call that
overlaps other allocations gives the same result as the default stream."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev_tensors
from parameter_space_moe_amd import swimba, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_scan_on_side_stream_matches_default():
    w = workloads.Workload("side", B=2, L=900, D=192, N=16, E=4, k=2, dtype="bf16", seed=31)
    inp = workloads.generate(w)
    t = dev_tensors(inp, "bf16", DEV)
    idx, gate = swimba.route(t["x"], t["Wr"], 2)
    a = (t["x"], t["dt_raw"], t["Bm"], t["Cm"], idx, gate, t["A"], t["dt_bias"], t["Dskip"])
    y0, h0 = swimba.scan(*a, chunk=64)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        y, h = swimba.scan(*a, chunk=64, stream=side)
        outs.append((y, h))
        # allocations on the current stream while the side stream may still run
        junk = torch.full((1 << 22,), 7.0, device=DEV)
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for y, h in outs:
        assert torch.equal(y, y0) and torch.equal(h, h0)
