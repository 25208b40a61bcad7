"""Seeded synthetic workloads for the Swimba scan: shapes and value recipes.

This module holds data only -- shapes, seeds and random draws -- and none of
the method's arithmetic, so both the HIP path's tests/benchmark and the CPU
oracle's tests can use it without sharing any computation.

The pages publish no layer shapes and measure only on public NLP benchmarks
with trained weights; these seeded tensors stand in for them at the layer
shapes named below.  Recipe (seed = workload index, numpy PCG64):
  draw order   Wr, A, dt_bias, Dskip, then x, dt_raw, B, C
               (decode: parameters first, then x, dt_raw, B, C per step)
  x, dt_raw, B, C ~ N(0, 1), rounded to bf16 (round-to-nearest-even) for the
               bf16 workloads
  A_e          = -exp(U(0, ln 16)), one draw per (e, d, n)  -> [-16, -1]
  dt_bias_e    ~ N(0, 0.1)   (variance 0.1)
  Dskip_e      ~ N(0, 1)
  Wr           ~ N(0, 1/D)   (variance 1/D: unit-variance logits)

Stream-mixed inputs (``generate_streams``; seed = the workload's seed + 1000):
  draw order   A, dt_bias, then X, dt_raw, Bs, Cs, gate
  A            = -exp(U(0, ln 16)) per (d, n); dt_bias ~ N(0, 0.1)
  X [B,L,k,D], dt_raw [B,L,D], Bs, Cs [B,L,k,N] ~ N(0, 1), bf16-rounded for
               bf16 workloads
  gate [B,L,k] ~ Dirichlet(1, ..., 1): convex weights of the k slots
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    D: int
    N: int
    E: int
    k: int
    dtype: str          # "f32" or "bf16": dtype of x, dt_raw, B, C (and y)
    seed: int
    chunk: int = 0      # 0 = library's choice
    steps: int = 0      # decode workloads: number of single-token steps

    @property
    def tokens(self) -> int:
        return self.B * self.L

    @property
    def tc(self) -> int:
        """token x channel count of one scan pass (decode: per step)."""
        return self.B * self.L * self.D


WORKLOADS = [
    Workload("tiny", B=1, L=256, D=64, N=16, E=4, k=1, dtype="f32", seed=0),
    Workload("mamba130m_layer", B=4, L=2048, D=1536, N=16, E=8, k=2, dtype="bf16", seed=1),
    Workload("mamba1p4b_layer", B=8, L=4096, D=4096, N=16, E=8, k=2, dtype="bf16", seed=2),
    Workload("long_context", B=1, L=65536, D=2560, N=16, E=16, k=2, dtype="bf16", seed=3,
             chunk=256),
    Workload("decode", B=256, L=1, D=5120, N=16, E=8, k=2, dtype="bf16", seed=4, steps=128),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 holding the rounded values (finite inputs only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    u = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(rng, shape, std=1.0):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


def params(w: Workload, rng: np.random.Generator | None = None, E: int | None = None,
           D: int | None = None, N: int | None = None):
    """Expert/router parameters, float32: Wr [D,E], A [E,D,N], dt_bias [E,D],
    Dskip [E,D].  ``rng`` defaults to a fresh PCG64(seed)."""
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(w.seed))
    E = E or w.E
    D = D or w.D
    N = N or w.N
    Wr = _normal(rng, (D, E), 1.0 / math.sqrt(D))
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=(E, D, N))).astype(np.float32)
    dt_bias = _normal(rng, (E, D), math.sqrt(0.1))
    Dskip = _normal(rng, (E, D))
    return dict(Wr=Wr, A=A, dt_bias=dt_bias, Dskip=Dskip)


def streams(w: Workload, rng: np.random.Generator, B: int | None = None, L: int | None = None,
            D: int | None = None, N: int | None = None):
    """Per-token streams x, dt_raw [B,L,D] and Bm, Cm [B,L,N] as float32
    values (bf16-rounded for bf16 workloads)."""
    B = B or w.B
    L = L or w.L
    D = D or w.D
    N = N or w.N
    out = {}
    for name, shape in (("x", (B, L, D)), ("dt_raw", (B, L, D)), ("Bm", (B, L, N)),
                        ("Cm", (B, L, N))):
        v = _normal(rng, shape)
        out[name] = bf16_round(v) if w.dtype == "bf16" else v
    return out


def generate(w: Workload):
    """Parameters and streams of a scan workload, drawn in the fixed order."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    p = params(w, rng)
    s = streams(w, rng)
    p.update(s)
    return p


def decode_steps(w: Workload, steps: int | None = None):
    """Parameters, then a generator of per-step streams x, dt_raw [B,D],
    Bm, Cm [B,N] for the decode workload."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    p = params(w, rng)
    n = w.steps if steps is None else steps

    def gen():
        for _ in range(n):
            s = streams(w, rng, L=1)
            yield {k: v[:, 0] for k, v in s.items()}

    return p, gen()


def generate_streams(w: Workload, k: int | None = None, B: int | None = None,
                     L: int | None = None, D: int | None = None):
    """Inputs of the stream-mixed scan at a workload's shape: shared A [D,N],
    dt_bias [D]; per-slot streams X [B,L,k,D], Bs, Cs [B,L,k,N]; dt_raw
    [B,L,D]; gate [B,L,k].  float32 arrays (streams bf16-rounded for bf16
    workloads)."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
    k = k or w.k
    B = w.B if B is None else B
    L = w.L if L is None else L
    D = D or w.D
    N = w.N
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=(D, N))).astype(np.float32)
    dt_bias = _normal(rng, (D,), math.sqrt(0.1))
    out = dict(A=A, dt_bias=dt_bias)
    for name, shape in (("X", (B, L, k, D)), ("dt_raw", (B, L, D)), ("Bs", (B, L, k, N)),
                        ("Cs", (B, L, k, N))):
        v = _normal(rng, shape)
        out[name] = bf16_round(v) if w.dtype == "bf16" else v
    out["gate"] = rng.dirichlet(np.ones(k), size=(B, L)).astype(np.float32)
    return out


def switching_routing(B: int, L: int, E: int, p: float, seed: int):
    """Top-1 routing that switches expert with probability p per token: the
    first token's expert is uniform over E; afterwards each token keeps the
    previous expert with probability 1 - p, else takes one of the other
    E - 1 uniformly.  Returns idx [B, L, 1] int32 and gate [B, L, 1] = 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = np.empty((B, L), np.int32)
    idx[:, 0] = rng.integers(0, E, size=B)
    switch = rng.random((B, L)) < p
    step = rng.integers(1, E, size=(B, L)) if E > 1 else np.zeros((B, L), np.int64)
    for t in range(1, L):
        idx[:, t] = np.where(switch[:, t], (idx[:, t - 1] + step[:, t]) % E, idx[:, t - 1])
    return idx[:, :, None].copy(), np.ones((B, L, 1), np.float32)
