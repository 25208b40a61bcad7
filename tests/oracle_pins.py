"""Pins for the CPU oracle: checks that fix what the oracle computes from
something other than the oracle itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load(path)``)
and raises ``AssertionError`` when the oracle disagrees with what the pages
and the mathematics fix:
  * hand-derived worked examples (``tests/golden/worked_examples.json``);
  * closed forms (the geometric series for constant inputs);
  * brute-force unrolling of the recurrence on tiny inputs;
  * special cases that reduce to another computation (E = 1 and identical
    experts reduce to the plain Mamba scan, Theorem 1 of "Swimba: Switch Mamba
    Model Scales State Space Models"; top-1 one-hot routing runs one expert
    alone; k = E in the separate design is E independent scans);
  * invariants (stability bound, Theorem 3; split-sequence composition;
    linearity in x; the two designs differ under time-varying routing,
    Theorem 4);
  * brute-force sorting for the router;
  * the zero-order-hold option: the continuous equilibrium under constant
    input, the semigroup property (two half steps = one step), and the
    small-A limit where it meets Euler;
  * per-slot trajectories (the other separate reading): each slot is the
    mixed scan's gate-1 top-1 form of that slot's routing, its state carries
    across expert switches, gates weight only the outputs, and constant
    routing meets the per-expert trajectories;
  * the backward of the mixed scan against central differences of the
    forward, and the support of its gradients for a single-token loss;
  * for the stream-mixed form (shared A, mixed B X injection and C readout):
    one slot or identical slots reduce to the plain Mamba scan, a zero-weight
    slot drops out, slots permute freely, the state superposes over slots
    and the readout is linear in C, plus its own worked examples, closed
    form, stability bound and split composition.
The same functions run against mutated copies of the oracle in
``test_oracle_mutations.py``: every planted mistake must trip at least one.
"""
from __future__ import annotations

import fractions
import json
import math
import os
import re

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.json")

_TOK = re.compile(r"\s*(ln|e\b|[0-9.]+|[-+*/()])")


def eval_expr(s: str) -> float:
    """Evaluate an input string of the golden file: numbers, e, ln(), + - * /."""
    toks = []
    pos = 0
    s = s.strip()
    while pos < len(s):
        m = _TOK.match(s, pos)
        if not m:
            raise ValueError("bad token in %r" % s)
        toks.append(m.group(1))
        pos = m.end()
    toks.append(None)
    i = [0]

    def peek():
        return toks[i[0]]

    def take():
        t = toks[i[0]]
        i[0] += 1
        return t

    def atom():
        t = take()
        if t == "(":
            v = expr()
            assert take() == ")"
            return v
        if t == "-":
            return -atom()
        if t == "ln":
            assert take() == "("
            v = expr()
            assert take() == ")"
            return math.log(v)
        if t == "e":
            return math.e
        return float(t)

    def term():
        v = atom()
        while peek() in ("*", "/"):
            if take() == "*":
                v *= atom()
            else:
                v /= atom()
        return v

    def expr():
        v = term()
        while peek() in ("+", "-"):
            if take() == "+":
                v += term()
            else:
                v -= term()
        return v

    v = expr()
    assert peek() is None, s
    return v


def _arr(nested, fn=eval_expr):
    if isinstance(nested, list):
        return [_arr(v, fn) for v in nested]
    return fn(nested)


def _frac(nested):
    return np.array(_arr(nested, lambda s: float(fractions.Fraction(s))))


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, "%s: max err %.3e > %.1e" % (what, err, tol * scale)


def _softplus(z):
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _rand_case(rng, B=2, L=7, D=3, N=4, E=3, k=2, h0=True):
    x = rng.standard_normal((B, L, D))
    dt_raw = rng.standard_normal((B, L, D))
    Bm = rng.standard_normal((B, L, N))
    Cm = rng.standard_normal((B, L, N))
    A = -np.exp(rng.uniform(0, math.log(16), (E, D, N)))
    dt_bias = rng.standard_normal((E, D)) * 0.3
    Dskip = rng.standard_normal((E, D))
    idx = np.stack([np.stack([rng.permutation(E)[:k] for _ in range(L)]) for _ in range(B)])
    g = rng.uniform(0.1, 1.0, (B, L, k))
    gate = g / g.sum(-1, keepdims=True)
    H = rng.standard_normal((B, D, N)) if h0 else None
    return dict(x=x, dt_raw=dt_raw, Bm=Bm, Cm=Cm, idx=idx.astype(np.int32), gate=gate, A=A,
                dt_bias=dt_bias, Dskip=Dskip, h0=H)


# ------------------------------------------------------------ worked examples
def pin_worked_scan(lib):
    """Hand-derived examples: softplus at three closed-form points, mixing
    with unequal gates, readout after the update, the D term."""
    gold = json.load(open(GOLDEN))
    for c in gold["scan_cases"]:
        y, hf = oracle.scan(_arr(c["x"]), _arr(c["dt_raw"]), _arr(c["Bm"]), _arr(c["Cm"]),
                            np.array(c["idx"], np.int32), _arr(c["gate"]), _arr(c["A"]),
                            _arr(c["dt_bias"]), _arr(c["Dskip"]), lib=lib)
        _close(y, _frac(c["expected_y"]), 1e-12, c["name"] + " y")
        _close(hf, _frac(c["expected_h_final"]), 1e-12, c["name"] + " h_final")


def pin_worked_separate(lib):
    gold = json.load(open(GOLDEN))
    for c in gold["separate_cases"]:
        y, hf = oracle.scan_separate(_arr(c["x"]), _arr(c["dt_raw"]), _arr(c["Bm"]),
                                     _arr(c["Cm"]), np.array(c["idx"], np.int32),
                                     _arr(c["gate"]), _arr(c["A"]), _arr(c["dt_bias"]),
                                     _arr(c["Dskip"]), lib=lib)
        _close(y, _frac(c["expected_y"]), 1e-12, c["name"] + " y")
        _close(hf, _frac(c["expected_h_final"]), 1e-12, c["name"] + " h_final")


def pin_worked_route(lib):
    gold = json.load(open(GOLDEN))
    for c in gold["route_cases"]:
        idx, gate, logits, _ = oracle.route(_arr(c["x"]), _arr(c["Wr"]), c["k"], lib=lib)
        assert idx.tolist() == c["expected_idx"], (c["name"], idx.tolist())
        _close(gate, _arr(c["expected_gate"]), 1e-15, c["name"] + " gate")


# --------------------------------------------------------------- closed forms
def pin_constant_input_geometric(lib):
    """Constant x, dt_raw, B, C and routing: a and b are constant, so
    h_t = a^t h0 + b (1 - a^t) / (1 - a) and y_t = C.h_t + delta x."""
    B, L, D, N, E, k = 1, 40, 2, 3, 3, 2
    x = np.broadcast_to(np.array([0.7, -1.3]), (B, L, D)).copy()
    dt_raw = np.broadcast_to(np.array([0.2, -0.9]), (B, L, D)).copy()
    Bv, Cv = np.array([0.5, -1.0, 2.0]), np.array([1.5, 0.25, -0.75])
    Bm = np.broadcast_to(Bv, (B, L, N)).copy()
    Cm = np.broadcast_to(Cv, (B, L, N)).copy()
    A = -np.array([[[1.0, 2.0, 4.0], [1.5, 3.0, 0.5]],
                   [[8.0, 1.25, 2.5], [0.75, 6.0, 1.0]],
                   [[3.0, 3.0, 3.0], [2.0, 2.0, 2.0]]])
    dt_bias = np.array([[0.1, -0.2], [0.3, 0.05], [-0.4, 0.6]])
    Dskip = np.array([[1.0, -0.5], [0.25, 2.0], [3.0, 3.0]])
    e = np.array([2, 0], np.int32)
    g = np.array([0.6, 0.4])
    idx = np.broadcast_to(e, (B, L, k)).copy()
    gate = np.broadcast_to(g, (B, L, k)).copy()
    h0 = np.array([[[0.3, -0.2, 1.0], [2.0, 0.0, -1.0]]])
    y, hf = oracle.scan(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, lib=lib)
    t = np.arange(1, L + 1)[:, None]
    for d in range(D):
        beta = g[0] * dt_bias[2, d] + g[1] * dt_bias[0, d]
        delta = g[0] * Dskip[2, d] + g[1] * Dskip[0, d]
        Dt = math.log1p(math.exp(dt_raw[0, 0, d] + beta))
        a = np.exp(Dt * (g[0] * A[2, d] + g[1] * A[0, d]))
        b = Dt * Bv * x[0, 0, d]
        h = a ** t * h0[0, d] + b * (1 - a ** t) / (1 - a)
        _close(y[0, :, d], h @ Cv + delta * x[0, 0, d], 1e-12, "geometric y d=%d" % d)
        _close(hf[0, d], h[-1], 1e-12, "geometric h d=%d" % d)


def pin_bruteforce_unroll(lib):
    """h_t = prod_{1..t} a * h0 + sum_{s<=t} (prod_{s<tau<=t} a_tau) b_s, with
    y_t read from h_t: fixes the order of update and readout and the carry."""
    rng = np.random.default_rng(11)
    c = _rand_case(rng, B=1, L=6, D=2, N=3, E=3, k=2)
    y, hf = oracle.scan(**c, lib=lib)
    for d in range(2):
        idx, g = c["idx"][0], c["gate"][0]
        beta = np.einsum("tj,tj->t", g, c["dt_bias"][idx, d])
        delta = np.einsum("tj,tj->t", g, c["Dskip"][idx, d])
        Dt = _softplus(c["dt_raw"][0, :, d] + beta)
        Abar = np.einsum("tj,tjn->tn", g, c["A"][idx, d])
        a = np.exp(Dt[:, None] * Abar)
        b = Dt[:, None] * c["Bm"][0] * c["x"][0, :, d][:, None]
        for t in range(6):
            h = np.prod(a[:t + 1], axis=0) * c["h0"][0, d]
            for s in range(t + 1):
                h = h + np.prod(a[s + 1:t + 1], axis=0) * b[s]
            want = c["Cm"][0, t] @ h + delta[t] * c["x"][0, t, d]
            _close(y[0, t, d], want, 1e-12, "unroll y t=%d d=%d" % (t, d))
        _close(hf[0, d], h, 1e-12, "unroll h d=%d" % d)


# --------------------------------------------------------- special cases
def pin_single_expert_is_mamba(lib):
    """E = 1 (gate 1): the mixed scan is the plain selective scan."""
    rng = np.random.default_rng(12)
    c = _rand_case(rng, B=2, L=9, D=3, N=4, E=1, k=1)
    c["gate"][:] = 1.0
    y, hf = oracle.scan(**c, lib=lib)
    ym, hm = oracle.mamba_scan(c["x"], c["dt_raw"], c["Bm"], c["Cm"], c["A"][0],
                               c["dt_bias"][0], c["Dskip"][0], c["h0"], lib=lib)
    _close(y, ym, 1e-13, "E=1 y")
    _close(hf, hm, 1e-13, "E=1 h")


def pin_identical_experts_is_mamba(lib):
    """Identical experts with any convex routing collapse to one expert."""
    rng = np.random.default_rng(13)
    c = _rand_case(rng, B=1, L=8, D=3, N=4, E=4, k=3)
    for key in ("A", "dt_bias", "Dskip"):
        c[key] = np.broadcast_to(c[key][:1], c[key].shape).copy()
    y, hf = oracle.scan(**c, lib=lib)
    ym, hm = oracle.mamba_scan(c["x"], c["dt_raw"], c["Bm"], c["Cm"], c["A"][0],
                               c["dt_bias"][0], c["Dskip"][0], c["h0"], lib=lib)
    _close(y, ym, 1e-12, "identical experts y")
    _close(hf, hm, 1e-12, "identical experts h")


def pin_top1_onehot_is_expert_alone(lib):
    """Forced top-1 routing to expert e: the scan is expert e's scan alone."""
    rng = np.random.default_rng(14)
    c = _rand_case(rng, B=1, L=8, D=3, N=2, E=4, k=1)
    c["gate"][:] = 1.0
    for e in range(4):
        c["idx"][:] = e
        y, hf = oracle.scan(**c, lib=lib)
        ym, hm = oracle.mamba_scan(c["x"], c["dt_raw"], c["Bm"], c["Cm"], c["A"][e],
                                   c["dt_bias"][e], c["Dskip"][e], c["h0"], lib=lib)
        _close(y, ym, 1e-13, "top-1 expert %d y" % e)
        _close(hf, hm, 1e-13, "top-1 expert %d h" % e)


def pin_split_composition(lib):
    """scan(L1 ++ L2) = scan(L2, h0 = scan(L1).h_final): state carry."""
    rng = np.random.default_rng(15)
    c = _rand_case(rng, B=2, L=10, D=3, N=4, E=3, k=2)
    y, hf = oracle.scan(**c, lib=lib)
    first = {k_: (v[:, :4] if k_ in ("x", "dt_raw", "Bm", "Cm", "idx", "gate") else v)
             for k_, v in c.items()}
    second = {k_: (v[:, 4:] if k_ in ("x", "dt_raw", "Bm", "Cm", "idx", "gate") else v)
              for k_, v in c.items()}
    y1, h1 = oracle.scan(**first, lib=lib)
    second["h0"] = h1
    y2, h2 = oracle.scan(**second, lib=lib)
    _close(np.concatenate([y1, y2], 1), y, 1e-13, "split y")
    _close(h2, hf, 1e-13, "split h")


def pin_linear_in_x(lib):
    """With dt_raw and routing fixed, y and h are linear in (x, h0)."""
    rng = np.random.default_rng(16)
    c1 = _rand_case(rng, B=1, L=8, D=3, N=4, E=3, k=2)
    c2 = dict(c1)
    c2["x"] = rng.standard_normal(c1["x"].shape)
    c2["h0"] = rng.standard_normal(c1["h0"].shape)
    c3 = dict(c1)
    c3["x"] = 2.0 * c1["x"] - 3.0 * c2["x"]
    c3["h0"] = 2.0 * c1["h0"] - 3.0 * c2["h0"]
    ya, ha = oracle.scan(**c1, lib=lib)
    yb, hb = oracle.scan(**c2, lib=lib)
    yc, hc = oracle.scan(**c3, lib=lib)
    _close(yc, 2 * ya - 3 * yb, 1e-12, "linearity y")
    _close(hc, 2 * ha - 3 * hb, 1e-12, "linearity h")


def pin_stability_bound(lib):
    """Theorem 3 (BIBO under contractive transitions): with A <= Amax < 0,
    Delta >= Dmin > 0, |x|, |B| <= 1 and Delta <= Dmax, every state stays
    within Dmax / (1 - exp(Dmin Amax)), and the mixed decay lies between the
    selected experts' extremes."""
    rng = np.random.default_rng(17)
    B, L, D, N, E, k = 1, 200, 3, 4, 4, 2
    c = _rand_case(rng, B=B, L=L, D=D, N=N, E=E, k=k, h0=False)
    c["x"] = rng.uniform(-1, 1, c["x"].shape)
    c["Bm"] = rng.uniform(-1, 1, c["Bm"].shape)
    c["dt_bias"][:] = 0.0
    c["dt_raw"] = rng.uniform(-2, 2, c["dt_raw"].shape)
    y, hf = oracle.scan(**c, lib=lib)
    Dmin, Dmax = _softplus(-2.0), _softplus(2.0)
    Amax = c["A"].max()
    bound = Dmax / (1 - math.exp(Dmin * Amax))
    # the state at every step: run prefixes
    for L1 in (1, 7, 50, 200):
        part = {k_: (v[:, :L1] if k_ in ("x", "dt_raw", "Bm", "Cm", "idx", "gate") else v)
                for k_, v in c.items()}
        _, h = oracle.scan(**part, lib=lib)
        assert np.all(np.abs(h) <= bound * (1 + 1e-12)), "stability bound violated"
    assert np.all(np.isfinite(y))
    # forward a single token from a known state: 0 < a < 1 (a = decay of h0)
    one = {k_: (v[:, :1] if k_ in ("x", "dt_raw", "Bm", "Cm", "idx", "gate") else v)
           for k_, v in c.items()}
    one["x"] = np.zeros_like(one["x"])
    one["h0"] = np.ones((B, D, N))
    _, h = oracle.scan(**one, lib=lib)
    e = one["idx"][0, 0]
    Dt = _softplus(one["dt_raw"][0, 0])
    lo = np.exp(Dt[:, None] * c["A"][e].min(0))
    hi = np.exp(Dt[:, None] * c["A"][e].max(0))
    assert np.all(h[0] > 0) and np.all(h[0] < 1), "mixed decay outside (0,1)"
    assert np.all(h[0] >= lo * (1 - 1e-12)) and np.all(h[0] <= hi * (1 + 1e-12)), \
        "mixed decay outside the selected experts' range"


# --------------------------------------------------------------- separate
def pin_separate_all_experts(lib):
    """k = E: every expert advances at every token, so the separate design is
    E independent plain scans whose outputs are mixed by the gates."""
    rng = np.random.default_rng(18)
    B, L, D, N, E = 1, 7, 2, 3, 3
    c = _rand_case(rng, B=B, L=L, D=D, N=N, E=E, k=E, h0=False)
    H0 = rng.standard_normal((B, E, D, N))
    y, hf = oracle.scan_separate(**{**c, "h0": H0}, lib=lib)
    want = np.zeros((B, L, D))
    for e in range(E):
        ye, he = oracle.mamba_scan(c["x"], c["dt_raw"], c["Bm"], c["Cm"], c["A"][e],
                                   c["dt_bias"][e], c["Dskip"][e], H0[:, e], lib=lib)
        w = (c["gate"] * (c["idx"] == e)).sum(-1)
        want += w[..., None] * ye
        _close(hf[:, e], he, 1e-13, "separate k=E state %d" % e)
    _close(y, want, 1e-12, "separate k=E y")


def pin_separate_constant_top1_equals_mixed(lib):
    """k = 1 with constant routing: one expert only, both designs agree."""
    rng = np.random.default_rng(19)
    c = _rand_case(rng, B=2, L=9, D=3, N=4, E=3, k=1, h0=False)
    c["idx"][:] = 2
    c["gate"][:] = 1.0
    ym, hm = oracle.scan(**c, lib=lib)
    ys, hs = oracle.scan_separate(**c, lib=lib)
    _close(ys, ym, 1e-13, "const top-1 y")
    _close(hs[:, 2], hm, 1e-13, "const top-1 h")
    assert np.all(hs[:, :2] == 0.0), "unselected experts must stay at their initial state"


def pin_separate_block_resume(lib):
    """Routing e0 | e1 | e0 in blocks: in block 3 expert e0 resumes from the
    state it had at the end of block 1; e1's state is frozen meanwhile."""
    rng = np.random.default_rng(20)
    B, L, D, N, E = 1, 12, 2, 3, 2
    c = _rand_case(rng, B=B, L=L, D=D, N=N, E=E, k=1, h0=False)
    c["gate"][:] = 1.0
    c["idx"][:] = 0
    c["idx"][:, 4:8] = 1
    y, hf = oracle.scan_separate(**c, lib=lib)

    def sl(a, b):
        return {k_: (v[:, a:b] if k_ in ("x", "dt_raw", "Bm", "Cm") else v)
                for k_, v in c.items() if k_ not in ("idx", "gate", "h0")}

    def run(e, a, b, h0):
        s = sl(a, b)
        return oracle.mamba_scan(s["x"], s["dt_raw"], s["Bm"], s["Cm"], c["A"][e],
                                 c["dt_bias"][e], c["Dskip"][e], h0, lib=lib)

    y1, h1 = run(0, 0, 4, None)
    y2, h2 = run(1, 4, 8, None)
    y3, h3 = run(0, 8, 12, h1)
    _close(y, np.concatenate([y1, y2, y3], 1), 1e-13, "block resume y")
    _close(hf[:, 0], h3, 1e-13, "block resume h e0")
    _close(hf[:, 1], h2, 1e-13, "block resume h e1")


def pin_designs_differ_when_routing_varies(lib):
    """Theorem 4: with time-varying top-1 routing the separate design (one
    trajectory per expert) and the mixed design (one trajectory) differ."""
    rng = np.random.default_rng(21)
    c = _rand_case(rng, B=1, L=10, D=2, N=3, E=2, k=1, h0=False)
    c["gate"][:] = 1.0
    c["idx"][0, :, 0] = np.array([0, 1] * 5)
    ym, _ = oracle.scan(**c, lib=lib)
    ys, _ = oracle.scan_separate(**c, lib=lib)
    _close(ys[:, :1], ym[:, :1], 1e-13, "first token agrees")
    # from the second token on, the mixed trajectory carries expert 0's state
    # into expert 1's update, while expert 1's own trajectory starts at zero
    assert np.min(np.max(np.abs(ys[0, 1:] - ym[0, 1:]), axis=-1)) > 1e-6, "designs should differ"


# ----------------------------------------------------- per-slot trajectories
def _slot_as_top1(c, j):
    """The case routed by slot j alone, gate 1: the mixed scan's top-1 form."""
    return {**c, "idx": np.ascontiguousarray(c["idx"][:, :, j:j + 1]),
            "gate": np.ones(c["gate"].shape[:2] + (1,))}


def pin_slots_are_gated_top1_scans(lib):
    """Slot j's trajectory is the mixed scan routed by slot j alone with gate 1
    (mixing one expert with weight 1 gives that expert's A, dt_bias and Dskip,
    including across expert switches), and y adds the slots' outputs weighted
    by their gates; for both input terms and with an initial state."""
    rng = np.random.default_rng(23)
    B, L, D, N, E, k = 2, 9, 3, 4, 4, 3
    c = _rand_case(rng, B=B, L=L, D=D, N=N, E=E, k=k, h0=False)
    H0 = rng.standard_normal((B, k, D, N))
    for zoh in (False, True):
        y, hf = oracle.scan_slots(**{**c, "h0": H0}, lib=lib, zoh=zoh)
        want = np.zeros((B, L, D))
        for j in range(k):
            yj, hj = oracle.scan(**{**_slot_as_top1(c, j), "h0": H0[:, j]}, lib=lib, zoh=zoh)
            want += c["gate"][:, :, j:j + 1] * yj
            _close(hf[:, j], hj, 1e-13, "slot %d state (zoh=%d)" % (j, zoh))
        _close(y, want, 1e-12, "slots y (zoh=%d)" % zoh)


def pin_slots_state_carries_across_switch(lib):
    """Top-1 routing e0 | e1 | e0 in blocks: the one slot's state passes from
    each block to the next (unlike the per-expert trajectories, where e0
    resumes its own state in block 3) -- a chain of plain scans."""
    rng = np.random.default_rng(24)
    B, L, D, N, E = 1, 12, 2, 3, 2
    c = _rand_case(rng, B=B, L=L, D=D, N=N, E=E, k=1, h0=True)
    c["gate"][:] = 1.0
    c["idx"][:] = 0
    c["idx"][:, 4:8] = 1
    y, hf = oracle.scan_slots(**{**c, "h0": c["h0"][:, None]}, lib=lib)
    h = c["h0"]
    ys = []
    for e, a, b in ((0, 0, 4), (1, 4, 8), (0, 8, 12)):
        yb, h = oracle.mamba_scan(c["x"][:, a:b], c["dt_raw"][:, a:b], c["Bm"][:, a:b],
                                  c["Cm"][:, a:b], c["A"][e], c["dt_bias"][e], c["Dskip"][e], h,
                                  lib=lib)
        ys.append(yb)
    _close(y, np.concatenate(ys, 1), 1e-13, "slot switch y")
    _close(hf[:, 0], h, 1e-13, "slot switch h")


def pin_slots_gates_weight_outputs_only(lib):
    """The states do not depend on the gates: scaling every gate by 3 scales y
    by 3 and leaves h_final unchanged; a zero gate removes that slot from y
    while its state still advances."""
    rng = np.random.default_rng(25)
    c = _rand_case(rng, B=1, L=8, D=3, N=4, E=3, k=2, h0=False)
    y1, h1 = oracle.scan_slots(**c, lib=lib)
    y3, h3 = oracle.scan_slots(**{**c, "gate": 3.0 * c["gate"]}, lib=lib)
    _close(y3, 3.0 * y1, 1e-13, "gate scaling y")
    _close(h3, h1, 0.0, "gate scaling h")
    g0 = c["gate"].copy()
    g0[:, :, 1] = 0.0
    yz, hz = oracle.scan_slots(**{**c, "gate": g0}, lib=lib)
    y_one, _ = oracle.scan_slots(**{**c, "idx": c["idx"][:, :, :1].copy(),
                                    "gate": g0[:, :, :1].copy()}, lib=lib)
    _close(yz, y_one, 1e-13, "zero-gate slot drops out of y")
    _close(hz, h1, 0.0, "zero-gate slot still advances")
    assert np.max(np.abs(h1[:, 1])) > 1e-3


def pin_slots_constant_routing_equals_separate(lib):
    """Each slot keeps one expert for the whole sequence (distinct experts):
    slot j's trajectory is expert idx[j]'s own, so the two separate readings
    agree on y and on those experts' states."""
    rng = np.random.default_rng(26)
    c = _rand_case(rng, B=2, L=9, D=3, N=4, E=4, k=2, h0=False)
    c["idx"][:] = np.array([3, 1], np.int32)
    ys, hs = oracle.scan_slots(**c, lib=lib)
    ye, he = oracle.scan_separate(**c, lib=lib)
    _close(ys, ye, 1e-13, "constant routing y")
    _close(hs[:, 0], he[:, 3], 1e-13, "constant routing slot 0")
    _close(hs[:, 1], he[:, 1], 1e-13, "constant routing slot 1")


# ----------------------------------------------- every expert advances
def _plain_scans(c, H0, lib, zoh):
    """Each expert's plain selective scan over the whole sequence (the
    independently written ref_mamba_scan): outputs [B,L,D,E], states [B,E,D,N]."""
    E = c["A"].shape[0]
    ys, hs = [], []
    for e in range(E):
        ye, he = oracle.mamba_scan(c["x"], c["dt_raw"], c["Bm"], c["Cm"], c["A"][e],
                                   c["dt_bias"][e], c["Dskip"][e], H0[:, e], lib=lib, zoh=zoh)
        ys.append(ye)
        hs.append(he)
    return np.stack(ys, -1), np.stack(hs, 1)


def pin_all_experts_are_plain_scans(lib):
    """Every expert's trajectory is the plain scan with that expert's own
    parameters over all tokens, and y gathers the selected experts' outputs
    of those scans weighted by the gates (repeated experts add up); both
    input terms, with an initial state."""
    rng = np.random.default_rng(27)
    B, L, D, N, E, k = 2, 9, 3, 4, 4, 3
    c = _rand_case(rng, B=B, L=L, D=D, N=N, E=E, k=k, h0=False)
    c["idx"][0, 2] = np.array([1, 1, 3], np.int32)   # a repeated expert
    H0 = rng.standard_normal((B, E, D, N))
    for zoh in (False, True):
        y, hf = oracle.scan_all_experts(**{**c, "h0": H0}, lib=lib, zoh=zoh)
        ye, he = _plain_scans(c, H0, lib, zoh)
        want = np.zeros((B, L, D))
        for j in range(k):
            pick = np.take_along_axis(ye, c["idx"][:, :, None, j:j + 1].astype(np.int64), -1)[..., 0]
            want += c["gate"][:, :, j:j + 1] * pick
        _close(hf, he, 1e-13, "all-experts states (zoh=%d)" % zoh)
        _close(y, want, 1e-12, "all-experts y (zoh=%d)" % zoh)


def pin_all_experts_states_ignore_routing(lib):
    """The routing decides only which outputs are mixed: two unrelated
    routings give the same final states and different outputs."""
    rng = np.random.default_rng(28)
    c = _rand_case(rng, B=1, L=10, D=3, N=4, E=4, k=2, h0=False)
    y1, h1 = oracle.scan_all_experts(**c, lib=lib)
    c2 = _rand_case(np.random.default_rng(29), B=1, L=10, D=3, N=4, E=4, k=2, h0=False)
    y2, h2 = oracle.scan_all_experts(**{**c, "idx": c2["idx"], "gate": c2["gate"]}, lib=lib)
    _close(h2, h1, 0.0, "states independent of routing")
    assert np.max(np.abs(y2 - y1)) > 1e-3


def pin_all_experts_full_routing_equals_separate(lib):
    """With k = E and every expert selected at every token, the per-expert
    trajectories (advanced when selected) advance at every token too, so
    the two readings agree on y and on every state."""
    rng = np.random.default_rng(30)
    c = _rand_case(rng, B=2, L=8, D=3, N=4, E=3, k=3, h0=False)
    H0 = rng.standard_normal((2, 3, 3, 4))
    ya, ha = oracle.scan_all_experts(**{**c, "h0": H0}, lib=lib)
    ys, hs = oracle.scan_separate(**{**c, "h0": H0}, lib=lib)
    _close(ya, ys, 1e-12, "k = E y")
    _close(ha, hs, 1e-13, "k = E states")


# ------------------------------------------------------------------ router
def pin_route_bruteforce(lib):
    """Top-k equals a full sort by (-logit, index); gates are the softmax of
    the selected logits; k = E gives the full softmax."""
    rng = np.random.default_rng(22)
    T, D, E = 50, 16, 6
    x = rng.standard_normal((T, D))
    Wr = rng.standard_normal((D, E)) / 4
    Wr[:, 4] = Wr[:, 1]                     # exact ties between experts 1 and 4
    logits_np = x @ Wr
    for k in (1, 2, 3, E):
        idx, gate, logits, absdot = oracle.route(x, Wr, k, lib=lib)
        _close(logits, logits_np, 1e-13, "logits")
        _close(absdot, np.abs(x[:, :, None] * Wr[None]).sum(1), 1e-13, "absdot")
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-logits[t, e], e))
            assert list(idx[t]) == order[:k], (t, list(idx[t]), order[:k])
            sel = logits[t, order[:k]]
            w = np.exp(sel - sel.max())
            _close(gate[t], w / w.sum(), 1e-14, "gate")
        if k == 1:
            assert np.all(gate == 1.0)
        if k == E:
            full = np.exp(logits - logits.max(1, keepdims=True))
            full /= full.sum(1, keepdims=True)
            _close(np.take_along_axis(full, idx, 1), gate, 1e-14, "full softmax")


def pin_route_permutation(lib):
    """Permuting the experts (columns of Wr) permutes idx accordingly."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((30, 8))
    Wr = rng.standard_normal((8, 5))
    perm = rng.permutation(5)
    idx, gate, _, _ = oracle.route(x, Wr, 2, lib=lib)
    idx_p, gate_p, _, _ = oracle.route(x, Wr[:, perm], 2, lib=lib)
    assert np.array_equal(perm[idx_p], idx)
    _close(gate_p, gate, 1e-15, "perm gates")


# ------------------------------------------------------------------- step
def pin_step_equals_scan(lib):
    """Repeated decode steps on a carried state equal one scan over the same
    tokens; routed steps use the router on each step's x."""
    rng = np.random.default_rng(24)
    B, L, D, N, E, k = 2, 12, 4, 3, 4, 2
    c = _rand_case(rng, B=B, L=L, D=D, N=N, E=E, k=k)
    Wr = rng.standard_normal((D, E))
    T = B * L
    idx, gate, _, _ = oracle.route(c["x"].reshape(T, D), Wr, k, lib=lib)
    c["idx"] = idx.reshape(B, L, k)
    c["gate"] = gate.reshape(B, L, k)
    y, hf = oracle.scan(**c, lib=lib)
    state = np.ascontiguousarray(c["h0"].copy())
    for t in range(L):
        yt, it, gt = oracle.step(c["x"][:, t], c["dt_raw"][:, t], c["Bm"][:, t], c["Cm"][:, t],
                                 c["A"], c["dt_bias"], c["Dskip"], state, Wr=Wr, k=k, lib=lib)
        _close(yt, y[:, t], 1e-13, "step y t=%d" % t)
        assert np.array_equal(it, c["idx"][:, t])
        _close(gt, c["gate"][:, t], 1e-15, "step gate")
    _close(state, hf, 1e-13, "step state")
    # forced routing
    state = np.ascontiguousarray(c["h0"].copy())
    for t in range(L):
        yt, _, _ = oracle.step(c["x"][:, t], c["dt_raw"][:, t], c["Bm"][:, t], c["Cm"][:, t],
                               c["A"], c["dt_bias"], c["Dskip"], state, idx=c["idx"][:, t],
                               gate=c["gate"][:, t], lib=lib)
        _close(yt, y[:, t], 1e-13, "forced step y t=%d" % t)


# -------------------------------------------------- stream-mixed form
def _stream_case(rng, B=2, L=7, D=3, N=4, k=2, h0=True):
    X = rng.standard_normal((B, L, k, D))
    dt_raw = rng.standard_normal((B, L, D))
    Bs = rng.standard_normal((B, L, k, N))
    Cs = rng.standard_normal((B, L, k, N))
    g = rng.uniform(0.1, 1.0, (B, L, k))
    gate = g / g.sum(-1, keepdims=True)
    A = -np.exp(rng.uniform(0, math.log(16), (D, N)))
    dt_bias = rng.standard_normal(D) * 0.3
    H = rng.standard_normal((B, D, N)) if h0 else None
    return dict(X=X, dt_raw=dt_raw, Bs=Bs, Cs=Cs, gate=gate, A=A, dt_bias=dt_bias, h0=H)


def pin_worked_streams(lib):
    """Hand-derived stream-mixed examples: gates that change per token, a
    zero-weight slot, two channels with different step sizes, h0."""
    gold = json.load(open(GOLDEN))
    for c in gold["streams_cases"]:
        h0 = _arr(c["h0"]) if "h0" in c else None
        y, hf = oracle.scan_streams(_arr(c["X"]), _arr(c["dt_raw"]), _arr(c["Bs"]),
                                    _arr(c["Cs"]), _arr(c["gate"]), _arr(c["A"]),
                                    _arr(c["dt_bias"]), h0, lib=lib)
        _close(y, _frac(c["expected_y"]), 1e-12, c["name"] + " y")
        _close(hf, _frac(c["expected_h_final"]), 1e-12, c["name"] + " h_final")


def pin_streams_one_slot_is_mamba(lib):
    """One slot with weight 1: the stream form is the plain selective scan of
    that slot's streams (no feed-through term)."""
    rng = np.random.default_rng(30)
    c = _stream_case(rng, B=2, L=9, D=3, N=4, k=1)
    c["gate"][:] = 1.0
    y, hf = oracle.scan_streams(**c, lib=lib)
    ym, hm = oracle.mamba_scan(c["X"][:, :, 0], c["dt_raw"], c["Bs"][:, :, 0], c["Cs"][:, :, 0],
                               c["A"], c["dt_bias"], np.zeros(3), c["h0"], lib=lib)
    _close(y, ym, 1e-13, "one slot y")
    _close(hf, hm, 1e-13, "one slot h")


def pin_streams_identical_slots_is_mamba(lib):
    """Every slot carrying the same streams, convex gates: the mixture is that
    one stream, whatever the gates (Theorem 1: one selective SSM)."""
    rng = np.random.default_rng(31)
    c = _stream_case(rng, B=2, L=8, D=3, N=4, k=3)
    for key in ("X", "Bs", "Cs"):
        c[key][:, :, 1:] = c[key][:, :, :1]
    y, hf = oracle.scan_streams(**c, lib=lib)
    ym, hm = oracle.mamba_scan(c["X"][:, :, 0], c["dt_raw"], c["Bs"][:, :, 0], c["Cs"][:, :, 0],
                               c["A"], c["dt_bias"], np.zeros(3), c["h0"], lib=lib)
    _close(y, ym, 1e-12, "identical slots y")
    _close(hf, hm, 1e-12, "identical slots h")


def pin_streams_superposition(lib):
    """A is shared, so the transition does not depend on the slots and the
    state is linear in the injections: the k-slot state is the sum of the
    single-slot states (slot j alone with its own gate; h0 carried by one of
    them).  With one readout vector C in every slot, the k-slot readout is C
    (convex gates) and single-slot run j reads C / g_j, so y adds up too."""
    rng = np.random.default_rng(32)
    c = _stream_case(rng, B=2, L=10, D=3, N=4, k=3)
    c["Cs"][:, :, 1:] = c["Cs"][:, :, :1]
    y, hf = oracle.scan_streams(**c, lib=lib)
    ys, hs = np.zeros_like(y), np.zeros_like(hf)
    for j in range(3):
        g = c["gate"][:, :, j:j + 1]
        yj, hj = oracle.scan_streams(c["X"][:, :, j:j + 1], c["dt_raw"], c["Bs"][:, :, j:j + 1],
                                     c["Cs"][:, :, :1] / g[..., None], g, c["A"], c["dt_bias"],
                                     c["h0"] if j == 0 else np.zeros_like(c["h0"]), lib=lib)
        ys += yj
        hs += hj
    _close(hf, hs, 1e-12, "superposition h")
    _close(y, ys, 1e-12, "superposition y")


def pin_streams_readout_linear_in_C(lib):
    """For fixed injections the state does not depend on C, and y is linear
    in the C streams: the output equals the sum of the outputs with all but
    one slot's C zeroed."""
    rng = np.random.default_rng(33)
    c = _stream_case(rng, B=1, L=9, D=4, N=3, k=3)
    y, hf = oracle.scan_streams(**c, lib=lib)
    ys = np.zeros_like(y)
    for j in range(3):
        cj = dict(c)
        cj["Cs"] = np.zeros_like(c["Cs"])
        cj["Cs"][:, :, j] = c["Cs"][:, :, j]
        yj, hj = oracle.scan_streams(**cj, lib=lib)
        _close(hj, hf, 1e-14, "state independent of C")
        ys += yj
    _close(y, ys, 1e-12, "readout linear in C")


def pin_streams_zero_gate_slot(lib):
    """A slot with weight zero contributes nothing, whatever its streams."""
    rng = np.random.default_rng(34)
    c = _stream_case(rng, B=2, L=8, D=3, N=4, k=3)
    c["gate"][:, :, 1] = 0.0
    y, hf = oracle.scan_streams(**c, lib=lib)
    keep = [0, 2]
    y2, h2 = oracle.scan_streams(c["X"][:, :, keep], c["dt_raw"], c["Bs"][:, :, keep],
                                 c["Cs"][:, :, keep], c["gate"][:, :, keep], c["A"],
                                 c["dt_bias"], c["h0"], lib=lib)
    _close(y, y2, 1e-14, "zero-gate slot y")
    _close(hf, h2, 1e-14, "zero-gate slot h")


def pin_streams_slot_permutation(lib):
    """The mixture is a sum over slots: permuting the slots (streams and
    gates together) changes nothing."""
    rng = np.random.default_rng(35)
    c = _stream_case(rng, B=2, L=8, D=3, N=4, k=3)
    y, hf = oracle.scan_streams(**c, lib=lib)
    perm = [2, 0, 1]
    cp = dict(c)
    for key in ("X", "Bs", "Cs", "gate"):
        cp[key] = c[key][:, :, perm]
    yp, hp = oracle.scan_streams(**cp, lib=lib)
    _close(yp, y, 1e-13, "slot permutation y")
    _close(hp, hf, 1e-13, "slot permutation h")


def pin_streams_constant_geometric(lib):
    """Constant streams and gates: h_t = a^t h0 + u (1 - a^t) / (1 - a) with
    a = exp(Delta A) and u = Delta sum_j g_j B_j X_j; y_t = c . h_t."""
    B, L, D, N, k = 1, 30, 2, 3, 2
    Xv = np.array([[0.5, -2.0], [1.5, 0.25]])            # [k, D]
    Bv = np.array([[1.0, -0.5, 2.0], [0.25, 1.0, -1.0]])  # [k, N]
    Cv = np.array([[2.0, 0.0, -1.0], [-1.0, 3.0, 0.5]])
    g = np.array([0.3, 0.7])
    X = np.broadcast_to(Xv, (B, L, k, D)).copy()
    Bs = np.broadcast_to(Bv, (B, L, k, N)).copy()
    Cs = np.broadcast_to(Cv, (B, L, k, N)).copy()
    gate = np.broadcast_to(g, (B, L, k)).copy()
    dt_raw = np.broadcast_to(np.array([0.4, -1.1]), (B, L, D)).copy()
    A = -np.array([[1.0, 3.0, 0.5], [2.0, 0.25, 6.0]])
    dt_bias = np.array([-0.2, 0.3])
    h0 = np.array([[[1.0, -1.0, 0.5], [0.0, 2.0, -3.0]]])
    y, hf = oracle.scan_streams(X, dt_raw, Bs, Cs, gate, A, dt_bias, h0, lib=lib)
    t = np.arange(1, L + 1)[:, None]
    cvec = g[0] * Cv[0] + g[1] * Cv[1]
    for d in range(D):
        Dt = math.log1p(math.exp(dt_raw[0, 0, d] + dt_bias[d]))
        a = np.exp(Dt * A[d])
        u = Dt * (g[0] * Bv[0] * Xv[0, d] + g[1] * Bv[1] * Xv[1, d])
        h = a ** t * h0[0, d] + u * (1 - a ** t) / (1 - a)
        _close(y[0, :, d], h @ cvec, 1e-12, "stream geometric y d=%d" % d)
        _close(hf[0, d], h[-1], 1e-12, "stream geometric h d=%d" % d)


def pin_streams_stability_bound(lib):
    """Theorem 3 for the stream form: with a contractive shared transition and
    convex gates, |h_t[n]| <= a*^t |h0| + M (1 - a*^t) / (1 - a*), where a* is
    the largest decay and M bounds Delta |B_j[n] X_j[d]| over tokens and slots."""
    rng = np.random.default_rng(36)
    c = _stream_case(rng, B=1, L=40, D=3, N=4, k=3)
    L = 40
    Dt = _softplus(c["dt_raw"][0] + c["dt_bias"][None, :])       # [L, D]
    for t_end in (5, 17, 40):
        y, hf = oracle.scan_streams(c["X"][:, :t_end], c["dt_raw"][:, :t_end],
                                    c["Bs"][:, :t_end], c["Cs"][:, :t_end], c["gate"][:, :t_end],
                                    c["A"], c["dt_bias"], c["h0"], lib=lib)
        for d in range(3):
            amax = np.max(np.exp(Dt[:t_end, d][:, None] * c["A"][d][None, :]), axis=0)   # [N]
            M = np.max(Dt[:t_end, d][:, None, None] * np.abs(c["Bs"][0, :t_end])
                       * np.abs(c["X"][0, :t_end, :, d])[:, :, None], axis=(0, 1))      # [N]
            bound = amax ** t_end * np.abs(c["h0"][0, d]) + M * (1 - amax ** t_end) / (1 - amax)
            assert np.all(np.abs(hf[0, d]) <= bound * (1 + 1e-12)), ("bound", t_end, d)
            assert np.all(amax < 1.0)
    assert L == 40


def pin_streams_split_composition(lib):
    """scan(L1 || L2) = scan(L2, h0 = scan(L1).h_final), for y and h."""
    rng = np.random.default_rng(37)
    c = _stream_case(rng, B=2, L=11, D=3, N=4, k=2)
    y, hf = oracle.scan_streams(**c, lib=lib)
    keys = ("X", "dt_raw", "Bs", "Cs", "gate")
    c1 = dict(c, **{k_: c[k_][:, :4] for k_ in keys})
    c2 = dict(c, **{k_: c[k_][:, 4:] for k_ in keys})
    y1, h1 = oracle.scan_streams(**c1, lib=lib)
    c2["h0"] = h1
    y2, h2 = oracle.scan_streams(**c2, lib=lib)
    _close(np.concatenate([y1, y2], axis=1), y, 1e-13, "stream split y")
    _close(h2, hf, 1e-13, "stream split h")


# --------------------------------------------------------- zero-order hold
def _softplus_inv(v):
    return math.log(math.expm1(v))


def pin_zoh_equilibrium(lib):
    """With constant inputs the zero-order-hold recurrence has the fixed point
    of the continuous system, h* = -B x / Abar, whatever the step size:
    h_t = a^t h0 + (1 - a^t) h* exactly (Euler's fixed point is
    Delta B x / (1 - a) instead)."""
    B, L, D, N, E, k = 1, 30, 2, 3, 3, 2
    x = np.broadcast_to(np.array([0.8, -1.6]), (B, L, D)).copy()
    dt_raw = np.broadcast_to(np.array([0.5, -0.7]), (B, L, D)).copy()
    Bv, Cv = np.array([1.0, -0.5, 2.0]), np.array([0.5, 1.5, -1.0])
    Bm = np.broadcast_to(Bv, (B, L, N)).copy()
    Cm = np.broadcast_to(Cv, (B, L, N)).copy()
    A = -np.array([[[0.5, 2.0, 8.0], [1.0, 3.0, 0.25]],
                   [[4.0, 1.0, 0.5], [2.0, 0.75, 6.0]],
                   [[1.5, 1.5, 1.5], [0.5, 0.5, 0.5]]])
    dt_bias = np.array([[0.1, -0.2], [0.0, 0.3], [-0.3, 0.1]])
    Dskip = np.array([[0.5, 1.0], [-1.0, 0.0], [2.0, -0.5]])
    g = np.array([0.65, 0.35])
    idx = np.broadcast_to(np.array([1, 2], np.int32), (B, L, k)).copy()
    gate = np.broadcast_to(g, (B, L, k)).copy()
    h0 = np.array([[[1.0, -2.0, 0.5], [0.0, 1.0, -1.0]]])
    y, hf = oracle.scan(x, dt_raw, Bm, Cm, idx, gate, A, dt_bias, Dskip, h0, lib=lib, zoh=True)
    t = np.arange(1, L + 1)[:, None]
    for d in range(D):
        beta = g[0] * dt_bias[1, d] + g[1] * dt_bias[2, d]
        delta = g[0] * Dskip[1, d] + g[1] * Dskip[2, d]
        Dt = math.log1p(math.exp(dt_raw[0, 0, d] + beta))
        Abar = g[0] * A[1, d] + g[1] * A[2, d]
        a = np.exp(Dt * Abar)
        hstar = -Bv * x[0, 0, d] / Abar
        h = a ** t * h0[0, d] + (1 - a ** t) * hstar
        _close(y[0, :, d], h @ Cv + delta * x[0, 0, d], 1e-12, "zoh equilibrium y d=%d" % d)
        _close(hf[0, d], h[-1], 1e-12, "zoh equilibrium h d=%d" % d)


def pin_zoh_semigroup(lib):
    """Zero-order hold is exact for an input held constant: two steps of
    Delta with the same B, x and routing equal one step of 2 Delta (Euler
    does not compose so)."""
    rng = np.random.default_rng(42)
    c = _rand_case(rng, B=1, L=2, D=3, N=4, E=2, k=2)
    for key in ("x", "Bm", "Cm"):
        c[key][:, 1] = c[key][:, 0]
    c["idx"][:, 1] = c["idx"][:, 0]
    c["gate"][:, 1] = c["gate"][:, 0]
    c["dt_raw"][:, 1] = c["dt_raw"][:, 0]
    _, h2 = oracle.scan(**c, lib=lib, zoh=True)
    one = {k_: (v[:, :1].copy() if k_ in ("x", "dt_raw", "Bm", "Cm", "idx", "gate") else v)
           for k_, v in c.items()}
    idx0, g0 = c["idx"][0, 0], c["gate"][0, 0]
    for d in range(3):
        beta = g0[0] * c["dt_bias"][idx0[0], d] + g0[1] * c["dt_bias"][idx0[1], d]
        Dt = math.log1p(math.exp(c["dt_raw"][0, 0, d] + beta))
        one["dt_raw"][0, 0, d] = _softplus_inv(2 * Dt) - beta
    _, h1 = oracle.scan(**one, lib=lib, zoh=True)
    _close(h1, h2, 1e-12, "zoh semigroup")


def pin_zoh_small_transition_is_euler(lib):
    """As A -> 0 the zero-order-hold coefficient (exp(Delta A) - 1)/A tends
    to Delta: with |A| ~ 1e-9 the two discretisations agree to ~1e-9."""
    rng = np.random.default_rng(43)
    c = _rand_case(rng, B=2, L=9, D=3, N=4, E=3, k=2)
    c["A"] = c["A"] * 1e-9
    yz, hz = oracle.scan(**c, lib=lib, zoh=True)
    ye, he = oracle.scan(**c, lib=lib)
    _close(yz, ye, 1e-7, "zoh small A y")
    _close(hz, he, 1e-7, "zoh small A h")


# ------------------------------------------------------------- backward
def pin_backward_finite_differences(lib):
    """Every gradient of the mixed scan against central differences of the
    forward oracle, for L = sum(dy * y) + sum(dh_final * h_final): an
    independent derivative of the pinned forward (step 1e-6 in fp64, error
    ~1e-10 relative)."""
    rng = np.random.default_rng(40)
    c = _rand_case(rng, B=2, L=6, D=3, N=4, E=3, k=2)
    dy = rng.standard_normal(c["x"].shape)
    dhf = rng.standard_normal(c["h0"].shape)
    g = oracle.scan_backward(**c, dy=dy, dh_final=dhf, lib=lib)

    def loss(**kw):
        a = dict(c)
        a.update(kw)
        y, hf = oracle.scan(**a, lib=lib)
        return float(np.sum(y * dy) + np.sum(hf * dhf))

    eps = 1e-6
    for name, key in (("x", "dx"), ("dt_raw", "ddt_raw"), ("Bm", "dBm"), ("Cm", "dCm"),
                      ("gate", "dgate"), ("A", "dA"), ("dt_bias", "dbias"), ("Dskip", "dDskip"),
                      ("h0", "dh0")):
        arr = c[name]
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[i] += eps
            m[i] -= eps
            fd[i] = (loss(**{name: p}) - loss(**{name: m})) / (2 * eps)
        _close(g[key], fd, 1e-7, "backward d%s" % name)


def pin_backward_without_final_gradient(lib):
    """dh_final = 0 (None) and dy = 0 except one token: the adjoint starts at
    that token, so every gradient of later tokens is zero, dC is nonzero only
    there, and dh0 equals the finite difference of that single output."""
    rng = np.random.default_rng(41)
    c = _rand_case(rng, B=1, L=8, D=2, N=3, E=3, k=2)
    dy = np.zeros(c["x"].shape)
    dy[0, 4] = rng.standard_normal(2)
    g = oracle.scan_backward(**c, dy=dy, lib=lib)
    assert np.all(g["dx"][0, 5:] == 0) and np.all(g["ddt_raw"][0, 5:] == 0)
    assert np.all(g["dCm"][0, :4] == 0) and np.all(g["dCm"][0, 5:] == 0)
    assert np.all(g["dBm"][0, 5:] == 0) and np.all(g["dgate"][0, 5:] == 0)
    eps = 1e-6
    fd = np.zeros_like(c["h0"])
    for i in np.ndindex(c["h0"].shape):
        p, m = c["h0"].copy(), c["h0"].copy()
        p[i] += eps
        m[i] -= eps
        yp, _ = oracle.scan(**dict(c, h0=p), lib=lib)
        ym, _ = oracle.scan(**dict(c, h0=m), lib=lib)
        fd[i] = np.sum((yp - ym) * dy) / (2 * eps)
    _close(g["dh0"], fd, 1e-7, "dh0 single token")


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
