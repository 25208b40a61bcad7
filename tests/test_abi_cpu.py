"""The C ABI on the CPU: the library loads, exports what include/swimba.h
declares, the ctypes mirrors match the C structs, and invalid arguments are
rejected before anything is launched (no GPU work is started here)."""
import ctypes
import os
import re
import subprocess

import pytest

from parameter_space_moe_amd import swimba as sw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swimba.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swimba_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sw.load()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert {"swimba_route", "swimba_scan", "swimba_scan_separate", "swimba_scan_slots",
            "swimba_step",
            "swimba_scan_workspace_size", "swimba_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_exports_nothing_but_the_abi():
    out = subprocess.run(["nm", "-D", "--defined-only", sw.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    ours = {n for n in exported if n.startswith("swimba_")}
    assert ours == set(header_functions())


STRUCTS = (("swimba_scan_args", sw.ScanArgs), ("swimba_step_args", sw.StepArgs),
           ("swimba_stream_args", sw.StreamArgs), ("swimba_scan_grad_args", sw.GradArgs))

LAYOUT_SRC = r"""
#include <cstddef>
#include <cstdio>
#include "swimba.h"
#define F(S, m) std::printf(#S " " #m " %zu\n", offsetof(S, m));
int main() {
  std::printf("swimba_scan_args sizeof %zu\n", sizeof(swimba_scan_args));
  std::printf("swimba_step_args sizeof %zu\n", sizeof(swimba_step_args));
  std::printf("swimba_stream_args sizeof %zu\n", sizeof(swimba_stream_args));
  std::printf("swimba_scan_grad_args sizeof %zu\n", sizeof(swimba_scan_grad_args));
  %FIELDS%
  return 0;
}
"""


def test_ctypes_structs_match_header(tmp_path):
    lines = []
    for cname, cls in STRUCTS:
        for f, _ in cls._fields_:
            lines.append("F(%s, %s)" % (cname, f))
    src = tmp_path / "layout.cpp"
    src.write_text(LAYOUT_SRC.replace("%FIELDS%", "\n  ".join(lines)))
    exe = tmp_path / "layout"
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {}
    for l in out.splitlines():
        s, m, v = l.split()
        got[(s, m)] = int(v)
    for cname, cls in STRUCTS:
        assert got[(cname, "sizeof")] == ctypes.sizeof(cls), cname
    for cname, cls in STRUCTS:
        for f, _ in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


def scan_args(**kw):
    a = sw.ScanArgs()
    a.B, a.L, a.D, a.N, a.E, a.k = 1, 1024, 128, 16, 4, 2
    a.in_dtype, a.y_dtype = sw.BF16, sw.BF16
    fake = 0x100000  # never dereferenced: every call below fails validation first
    for f in ("x", "dt_raw", "Bm", "Cm", "idx", "gate", "A", "dt_bias", "Dskip", "y"):
        setattr(a, f, fake)
    a.chunk = 0
    a.carry = 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, sw.EINVAL), ("k", 5, sw.EINVAL), ("E", 0, sw.EINVAL), ("D", 0, sw.EINVAL),
    ("B", -1, sw.EINVAL), ("L", -1, sw.EINVAL), ("chunk", -1, sw.EINVAL), ("carry", 7, sw.EINVAL),
    ("in_dtype", 5, sw.EINVAL), ("N", 8, sw.EUNSUPPORTED), ("E", 65, sw.EUNSUPPORTED),
    ("x", None, sw.EINVAL), ("A", None, sw.EINVAL),
    ("idx", None, sw.EINVAL), ("a_form", 2, sw.EINVAL), ("disc", 2, sw.EINVAL),
])
def test_scan_rejects(lib, field, value, status):
    a = scan_args(**{field: value})
    assert lib.swimba_scan(ctypes.byref(a), None, 0, None) == status


def test_separate_designs_take_up_to_64_experts(lib):
    # one wave per expert up to 16, then 16 waves of 2 or 4 experts each;
    # valid: the call gets as far as the (missing) workspace
    for E in (17, 32, 33, 64):
        for design, fn in ((sw.DESIGN_SEPARATE, lib.swimba_scan_separate),
                           (sw.DESIGN_ALL_EXPERTS, lib.swimba_scan_all_experts)):
            a = scan_args(E=E)
            assert sw.workspace_size(a, design) > 0
            assert fn(ctypes.byref(a), None, 0, None) == sw.EWORKSPACE
    a = scan_args(E=65, k=2)
    assert lib.swimba_scan_separate(ctypes.byref(a), None, 0, None) == sw.EUNSUPPORTED


def test_mixed_scan_takes_up_to_64_experts(lib):
    # valid: the call gets as far as the (missing) workspace
    for E in (17, 32, 64):
        a = scan_args(E=E)
        assert sw.workspace_size(a, sw.DESIGN_MIXED) > 0
        assert lib.swimba_scan(ctypes.byref(a), None, 0, None) == sw.EWORKSPACE
    # expert rows beyond 32-bit buffer offsets
    a = scan_args(E=64, D=1 << 19)
    assert lib.swimba_scan(ctypes.byref(a), None, 0, None) == sw.EUNSUPPORTED


def test_slots_rejects_and_workspace(lib):
    # k slot states per lane live in registers: k <= 4
    a = scan_args(E=8, k=5)
    assert lib.swimba_scan_slots(ctypes.byref(a), None, 0, None) == sw.EUNSUPPORTED
    # more than 16 experts: rows from memory, k <= 2 (and a per-tile A check
    # in the workspace)
    assert lib.swimba_scan_slots(ctypes.byref(scan_args(E=17, k=3)), None, 0, None) == \
        sw.EUNSUPPORTED
    for E in (17, 64):
        a = scan_args(E=E, k=2)
        assert lib.swimba_scan_slots(ctypes.byref(a), None, 0, None) == sw.EWORKSPACE
    a = scan_args(B=2, L=4096, D=256, E=24, k=2, chunk=512)
    arr = 2 * 8 * 2 * 16 * 256 * 4
    flags = 2 * 8 * 4 * 4
    assert lib.swimba_scan_workspace_size(ctypes.byref(a), sw.DESIGN_SLOTS) == \
        2 * arr + flags + 256
    assert lib.swimba_scan_slots(ctypes.byref(scan_args(x=None)), None, 0, None) == sw.EINVAL
    # workspace: k x 16 state rows per (sequence, chunk, channel), plus flags
    a = scan_args(B=2, L=4096, D=256, E=8, k=3, chunk=512)
    arr = 2 * 8 * 3 * 16 * 256 * 4
    flags = 2 * 8 * 4 * 4
    assert lib.swimba_scan_workspace_size(ctypes.byref(a), sw.DESIGN_SLOTS) == 2 * arr + flags
    assert lib.swimba_scan_slots(ctypes.byref(a), None, 0, None) == sw.EWORKSPACE
    # an unknown design
    assert lib.swimba_scan_workspace_size(ctypes.byref(a), 4) == 0
    c, n = ctypes.c_int(), ctypes.c_int()
    assert lib.swimba_scan_plan(ctypes.byref(a), 4, ctypes.byref(c), ctypes.byref(n)) == \
        sw.EINVAL
    assert lib.swimba_scan_plan(ctypes.byref(a), sw.DESIGN_SLOTS, ctypes.byref(c),
                                ctypes.byref(n)) == sw.OK
    assert (c.value, n.value) == (512, 8)


def test_separate_plan_single_pass_when_tiles_fill_the_gpu(lib):
    # (sequence, tile) workgroups of one wave per expert: 20 / E per compute
    # unit up to 4 experts (at most ten), two up to 10 experts, one beyond
    # (256 CUs when no device answers); the
    # separate design runs each sequence in one chunk when they fill those
    # slots, else in as many long chunks as fill them once
    c, n = ctypes.c_int(), ctypes.c_int()
    a = scan_args(B=8, L=4096, D=4096, E=8, k=2)
    assert lib.swimba_scan_plan(ctypes.byref(a), sw.DESIGN_SEPARATE, ctypes.byref(c),
                                ctypes.byref(n)) == sw.OK
    assert (c.value, n.value) == (4096, 1)
    assert lib.swimba_scan_workspace_size(ctypes.byref(a), sw.DESIGN_SEPARATE) == 0
    a = scan_args(B=4, L=2048, D=1536, E=8, k=2)
    assert lib.swimba_scan_plan(ctypes.byref(a), sw.DESIGN_SEPARATE, ctypes.byref(c),
                                ctypes.byref(n)) == sw.OK
    assert n.value > 1 and c.value % 64 == 0
    assert (c.value, n.value) == (448, 5)  # 96 workgroups per chunk, 512 slots
    a = scan_args(B=1, L=65536, D=2560, E=16, k=2)
    assert lib.swimba_scan_plan(ctypes.byref(a), sw.DESIGN_SEPARATE, ctypes.byref(c),
                                ctypes.byref(n)) == sw.OK
    assert (c.value, n.value) == (10944, 6)  # 40 workgroups per chunk, 256 slots
    # two experts: 16-token rounds, ten 2-wave workgroups per CU
    a = scan_args(B=8, L=4096, D=4096, E=2, k=2)
    assert lib.swimba_scan_plan(ctypes.byref(a), sw.DESIGN_SEPARATE, ctypes.byref(c),
                                ctypes.byref(n)) == sw.OK
    assert (c.value, n.value) == (832, 5)  # 512 workgroups per chunk, 2560 slots


def test_all_experts_rejects_and_workspace(lib):
    # up to 64 experts, as the per-expert design
    assert lib.swimba_scan_all_experts(ctypes.byref(scan_args(E=65)), None, 0, None) == \
        sw.EUNSUPPORTED
    assert lib.swimba_scan_all_experts(ctypes.byref(scan_args(x=None)), None, 0, None) == \
        sw.EINVAL
    # the same E x 16 state rows per (sequence, chunk, channel) as the
    # per-expert design
    a = scan_args(B=2, L=4096, D=256, E=8, k=3, chunk=512)
    arr = 2 * 8 * 8 * 16 * 256 * 4
    flags = 2 * 8 * 4 * 4
    need = lib.swimba_scan_workspace_size(ctypes.byref(a), sw.DESIGN_ALL_EXPERTS)
    assert need == lib.swimba_scan_workspace_size(ctypes.byref(a), sw.DESIGN_SEPARATE)
    assert need == 2 * arr + 256 * ((flags + 255) // 256)
    assert lib.swimba_scan_all_experts(ctypes.byref(a), None, 0, None) == sw.EWORKSPACE


def test_workspace_checked_before_launch(lib):
    a = scan_args(chunk=256)
    need = lib.swimba_scan_workspace_size(ctypes.byref(a), 0)
    assert need > 0
    assert lib.swimba_scan(ctypes.byref(a), None, 0, None) == sw.EWORKSPACE
    assert lib.swimba_scan(ctypes.byref(a), 0x100000, need - 1, None) == sw.EWORKSPACE
    assert lib.swimba_scan(ctypes.byref(a), 0x100010, need, None) == sw.EWORKSPACE  # unaligned


def test_workspace_size_layout(lib):
    # long-context workload with chunk 256: 256 chunks x 16 states x 2560 channels, two
    # fp32 arrays (decays, states) and one int32 flag per (chunk, 64-channel tile)
    a = scan_args(B=1, L=65536, D=2560, E=16, k=2, chunk=256)
    arr = 256 * 16 * 2560 * 4
    flags = 256 * 40 * 4
    assert lib.swimba_scan_workspace_size(ctypes.byref(a), 0) == 2 * arr + flags
    sep = 256 * 16 * 16 * 2560 * 4
    assert lib.swimba_scan_workspace_size(ctypes.byref(a), 1) == 2 * sep + flags
    # one chunk: no workspace
    a = scan_args(L=100, chunk=100)
    assert lib.swimba_scan_workspace_size(ctypes.byref(a), 0) == 0
    # the query reads sizes only
    a = scan_args(chunk=256, x=None, A=None)
    assert lib.swimba_scan_workspace_size(ctypes.byref(a), 0) > 0


def test_route_and_step_reject(lib):
    assert lib.swimba_route(0x100000, sw.BF16, 0x100000, 10, 64, 4, 5, 0x100000, 0x100000,
                            None) == sw.EINVAL
    assert lib.swimba_route(0x100000, sw.BF16, 0x100000, 10, 64, 65, 2, 0x100000, 0x100000,
                            None) == sw.EUNSUPPORTED
    assert lib.swimba_route(None, sw.BF16, None, 0, 64, 4, 2, None, None, None) == sw.OK  # T = 0
    s = sw.StepArgs()
    s.B, s.D, s.N, s.E, s.k = 4, 128, 16, 8, 2
    s.in_dtype = s.y_dtype = sw.BF16
    for f in ("x", "dt_raw", "Bm", "Cm", "A", "dt_bias", "Dskip", "state", "y"):
        setattr(s, f, 0x100000)
    assert lib.swimba_step(ctypes.byref(s), None) == sw.EINVAL          # neither Wr nor idx
    s.Wr = 0x100000
    s.state = 0x100004
    assert lib.swimba_step(ctypes.byref(s), None) == sw.EINVAL          # unaligned state
    s.N = 8
    assert lib.swimba_step(ctypes.byref(s), None) == sw.EUNSUPPORTED


def test_status_strings(lib):
    for st in (sw.OK, sw.EINVAL, sw.EUNSUPPORTED, sw.EWORKSPACE, sw.EHIP, 123):
        assert isinstance(sw.status_string(st), str) and sw.status_string(st)


def stream_args(**kw):
    a = sw.StreamArgs()
    a.B, a.L, a.D, a.N, a.k = 1, 1024, 128, 16, 2
    a.in_dtype, a.y_dtype = sw.BF16, sw.BF16
    fake = 0x100000  # never dereferenced: every call below fails validation first
    for f in ("X", "dt_raw", "Bs", "Cs", "gate", "A", "dt_bias", "y"):
        setattr(a, f, fake)
    a.chunk = 0
    a.carry = 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, sw.EINVAL), ("k", 5, sw.EUNSUPPORTED), ("D", 0, sw.EINVAL), ("B", -1, sw.EINVAL),
    ("L", -1, sw.EINVAL), ("chunk", -1, sw.EINVAL), ("carry", 7, sw.EINVAL),
    ("in_dtype", 5, sw.EINVAL), ("N", 8, sw.EUNSUPPORTED), ("X", None, sw.EINVAL),
    ("A", None, sw.EINVAL), ("gate", None, sw.EINVAL), ("A", 0x100004, sw.EINVAL),
    ("Bs", 0x100002, sw.EINVAL),
])
def test_streams_rejects(lib, field, value, status):
    a = stream_args(**{field: value})
    assert lib.swimba_scan_streams(ctypes.byref(a), None, 0, None) == status


def test_streams_workspace_and_plan(lib):
    # 65536 tokens in chunks of 256: decays and states, no flag array
    a = stream_args(B=1, L=65536, D=2560, chunk=256)
    assert lib.swimba_scan_streams_workspace_size(ctypes.byref(a)) == 2 * 256 * 16 * 2560 * 4
    assert lib.swimba_scan_streams(ctypes.byref(a), None, 0, None) == sw.EWORKSPACE
    c, n = ctypes.c_int(), ctypes.c_int()
    assert lib.swimba_scan_streams_plan(ctypes.byref(a), ctypes.byref(c), ctypes.byref(n)) == 0
    assert (c.value, n.value) == (256, 256)
    a = stream_args(L=100, chunk=100)
    assert lib.swimba_scan_streams_workspace_size(ctypes.byref(a)) == 0
    a = stream_args(k=9)
    assert lib.swimba_scan_streams_workspace_size(ctypes.byref(a)) == 0


def grad_args(**kw):
    g = sw.GradArgs()
    g.fwd = scan_args(B=2, L=1000, D=256, E=8, k=2)
    fake = 0x100000
    for f in ("dy", "dx", "ddt_raw", "dBm", "dCm", "dgate", "dA", "ddt_bias", "dDskip"):
        setattr(g, f, fake)
    g.dy_dtype = sw.BF16
    for k, v in kw.items():
        setattr(g, k, v)
    return g


def test_backward_rejects_and_workspace(lib):
    g = grad_args()
    need = lib.swimba_scan_backward_workspace_size(ctypes.byref(g))
    # no state is kept per token: the block checkpoints (local state and decay
    # product every 8 tokens, 16 B per token-channel) and the per-chunk dA
    # partials (E x 64 B per chunk and channel) dominate, under half of the
    # 64 B per token-channel that every state would take
    tc = 2 * 1000 * 256
    assert 12 * tc <= need < 32 * tc
    assert lib.swimba_scan_backward(ctypes.byref(g), None, 0, None) == sw.EWORKSPACE
    for field, value, status in (("dy", None, sw.EINVAL), ("dA", None, sw.EINVAL),
                                 ("dy_dtype", 7, sw.EINVAL)):
        assert lib.swimba_scan_backward(ctypes.byref(grad_args(**{field: value})), None, 0,
                                        None) == status
    g = grad_args()
    g.fwd.a_form = 1
    assert lib.swimba_scan_backward(ctypes.byref(g), None, 0, None) == sw.EUNSUPPORTED
    g = grad_args()
    g.fwd.disc = 1
    assert lib.swimba_scan_backward(ctypes.byref(g), None, 0, None) == sw.EUNSUPPORTED
    for E in (17,):
        g = grad_args()
        g.fwd.E = E
        assert lib.swimba_scan_backward(ctypes.byref(g), None, 0, None) == sw.EUNSUPPORTED
