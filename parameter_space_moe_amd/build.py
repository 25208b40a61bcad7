"""Build libswimba.so (all HIP sources, gfx950) in-tree with hipcc.

Each source compiles to an object in parallel; the objects link into
parameter_space_moe_amd/libswimba.so."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libswimba.so")
OBJDIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 (v_pk_*_f32) instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source flags (none at present).
PER_SOURCE: dict[str, list[str]] = {}
# the host pass does not know the device-only feature name: drop that warning
_NOISE = "is not a recognized feature for this target"


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l]
    return res.returncode, "\n".join(msgs)


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False,
          jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    tag = "%d" % os.getpid()
    cmds = []
    objs = []
    for src in sources():
        obj = os.path.join(OBJDIR, os.path.basename(src) + "." + tag + ".o")
        objs.append(obj)
        per = PER_SOURCE.get(os.path.basename(src), [])
        cmds.append([HIPCC] + FLAGS + per + (extra or []) + inc + ["-c", src, "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 8)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, msg) in zip(cmds, results):
        if rc != 0 or (verbose and msg):
            sys.stderr.write(msg + "\n")
        failed |= rc != 0
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = out + ".tmp" + tag
    rc, msg = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    for o in objs:
        os.remove(o)
    if rc != 0:
        sys.stderr.write(msg + "\n")
        raise RuntimeError("link failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
