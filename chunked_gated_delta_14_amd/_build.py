"""Build of libgdr.so (gfx950) with hipcc, in-tree next to this file."""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libgdr.so")
SOURCES = ["gdr_api.cpp", "gdr_fwd.hip", "gdr_bwd.hip"]
HEADERS = ["gdr_device.h", "gdr_kernels.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source device code-generation options.  The adjoint-walk and gradient
# source keeps MFMA accumulators in ordinary VGPRs (no accumulator-register
# moves around the VALU work on them); the forward source leaves the choice to
# the compiler, whose accumulator registers relieve the forward walks' pressure.
EXTRA = {"gdr_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def commands(out: str = LIB_PATH, objdir: str | None = None) -> list[list[str]]:
    """hipcc -c for every source, then the link into the shared library."""
    objdir = objdir or os.path.dirname(out)
    objs, cmds = [], []
    common = [f for f in FLAGS if f != "-shared"]
    for src in SOURCES:
        obj = os.path.join(objdir, "%s.%d.o" % (src, os.getpid()))
        cmds.append([HIPCC, *common, *EXTRA.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    cmds.append([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out])
    return cmds


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libgdr.so (always recompiles)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmds = commands(tmp, PKG_DIR)
    try:
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed building libgdr.so")
        os.replace(tmp, LIB_PATH)
    finally:
        for obj in cmds[-1][4:-2]:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB_PATH


PROBE_SRC = "gdr_probe.hip"
PROBE_PATH = os.path.join(PKG_DIR, "libgdr_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The peak probes used by bench.py (a library of their own, outside libgdr's ABI)."""
    tmp = PROBE_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, os.path.join(CSRC, PROBE_SRC), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgdr_probe.so")
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


def stale() -> bool:
    """True when libgdr.so is missing or older than any of its sources."""
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    deps = [os.path.join(CSRC, s) for s in SOURCES + HEADERS] + [os.path.join(INCLUDE, "gdr.h")]
    return any(os.path.getmtime(d) > t for d in deps if os.path.exists(d))


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
