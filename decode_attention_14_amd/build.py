"""Build the C-ABI library ``libfd.so`` for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfd.so")
SOURCES = ["fd_api.cpp", "fd_select.cpp", "fd_decode.hip", "fd_mfma.hip", "fd_chunk.hip", "fd_scratch.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are disabled for every HIP translation unit.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: the kernels rescale them with
    # vector ops, which cannot read accumulation registers directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source into ``libfd.so`` (or ``out``); return its path.

    Each source is compiled to an object of its own (in parallel, under
    ``_build/``), then the objects are linked.  ``defines``: extra
    ``NAME=VALUE`` macros (the kernel's tuning constants).
    """
    from concurrent.futures import ThreadPoolExecutor

    tag = os.path.splitext(os.path.basename(out))[0]
    objdir = os.path.join(PKG, "_build", tag)
    os.makedirs(objdir, exist_ok=True)
    common = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[*common, "-c", "-x", "hip", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    for c in cmds:
        c.remove("-shared")
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


# The workgroup-timeline diagnostic build of the library (see timeline.py):
# the same sources with FD_WG_TIMELINE=1.
TIMELINE_LIB = os.path.join(PKG, "libfd_timeline.so")


def build_timeline(verbose: bool = False) -> str:
    return build(verbose=verbose, out=TIMELINE_LIB, defines=("FD_WG_TIMELINE=1",))


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_timeline(verbose=True))
