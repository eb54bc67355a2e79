"""Build libmuir.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m gated_delta_rule_06_amd._build``. The library lands in this package
directory; the public header is ``include/muir.h`` at the repository root.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmuir.so")
SOURCES = ["api.cpp", "sizes.cpp", "decode.hip", "chunk_fwd.hip", "chunk_bwd.hip", "wy_fwd.hip", "gates_fwd.hip",
           "noalloc.hip", "chunk_scan_split.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of every kernel. MFMA accumulators are kept
# in ordinary VGPRs: the scan updates its fp32 state accumulators with vector
# instructions between matrix-core products, and in AGPRs every such update costs a copy
# out and back.
HIP_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmuir")
    return exe


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    return res.returncode, err


def build(verbose: bool = False, extra_flags=(), jobs: int | None = None) -> str:
    """Compile every source into ``libmuir.so`` (always recompiles); returns its path.

    Each source is compiled to an object of its own, in parallel, then linked."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}", *HIP_FLAGS, *extra_flags]
    cmds, objs = [], []
    for s in SOURCES:
        obj = os.path.join(objdir, s + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *flags, "-c", "-o", obj, os.path.join(CSRC, s)])
    t0 = time.time()
    if verbose:
        for c in cmds:
            print(" ".join(c), file=sys.stderr)
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), c in zip(results, cmds):
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) on {c[-1]}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
