"""Build the in-tree HIP library ``libnvfp4.so`` for gfx950 with hipcc.

Usage: ``python -m block_scale_search_amd.build`` (``__graft_entry__.build()`` calls the same).
The library links against the HIP runtime that PyTorch itself loads, so that streams and
device pointers handed over from torch belong to the same runtime instance.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # binary32 expressions stay one IEEE operation each (fmas are written explicitly)
    "-ffp-contract=off",
    # no packed-FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _torch_hip_dir() -> str | None:
    try:
        import torch  # noqa: F401
    except Exception:
        return None
    d = os.path.join(os.path.dirname(__import__("torch").__file__), "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def _run(cmd: list[str], verbose: bool) -> list[str]:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    return msgs


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel, into a fresh private folder), then link
    the shared library. Every call compiles everything."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    hipcc = _hipcc()
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    with tempfile.TemporaryDirectory(dir=os.path.join(HERE, "_build")) as objdir:
        objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in srcs]
        jobs = max(1, min(len(srcs), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            msgs = list(pool.map(lambda so: _run([hipcc, *compile_flags, "-c", so[0], "-o", so[1]],
                                                 verbose), zip(srcs, objs)))
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
        tdir = _torch_hip_dir()
        if tdir:
            cmd += [f"-L{tdir}", f"-Wl,-rpath,{tdir}"]
        msgs.append(_run(cmd, verbose))
    if verbose:
        for m in msgs:
            if m:
                print("\n".join(m))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
