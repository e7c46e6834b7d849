"""Build libbd.so (the HIP library behind include/bd.h) in-tree for gfx950.

Usage: ``python -m block_diffusion_lm_amd.build`` (or ``build()`` from Python). Always compiles;
the result is ``block_diffusion_lm_amd/libbd.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libbd.so")

SOURCES = ["bd_api.cpp", "bd_attn.hip", "bd_unmask.hip", "bd_cache.hip", "bd_halt.hip", "bd_mamba.hip"]

# Packed fp32 vector instructions are disabled for every device compile (they are generated
# automatically from scalar float code by -O3).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 3) -> str:
    cc = hipcc()
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        cmd = [cc, *common]
        if src.endswith(".hip"):
            cmd += DEVICE_FLAGS + ["-x", "hip"]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len([p for p in procs if p[1].poll() is None]) >= jobs:
            procs[0][1].wait()
    for src, p in procs:
        out, _ = p.communicate()
        msgs = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
        if p.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
    tmp = OUT + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libbd.so failed:\n" + r.stdout)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
