"""Build libdpg.so (the C-ABI library and its gfx950 kernels) in place.

    python -m dp_grape_projection_amd.build

Compiles every csrc/*.hip for gfx950 with hipcc into
dp_grape_projection_amd/libdpg.so. No GPU is needed to build.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdpg.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"),
                 "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdpg.so)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile all sources and link libdpg.so; returns its path."""
    cc = hipcc()
    objs = []
    with tempfile.TemporaryDirectory(prefix="dpg_build_") as tmp:
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src,
                   "-o", obj]
            _run(cmd, verbose)
            objs.append(obj)
        out_tmp = LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
              "-o", out_tmp], verbose)
        os.replace(out_tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that
    # warning is expected and harmless.
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
