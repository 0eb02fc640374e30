"""Build the HIP library ``libfa.so`` in-tree with hipcc for gfx950.

Usage: ``python -m exact_tiled_attention_19_amd.build_lib`` (or ``__graft_entry__.build()``).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fp8.hip"]
OBJ_DIR = os.path.join(PKG_DIR, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    # packed fp32 VALU instructions stay off in every HIP build of this project
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _clean(stderr: str) -> str:
    # the host pass does not know the packed-fp32 feature and says so; that line is noise
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in (stderr or "").splitlines() if noise not in l)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libfa.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        _, err = p.communicate()
        err = _clean(err)
        if p.returncode != 0:
            failed.append(f"{src} ({p.returncode}):\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed: " + "\n".join(failed))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({r.returncode}):\n{_clean(r.stderr)}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
