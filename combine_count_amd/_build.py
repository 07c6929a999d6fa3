"""Build libepdc.so in-tree with hipcc for gfx950.

Each call compiles every source again (the build check must not trust a
stale library).  Objects go to combine_count_amd/_build/, the library to
combine_count_amd/libepdc.so.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libepdc.so")
SOURCES = ["epdc_api.cpp", "dispatch.hip", "combine.hip", "combine_push.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    # the only fused multiply-adds are the explicit ones
    "-ffp-contract=off",
]
# device code only: no packed fp32 (v_pk_*_f32) code generation
DEVICE = ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        lang = DEVICE if src.endswith(".hip") else []
        cmd = [HIPCC, *lang, *COMMON, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the device feature flag: drop that note
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if msg.strip() and (verbose or r.returncode):
            print(msg, flush=True)
        if r.returncode:
            raise subprocess.CalledProcessError(r.returncode, cmd)
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
