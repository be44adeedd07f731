"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, then linked into
routed_expert_quantized_amd/libmoe.so. Run: python -m routed_expert_quantized_amd.build

With --stamps the same sources are built with -DMOE_STAMPS into
libmoe_stamps.so instead: the timestamp build that
`python -m routed_expert_quantized_amd.timeline` loads (csrc/stamps.hpp).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
STAMPS_LIB = os.path.join(PKG, "libmoe_stamps.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions stay off: all float math is written as scalar code.
CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, stamps: bool = False) -> str:
    obj = os.path.join(BUILD, ("stamps_" if stamps else "") + os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *(["-DMOE_STAMPS"] if stamps else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, stamps: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = max(1, min(len(srcs), os.cpu_count() or 4, 16))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, stamps), srcs))
    lib = STAMPS_LIB if stamps else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, stamps="--stamps" in sys.argv[1:])
