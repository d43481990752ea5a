"""Build libkvq.so (HIP, gfx950) in-tree with hipcc.

Every kernel source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled (plain FP32 VALU arithmetic), and linked with the C-ABI
source into kv_cache_mixed_amd/libkvq.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["quantize.hip", "shrink.hip", "decode_attn.hip", "pairs.hip", "window.hip", "kvq_api.cpp", "alloc.cpp"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-flush-denormals-to-zero",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src + ".o")
    cmd = ["hipcc", "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + COMMON
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-6000:]))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "4")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-4000:])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
