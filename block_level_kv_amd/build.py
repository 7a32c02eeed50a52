"""Build libinfllm.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m block_level_kv_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libinfllm.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["infllm_api.cpp", "build.hip", "score.hip", "topk.hip", "attend_rows.hip",
           "attend_prefill.hip", "unit_cache.hip"]

ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return ["-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function", "-fvisibility=hidden", "-I" + os.path.join(ROOT, "include"),
            # the packed-fp32 VALU forms are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-munsafe-fp-atomics"]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
