"""Build the gfx950 HIP library ``libmoe.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["api.hip", "route.hip", "permute.hip", "ffn_decode.hip", "ffn_decode_shared.hip", "ffn_small.hip",
           "ffn_prefill.hip", "pack.hip", "noalloc.hip", "micro.hip",
           "combine.hip", "cache.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# host-only sources (the host side of the bandwidth-adaptive placement)
HOST_SOURCES = ["cpu_expert.cpp"]
CXX = os.environ.get("CXX_HOST", "g++")
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-fopenmp", "-I", INCLUDE]


def _compile(src: str) -> str:
    if src.endswith(".cpp"):
        obj = os.path.join(OBJDIR, src.replace(".cpp", ".o"))
        cmd = [CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"{CXX} failed on {src}")
        return obj
    obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + HOST_SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-lgomp"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    print(build())
