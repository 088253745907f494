"""Build ``liblily_moe.so`` (HIP, gfx950) in-tree with hipcc, and its
tracing twin ``liblily_moe_trace.so`` (the same objects but gemm_w4.hip and
decode.hip, compiled with LILY_TRACE_ITEMS: the traces of lily_trace.h).

Every source is compiled for gfx950 only. Packed FP32 instructions are
disabled on the device side (``-packed-fp32-ops``); the host pass warns that
it does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblily_moe.so")
TRACE_LIB = os.path.join(HERE, "liblily_moe_trace.so")

SOURCES = ["abi.hip", "route.hip", "route_host.hip", "gemm_w4.hip", "decode.hip", "router.hip",
           "residual.hip", "calib.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
         "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(src: str, trace: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_trace.o" if trace else ".o"))
    cmd = [_hipcc(), *FLAGS, *(["-DLILY_TRACE_ITEMS"] if trace else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link the shared library and its
    tracing twin."""
    os.makedirs(BUILD, exist_ok=True)
    traced_src = ("gemm_w4.hip", "decode.hip")
    units = [(src, False) for src in SOURCES] + [(src, True) for src in traced_src]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(units))) as ex:
        objs = list(ex.map(lambda u: _compile(*u), units))
    _link(objs[:len(SOURCES)], LIB)
    tobj = dict(zip(traced_src, objs[len(SOURCES):]))
    _link([tobj.get(src, o) for src, o in zip(SOURCES, objs)], TRACE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(*(int(a) for a in sys.argv[1:])))
