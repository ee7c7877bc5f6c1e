"""Build libmmssd.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m selective_state_space_12_amd._build`` or through
``__graft_entry__.build()``.  Objects go to ``_build/`` at the repository root;
the shared library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmmssd.so")

HIP_SOURCES = ["conv1d_silu.hip", "ssd_step.hip", "ssd_fwd.hip", "ssd_fwd_bf16.hip", "fused.hip",
               "gated_rmsnorm.hip", "ssd_bwd.hip", "conv1d_silu_bwd.hip",
               "noalloc.hip"]
CPP_SOURCES = ["abi.cpp", "validate.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def common_flags() -> list:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # packed fp32 VALU ops stay off (plain scalar/vector fp32 code only)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + common_flags() + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(extra_flags: list | None = None, verbose: bool = True) -> str:
    """Compile every HIP/C++ source for gfx950 and link libmmssd.so."""
    extra = list(extra_flags or [])
    os.makedirs(BUILD, exist_ok=True)
    sources = HIP_SOURCES + CPP_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), sources))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(sys.argv[1:])
