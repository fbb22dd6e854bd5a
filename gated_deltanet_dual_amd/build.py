"""Build libflare_gdn.so in-tree for gfx950 (hipcc) -- always recompiles.

Run as ``python -m gated_deltanet_dual_amd.build`` or through
``__graft_entry__.build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libflare_gdn.so")
BUILD = os.path.join(HERE, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]

SOURCES_HIP = ["api.hip", "block_step.hip", "shortconv.hip", "gdn_fwd.hip", "gdn_bwd.hip", "gdn_bwd_chunk.hip", "gdn_scan.hip", "gdn_bwd_pre.hip", "gdn_tri.hip", "gdn_fwd_pre.hip", "gdn_fwd_out.hip", "shortconv_bwd.hip", "route1.hip", "timing.hip", "noalloc.hip", "gdn_l2.hip", "gdn_fwd_prep.hip"]
SOURCES_CXX = ["host_plan.cpp"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC] + HIP_FLAGS + ["-c", path, "-o", obj]
    else:
        cmd = ["g++"] + CXX_FLAGS + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    noise = "'-packed-fp32-ops' is not a recognized feature"
    rest = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if rest:
        sys.stderr.write(rest + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES_HIP + SOURCES_CXX
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
