"""Build libeagle.so (the eagle.h C ABI) for gfx950 in-tree.

Usage: python -m speculative_decoding_parent_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libeagle.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -ffp-contract=off: sums and products round exactly as written (tree values
# are single fp32 adds; fused multiply-adds are spelled out with fmaf).
# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in generated code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE,
         "-Wall", "-Wno-unused-function"]

SOURCES = ["mask.hip", "tree.hip", "accept.hip", "lmhead.hip", "attn.hip", "layer.hip", "kv.hip", "sampling.hip",
           "status.hip"]


# Per-source options.  lmhead.hip: MFMA results in VGPR form, with AGPRs as
# spill space (the 8-tile LM head at 32 < T <= 64 holds 128 accumulators next
# to a k step of W; the default form spills 136 registers to memory).
SOURCE_FLAGS = {"lmhead.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libeagle.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(objs)} sources")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
