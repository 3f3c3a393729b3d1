"""Build libtt.so (the C-ABI library behind include/tt.h) for gfx950 with hipcc, in-tree.

    python -m block_mask_diffusion_amd.build            # compile + link
    python -m block_mask_diffusion_amd.build --isa      # also keep the gfx950 assembly (.s)

Every HIP source is compiled with packed-FP32 instruction generation disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns that it does not know
the feature, which is expected.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtt.so")
SOURCES = ["attn.hip", "lmhead.hip", "gemm.hip", "unmask.hip", "api.hip"]
# per-source extra flags: the large-M LM-head kernel keeps the next k-step's LDS reads in flight
# under the current MFMAs only with the ILP-oriented machine scheduler
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}
ARCH = os.environ.get("TT_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(isa: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)

    def one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if isa:
            cmd += ["-save-temps=obj"]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(isa="--isa" in sys.argv, verbose=True))
