"""Build libbqa.so for gfx950 with hipcc (one object per source, linked shared).

Run as ``python -m bit_quantized_attention_amd.csrc.build`` or through
``__graft_entry__.build()``.  Objects go to ``_build/`` at the repository
root; the library lands next to the Python binding.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libbqa.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "quant.hip", "attn_sage_fwd.hip", "attn_qat.hip", "select.hip", "attn_thrift.hip", "attn_sage_bwd.hip",
           "attn_qat_bwd.hip", "debug.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", HERE,
]
# Per-source additions.  The Thrift decode kernel runs vector work on its
# matrix accumulators every key block; with accumulators in AGPRs (the
# compiler's choice when one wavefront per SIMD leaves it 512 registers) each
# of those instructions costs two extra register-file moves.  The VGPR form
# keeps them in VGPRs (214 registers, no spills; the prefill kernel of the
# same file compiles to the same code either way).
# The attention kernels take row maxima of matrix results; their scores are
# finite or -inf (masked) and never NaN for finite inputs (non-finite inputs
# give unspecified results unless the BQA_DEBUG scan, built without this flag,
# rejects them), so with -fno-honor-nans the backend forms v_max3_f32 directly
# instead of first canonicalising each matrix result with a v_max x, x
# (measured: c3 backward 1.083 -> 1.058 ms).
EXTRA = {"attn_thrift.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
         "attn_qat.hip": ["-fno-honor-nans"],
         "attn_sage_fwd.hip": ["-fno-honor-nans"],
         "attn_sage_bwd.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip" if src.endswith(".hip") else "hip", "-c",
           os.path.join(HERE, src), "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # A kernel that spills registers to scratch memory runs several times
    # slower; refuse to build one (BQA_ALLOW_SCRATCH=1 overrides).
    spills, name = [], None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0 and name:
            spills.append(f"{name}: {m.group(1)} bytes/lane")
    if spills and os.environ.get("BQA_ALLOW_SCRATCH") != "1":
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills):\n  " + "\n  ".join(spills))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
