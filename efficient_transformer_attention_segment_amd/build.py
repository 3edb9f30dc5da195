"""Build libnysattn.so (gfx950) in-tree with hipcc.

Each HIP source is compiled to an object under <repo>/_build/ in parallel, then linked
into efficient_transformer_attention_segment_amd/libnysattn.so. Usage:
    python -m efficient_transformer_attention_segment_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnysattn.so")
SOURCES = ["segmeans.hip", "context.hip", "output.hip", "proj.hip", "backward.hip",
           "backward_general.hip", "flash.hip", "plan.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax reads every score, and results
    # parked in AGPRs would each cost a v_accvgpr_read before any VALU use
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
# The projection GEMMs keep 256 accumulators per lane and only feed them to stores: they
# belong in AGPRs, so those kernels are built without the VGPR-form setting.
NO_VGPR_FORM = {"proj.hip"}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    flags = FLAGS
    if src in NO_VGPR_FORM:
        i = flags.index("-amdgpu-mfma-vgpr-form=1")
        flags = flags[:i - 1] + flags[i + 1:]
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
