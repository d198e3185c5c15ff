"""Build libsdpa.so in-tree with hipcc for gfx950.

    python -m transformer_attention_sdpa_amd.build_lib

Compiles every source under csrc/ (host C ABI and HIP kernels) into
``transformer_attention_sdpa_amd/libsdpa.so``.  Runs without a GPU: hipcc
cross-compiles the gfx950 code objects.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsdpa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["sdpa_api.cpp", "sdpa_bf16.hip", "sdpa_bf16_short.hip", "sdpa_bf16_decode.hip",
           "sdpa_f32.hip", "sdpa_f32_short.hip", "sdpa_f32_bwd.hip", "sdpa_mha.hip", "sdpa_bf16_bwd.hip",
           "sdpa_bf16_width.hip", "sdpa_bf16_wide.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -amdgpu-mfma-vgpr-form: MFMA accumulators in VGPRs, so the softmax reads
#   the scores and rescales the output without AGPR copies.
FLAGS = [
    "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
