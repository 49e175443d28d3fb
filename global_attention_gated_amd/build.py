"""Build the zgattn HIP library (libzgattn.so) in-tree for gfx950 with hipcc.

Usage: python -m global_attention_gated_amd.build
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
LIB = os.path.join(PKG, "libzgattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU instructions are switched off for all device code.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include")]
# Device sources assume finite-or-infinite, never NaN, operands (NaN inputs are outside the library's
# contract); this lets fmaxf compile to plain v_max without quieting canonicalisations.
DEVICE_FLAGS = ["-fno-honor-nans"]
# The streaming SWA kernel fits one work-group per CU (LDS), which would let the compiler hand it 512 vector
# registers and put every MFMA accumulator in AGPRs; its softmax reads the score accumulators with VALU
# instructions, so its MFMAs are kept in VGPR form.
SOURCE_FLAGS = {"attn_swa_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
SOURCES = ["attn_tile.hip", "attn_swa_stream.hip", "attn_backward.hip", "decode.hip", "fp8.hip", "linear.cpp",
           "zgattn_api.cpp"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(BUILD, s + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if s.endswith(".cpp") else DEVICE_FLAGS + SOURCE_FLAGS.get(s, [])
        cmds.append([HIPCC] + HIP_FLAGS + lang + ["-c", src, "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + ["-L/opt/rocm/lib", "-lhipblaslt"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
