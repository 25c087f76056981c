"""Build libkda.so (the HIP kernels + the C ABI) in-tree for gfx950 with hipcc.

Usage: python -m gated_delta_rule_67_amd.build  (or call build()).
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_prefill.hip", "kda_chunk_bf16.hip",
           "kda_chunk_wy.hip", "kda_chunk_bwd.hip", "kda_gate.hip"]


def hipcc():
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def compile_command(out):
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # never emit packed-FP32 VALU instructions (v_pk_{add,mul,fma}_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkda.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
