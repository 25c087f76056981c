"""Build libkda.so (the HIP kernels + the C ABI) in-tree for gfx950 with hipcc.

Each source compiles to its own object in parallel (a translation unit carries its own
kernels, so no relocatable device code is needed); one hipcc call links the library.

Usage: python -m gated_delta_rule_67_amd.build  (or call build()).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_prefill.hip", "kda_chunk_bf16.hip",
           "kda_chunk_wy.hip", "kda_chunk_bwd.hip", "kda_gate.hip", "kda_stream.hip"]


def hipcc():
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def _flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        # never emit packed-FP32 VALU instructions (v_pk_{add,mul,fma}_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
    ]


def compile_command(src, obj):
    return [hipcc()] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs, out):
    return [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out] + objs


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
    return res.returncode


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as pool:
        codes = list(pool.map(lambda so: _run(compile_command(*so), verbose), zip(SOURCES, objs)))
    if any(codes):
        raise RuntimeError("hipcc failed compiling the KDA sources")
    tmp = LIB + ".tmp"
    if _run(link_command(objs, tmp), verbose) != 0:
        raise RuntimeError("hipcc failed linking libkda.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
