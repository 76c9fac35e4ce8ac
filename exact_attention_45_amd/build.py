"""Builds libmiattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m exact_attention_45_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmiattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.hip", "fwd_pp_kernel.hip", "fwd_sp_kernel.hip",
           "decode_kernel.hip", "decode_stream_kernel.hip", "bwd_kernel.hip"]
# Per-source extra flags. fwd_sp_kernel runs one wave per SIMD with more than
# 256 registers; by default the compiler then places every MFMA accumulator in
# accumulation registers, and the vector instructions that rescale O force
# copies of all of O at every loop iteration. The VGPR form keeps O and S in
# vector registers (other values still use accumulation registers). The
# backward's dK/dV kernel is in the same situation (its score accumulators
# feed the softmax arithmetic).
SOURCE_FLAGS = {"fwd_sp_kernel.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "bwd_kernel.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code; scalar/float2 math
# still compiles to ordinary VALU instructions.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; ROCm is required to build the library")
    return cand


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compiles every source and links the shared library. Always recompiles."""
    cc = hipcc()
    flags = HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC] + list(extra_flags or [])
    tmpdir = tempfile.mkdtemp(prefix="miattn_build_")
    try:
        objs = []

        def compile_one(src):
            obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
            cmd = [cc, *flags, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
            return obj

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = os.path.join(tmpdir, LIB_NAME)
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        # atomic replace so a running process never maps a half-written file
        staged = LIB_PATH + ".tmp"
        shutil.copyfile(tmp_lib, staged)
        os.replace(staged, LIB_PATH)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
