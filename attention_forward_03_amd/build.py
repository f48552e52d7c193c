"""Build the HIP library ``libattn.so`` in place (gfx950 only).

    python -m attention_forward_03_amd.build

Sources are compiled in parallel with hipcc, then linked into a shared library
next to this file. Packed fp32 VALU instructions are disabled for every HIP
translation unit. The instruction stream of the head_dim-128 prefill loop is
written by csrc/gen_prefill_r2.py into _build/gen first (prefill.hip includes it).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn.so"
SOURCES = ("prefill.hip", "prefill_fp8.hip", "backward.hip", "decode.hip", "probes.hip", "api.cpp")
ARCH = "gfx950"
# The compiler-built kernels take the VGPR form of the matrix-core instructions: their
# accumulators live in ordinary vector registers, so the vector work on them (rescale,
# masks, normalisation) needs no copies between the accumulation and vector register
# files, and a kernel that fits in 256 registers runs two waves per SIMD. The D=128
# prefill loop is inline asm either way; probes.hip keeps the default, so its measured
# peaks stay comparable across builds.
SOURCE_FLAGS = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"]
                for src in ("prefill.hip", "prefill_fp8.hip", "backward.hip", "decode.hip")}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def generate(out_dir: str) -> str:
    """Run the prefill loop generator; returns the include directory it wrote."""
    gen_dir = os.path.join(out_dir, "gen")
    cmd = [sys.executable, os.path.join(CSRC, "gen_prefill_r2.py"), gen_dir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"generating the prefill loop failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return gen_dir


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    hipcc = _hipcc()
    gen_dir = generate(out_dir)

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *common_flags(), *SOURCE_FLAGS.get(src, []), "-I", gen_dir, *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = os.path.join(HERE, LIB_NAME + ".tmp")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    final = os.path.join(HERE, LIB_NAME)
    os.replace(tmp, final)
    return final


if __name__ == "__main__":
    print(build(verbose=True))
