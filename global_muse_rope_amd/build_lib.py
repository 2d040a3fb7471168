"""Build libmuse_attn.so (HIP, gfx950 only) in-tree with hipcc.

Usage: python -m global_muse_rope_amd.build_lib
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmuse_attn.so")
SOURCES = ["api.hip", "prologue.hip", "prefill.hip", "decode.hip", "block.hip", "draft.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
]
# Per-source flags.  The decode and drafter kernels keep their MFMA
# accumulators in ordinary VGPRs: the accumulators are rescaled on a rarely
# taken branch, and in accumulation registers every pass would copy them out
# and back.
SOURCE_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "draft.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmuse_attn.so")


def _compile(src: str, defines=(), tag="") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *["-D" + d for d in defines], "-c",
           os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every HIP source for gfx950 and link the shared library.
    `defines` (macro definitions) and `out` select a variant build."""
    os.makedirs(BUILD, exist_ok=True)
    tag = "" if not defines else "_" + "_".join(d.replace("=", "") for d in defines)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, defines, tag), SOURCES))
    tmp = out + ".tmp"
    # hipBLASLt runs the block's two projection GEMMs
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp, "-lhipblaslt"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
