"""Build libfmlp.so (the C-ABI library) in-tree with hipcc, for gfx950 only.

    python -m gemm_epilogue_bf16_amd.build        # or build() from Python

Every source under csrc/ is compiled for --offload-arch=gfx950 (cross-compiles
without a GPU) and linked into gemm_epilogue_bf16_amd/libfmlp.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfmlp.so")
SOURCES = ["abi.cpp", "gemm.hip", "decode.hip", "decode_w8.hip", "small_mlp.hip", "moe.hip", "transpose.hip", "noalloc.hip",
           "glu_fused.hip"]
ARCH = "gfx950"
# Per-source flags.  The GEMM main loop is written in issue order (fragment
# reads of the next stage ahead of the MFMAs they hide behind); the pre-RA
# machine scheduler reorders it so that the 256 fp32 accumulators of a wave no
# longer fit in AGPRs next to the fragments, and the register allocator then
# shuffles them between register files on every MFMA.  Keeping the source
# order keeps them in place.  The FP8 decode loop is written the same way (one
# register batch's loads issued before the previous batch is converted).
EXTRA_FLAGS = {"gemm.hip": ["-mllvm", "-enable-misched=0"],
               "decode_w8.hip": ["-mllvm", "-enable-misched=0"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfmlp)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        f"-I{os.path.join(ROOT, 'include')}",
        # never emit packed fp32 arithmetic (hand-written or generated)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link libfmlp.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
