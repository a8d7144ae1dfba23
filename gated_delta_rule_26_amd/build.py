"""Build libkda.so (the HIP kernels and the C ABI of include/kda.h) for gfx950, in-tree."""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["kda_api.cpp", "kda_chunk.hip", "kda_chunk_bwd.hip", "kda_decode.hip", "kda_conv.hip", "kda_probe.hip"]
ARCH = "gfx950"
# Per-source extra flags. The matrix-core probe's loop-carried accumulators are kept in the
# VGPR form of the instruction: in the AGPR form the register allocator rotates the 4-float
# accumulators of the 16x16x32 products through copies in every iteration, and the probe
# would time the copies instead of the matrix cores.
EXTRA = {"kda_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def lib_path() -> str:
    return os.path.join(PKG, "libkda.so")


def _flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            # packed-fp32 instructions stay off: ordinary float code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libkda.so (always rebuilds)."""
    hipcc = os.environ.get("HIPCC", "hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *_flags(), *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(line for line in r.stderr.splitlines()
                        if "packed-fp32-ops" not in line)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    out = lib_path()
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
