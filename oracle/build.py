"""Build the oracle's C library with gcc (test infrastructure only)."""

from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile oracle/kda_oracle.c into oracle/libkda_oracle.so (always recompiles).

    IEEE float64 semantics: no -ffast-math and no FMA contraction, so every step rounds
    exactly as written."""
    src = os.path.join(_HERE, "kda_oracle.c")
    out = lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
