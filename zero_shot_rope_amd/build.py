"""Build the HIP library libbifocal.so in-tree for gfx950.

    python -m zero_shot_rope_amd.build [--verbose]

One hipcc invocation compiles the C ABI (api.cpp) and the kernels (*.hip) into
zero_shot_rope_amd/libbifocal.so. Packed FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbifocal.so")
SOURCES = ["api.cpp", "prefill.hip", "decode.hip", "unfused.hip", "scratch.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the bifocal library needs ROCm's hipcc to build")


def command(out: str = LIB, extra=()):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        *extra,
        "-x", "hip", *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    """Compile the library; return its path. Always recompiles."""
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    log = "\n".join(line for line in res.stdout.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{log}")
    if verbose and log.strip():
        print(log)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
