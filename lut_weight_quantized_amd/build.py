"""Compile the HIP library ``liblut6.so`` for gfx950, in-tree.

    python -m lut_weight_quantized_amd.build

Every call compiles (no up-to-date check): a stale library must never be
mistaken for the current sources.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "liblut6.so"
SOURCES = [CSRC / "lut6_linear.hip", CSRC / "lut6_quantize.hip", CSRC / "lut6_attention.hip",
           CSRC / "lut6_gated_delta.hip",
           CSRC / "lut6_format.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the LUT-6 library)")


def flags() -> list[str]:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            f"-I{ROOT / 'include'}", "-Wall", "-Wno-unused-result",
            # keep the compiler from forming packed-FP32 instructions
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> Path:
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [hipcc(), *flags(), "-o", str(tmp), *map(str, SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
