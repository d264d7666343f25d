"""Build libmoelora.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Run as ``python -m lora_expert_gemm_topk_amd.build``.  The library is built
in-tree next to this file so that it travels with the source tree.
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
LIB = PKG / "libmoelora.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # an inline-asm statement that clobbers a reserved register fails the build
    "-Werror=inline-asm",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.hpp")) + [ROOT / "include" / "moe_lora.h"]


def build(verbose: bool = False) -> Path:
    """Compile every HIP source into libmoelora.so (always recompiles)."""
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{ROOT / 'include'}", f"-I{CSRC}", str(CSRC / "moe_lora.hip"),
           "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(f"built {LIB}", file=sys.stderr)
