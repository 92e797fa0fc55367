"""Build liblisa.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m vision_transformer_token_amd.build
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("lisa_flow.hip", "lisa_resident.hip", "lisa_backward.hip", "lisa_layer.hip", "lisa_api.hip")]
LIB = os.path.join(PKG, "liblisa.so")

HIPCC_FLAGS = [
    "-O3",
    "-std=c++17",
    "--offload-arch=gfx950",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed fp32 VALU ops stay off: plain float code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the kernels feed them straight into
    # VALU work, which would otherwise copy them out of accumulation registers.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build liblisa.so")
    return path


def build(verbose=False):
    """Compile every HIP source into vision_transformer_token_amd/liblisa.so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (res.stdout + res.stderr).splitlines()
        if "is not a recognized feature for this target" not in line
    )
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
