"""Build the HIP library libnvfp4gg.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "nvfp4gg.hip")
LIB = os.path.join(PKG, "libnvfp4gg.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are switched off for all device code; the compiler
# otherwise forms them from plain float code.  MFMA accumulators are kept in
# VGPRs: with the unified register file of gfx950 that lets the register
# allocator share a wave's 256 registers between accumulators and operands
# as the kernel needs (AGPR accumulators cap the VGPRs at 128).
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-Wall",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(extra_flags=None, out: str = LIB) -> str:
    """Compile csrc/nvfp4gg.hip into ``out`` (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags or []) + [
        "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
