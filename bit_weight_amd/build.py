"""Build libsherry.so (gfx950) in-tree with hipcc.

    python -m bit_weight_amd.build

Every HIP source under csrc/ is compiled for gfx950 only and linked into
bit_weight_amd/libsherry.so.  Packed-FP32 instruction selection is switched
off for device code (-packed-fp32-ops); hipcc's host pass warns that it does
not know that feature, which is harmless.  MFMA accumulators are kept in arch
VGPRs (-amdgpu-mfma-vgpr-form).
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsherry.so")
SOURCES = ["sherry_abi.hip", "pack.hip", "lut_gemv.hip", "mfma_gemm.hip", "mfma_gemv.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in arch VGPRs: the matrix ops then accumulate in
    # place instead of shuffling accumulation registers every k-step
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Compile every source into libsherry.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
