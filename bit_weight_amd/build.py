"""Build libsherry.so (gfx950) in-tree with hipcc.

    python -m bit_weight_amd.build

Every HIP source under csrc/ is compiled for gfx950 only (one object each,
in parallel) and linked into bit_weight_amd/libsherry.so.  Packed-FP32
instruction selection is switched off for device code (-packed-fp32-ops);
hipcc's host pass warns that it does not know that feature, which is
harmless.  MFMA accumulators are kept in arch VGPRs (-amdgpu-mfma-vgpr-form).
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsherry.so")
SOURCES = ["sherry_abi.hip", "pack.hip", "lut_gemv.hip", "mfma_gemm.hip", "mfma_gemv.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# MFMA accumulators in arch VGPRs: the matrix ops then accumulate in place
# instead of shuffling accumulation registers every k-step
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# Kernel arguments preloaded into SGPRs at dispatch instead of read from the
# kernel-argument segment by the first instructions: the product kernels'
# eight leading ones (packed, x, xf, M, N, K and two plan integers, 11
# SGPRs), the quantizer's four (x, q, s_x, K)
PRELOAD = {"mfma_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
           "lut_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
           "mfma_gemm.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
           "pack.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=4"]}


def _filter(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    """Compile every source into libsherry.so (always recompiles)."""
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="sherry_build_") as obj_dir:
        procs = []
        for src in SOURCES:
            obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
            cmd = [HIPCC, *FLAGS, *VGPR_FORM, *PRELOAD.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                     stderr=subprocess.STDOUT, text=True)))
        objs = []
        for src, obj, proc in procs:
            out = _filter(proc.communicate()[0])
            if proc.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src} ({proc.returncode}):\n{out}")
            if verbose and out.strip():
                print(out, flush=True)
            objs.append(obj)
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_filter(res.stdout + res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
