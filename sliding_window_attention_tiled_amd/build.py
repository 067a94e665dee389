"""Build libswa.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m sliding_window_attention_tiled_amd.build

Every call recompiles.  The objects go to csrc/_build/ and the library to the
package directory, where binding.py loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libswa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["swa_api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "decode.hip", "bwd_bf16.hip",
           "bwd_f32.hip", "bwd_global.hip"]

# Packed FP32 instructions stay off: every float operation is scalar per lane.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source device flags.  The backward kernels keep loop-carried MFMA
# accumulators: in the VGPR form the compiler feeds them to the matrix cores
# where they live instead of copying them through the AGPR file on every step.
SOURCE_FLAGS = {"bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(PKG, "..", "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    extra = SOURCE_FLAGS.get(src, [])
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o",
               obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build() -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
