"""Build libswa.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m sliding_window_attention_tiled_amd.build

Every call recompiles.  The objects go to csrc/_build/ and the libraries to
the package directory, where binding.py loads them: libswa.so (release),
libswa_debug.so (SWA_DEBUG checks) and libswa_hostasan.so (host code under
AddressSanitizer).
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

SOURCES = ["swa_api.cpp", "fwd_bf16.hip", "fwd_pp.hip", "fwd_f32.hip", "decode.hip", "bwd_bf16.hip",
           "bwd_f32.hip", "bwd_global.hip"]

# Packed FP32 instructions stay off: every float operation is scalar per lane.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source device flags.  The backward kernels keep loop-carried MFMA
# accumulators: in the VGPR form the compiler feeds them to the matrix cores
# where they live instead of copying them through the AGPR file on every step.
SOURCE_FLAGS = {"bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(PKG, "..", "include")]


def _compile(src: str, objdir: str = OBJ, defines=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    extra = SOURCE_FLAGS.get(src, [])
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *extra, *defines, *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _link(objs, lib: str, extra=()) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build() -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    _link(objs, LIB)
    build_host_asan(objs)
    build_debug()
    return LIB


# The debug build: every source compiled with SWA_DEBUG, which turns on the
# kernels' index-contract counters (read with swa_debug_violations) and the
# extra barriers and immediate copy waits that serialise overlapped phases.
# Same C ABI as libswa.so; tests load it beside the release library and
# compare the two bit for bit.
DEBUG_LIB = os.path.join(PKG, "libswa_debug.so")
DEBUG_OBJ = os.path.join(OBJ, "debug")


def build_debug() -> str:
    os.makedirs(DEBUG_OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, DEBUG_OBJ, ["-DSWA_DEBUG"]), SOURCES))
    return _link(objs, DEBUG_LIB)


# AddressSanitizer on the host code only (the validator and planner in
# swa_api.cpp): the sanitizer applies to the host side of that one file, the
# kernels are the release objects.  The library expects the ASan runtime to be
# preloaded into the process that loads it (tests/test_host_asan.py does).
HOST_ASAN_LIB = os.path.join(PKG, "libswa_hostasan.so")
HOST_ASAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def build_host_asan(objs=None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    if objs is None:
        objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    api_obj = os.path.join(OBJ, "swa_api_hostasan.o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *HOST_ASAN_FLAGS, "-x", "hip", "-c",
           os.path.join(CSRC, "swa_api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on swa_api.cpp (host ASan)")
    others = [o for o in objs if not o.endswith(os.sep + "swa_api.o")]
    return _link([api_obj, *others], HOST_ASAN_LIB, HOST_ASAN_FLAGS)


if __name__ == "__main__":
    print(build())
