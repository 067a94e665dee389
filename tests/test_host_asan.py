"""Host-side AddressSanitizer run of the validator and planner (CPU only).

libswa_hostasan.so is libswa.so with swa_api.cpp's host code built under
AddressSanitizer (the kernels are the release objects).  A child process with
the ASan runtime preloaded drives the entry points through every path that
ends before anything is enqueued: argument checks, the sorting and
deduplication of global positions (out-of-range, duplicated, more than the
supported number), the planners' size and overflow checks, and the workspace
size queries over many shapes.  Any heap or stack error in that host code
aborts the child with an ASan report.  No HIP runtime call is made."""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sliding_window_attention_tiled_amd import build as swa_build  # noqa: E402

CHILD = r"""
import ctypes, sys
lib = ctypes.CDLL(sys.argv[1])
P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
lib.swa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, P, I, F, I, P, SZ, P]
lib.swa_fwd.restype = I
lib.swa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, I, F, I, P, SZ, P]
lib.swa_bwd.restype = I
for name, n in (("swa_fwd_workspace_size", 5), ("swa_decode_workspace_size", 4),
                ("swa_decode_sinks_workspace_size", 5), ("swa_bwd_workspace_size", 6)):
    getattr(lib, name).argtypes = [I] * n
    getattr(lib, name).restype = SZ
lib.swa_status_string.argtypes = [I]
lib.swa_status_string.restype = ctypes.c_char_p
lib.swa_decode.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, P, SZ, I, P]
lib.swa_decode.restype = I
lib.swa_kv_append_chunk.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P]
lib.swa_kv_append_chunk.restype = I

D = P(0x1000)   # a device pointer that no host path dereferences
BF16 = 1
ARG, UNSUP, WS = -1, -2, -3

def gidx(vals):
    return (ctypes.c_int32 * max(1, len(vals)))(*vals), len(vals)

def fwd(B=1, Hq=4, Hkv=2, N=1000, Dh=128, wl=100, wr=0, dil=1, g=(), scale=0.1, ws=None, wsb=0):
    arr, n = gidx(list(g))
    return lib.swa_fwd(D, D, D, D, None, B, Hq, Hkv, N, Dh, wl, wr, dil,
                       arr if n else None, n, scale, BF16, ws, wsb, None)

checks = 0
def expect(got, want, what):
    global checks
    checks += 1
    assert got == want, (what, got, want)

# argument checks
expect(fwd(B=0), ARG, "B=0"); expect(fwd(Hq=5, Hkv=2), ARG, "Hq % Hkv")
expect(fwd(Dh=96), UNSUP, "D"); expect(fwd(wl=-1), ARG, "wl<0"); expect(fwd(dil=0), ARG, "dil")
for sc in (0.0, -1.0, float("inf"), float("nan")):
    expect(fwd(scale=sc), ARG, f"scale {sc}")
expect(fwd(N=1 << 29), ARG, "N too large")
# global positions: out of range, duplicates, too many, workspace missing or short
expect(fwd(g=(5, 1000)), ARG, "global out of range"); expect(fwd(g=(-1,)), ARG, "global < 0")
expect(fwd(g=(3, 3, 3, 7, 7)), WS, "dupes, no workspace")
expect(fwd(g=list(range(0, 1000, 3))), UNSUP, "more than 256 distinct")
expect(fwd(g=[1] * 5000 + [2]), WS, "5001 entries, 2 distinct")
need = lib.swa_fwd_workspace_size(1, 4, 1000, 128, 2)
expect(fwd(g=(1, 2), ws=D, wsb=need - 1), WS, "short workspace")
# backward: the same checks through its own validator
arr, n = gidx([9, 9, 1])
expect(lib.swa_bwd(D, D, D, D, D, D, D, D, D, 1, 4, 2, 1000, 128, 100, 0, 1, arr, n, 0.1,
                   BF16, None, 0, None), WS, "bwd workspace")
arr, n = gidx([1000])
expect(lib.swa_bwd(D, D, D, D, D, D, D, D, D, 1, 4, 2, 1000, 128, 100, 0, 1, arr, n, 0.1,
                   BF16, D, 1 << 30, None), ARG, "bwd global out of range")
# decode and chunk append argument checks
expect(lib.swa_decode(D, D, D, D, D, D, None, 0, 32, 8, 4096, 128, 0.1, None, 0, BF16, None),
       ARG, "decode B=0")
expect(lib.swa_decode(D, D, D, D, D, D, None, 4, 32, 8, 4096, 128, 0.1, None, 0, BF16, None),
       WS, "decode no workspace")
expect(lib.swa_kv_append_chunk(D, D, D, D, D, D, 2, 8, 4096, -1, 128, BF16, None), ARG,
       "chunk n<0")
# planners over many shapes (sizes only; a query never launches anything)
for B in (1, 3, 64):
    for N in (1, 2, 63, 64, 65, 1000, 16384, 1 << 20):
        for Dh in (64, 128):
            for ng in (0, 1, 16, 256):
                lib.swa_fwd_workspace_size(B, 32, N, Dh, ng)
                lib.swa_bwd_workspace_size(B, 32, 8, N, Dh, ng)
                checks += 1
for W in (1, 64, 4095, 4096, 1 << 20):
    lib.swa_decode_workspace_size(64, 32, W, 128)
    lib.swa_decode_sinks_workspace_size(64, 32, W, 128, 4)
    checks += 1
for st in range(-8, 3):
    lib.swa_status_string(st)
print("ASAN_OK", checks)
"""


def _asan_runtime():
    r = subprocess.run([swa_build.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path):
        found = glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = found[0] if found else ""
    return path


def test_host_validator_and_planner_under_asan():
    if not os.path.exists(swa_build.HOST_ASAN_LIB):
        swa_build.build_host_asan()
    rt = _asan_runtime()
    assert os.path.exists(rt), "ASan runtime not found"
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1")
    r = subprocess.run([sys.executable, "-c", CHILD, swa_build.HOST_ASAN_LIB],
                       capture_output=True, text=True, env=env, timeout=600)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    assert "ASAN_OK" in r.stdout
