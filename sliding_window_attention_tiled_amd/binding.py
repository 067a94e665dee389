"""ctypes binding of libswa.so (the C ABI in include/swa.h).

Argument marshalling only: shapes are read from the torch tensors, pointers
and the current HIP stream are passed through, and every step of the
computation runs in the library's kernels.  There is no fallback: if the
library has not been built, the first call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswa.so")
DEBUG_LIB_PATH = os.path.join(_PKG, "libswa_debug.so")

SWA_F32, SWA_BF16 = 0, 1
_STATUS = {0: "SWA_OK", -1: "SWA_ERR_ARG", -2: "SWA_ERR_UNSUPPORTED",
           -3: "SWA_ERR_WORKSPACE", -4: "SWA_ERR_HIP"}

_lib = None


class SwaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libswa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(path)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Route this module's calls through another build of the library with the
    same C ABI (libswa_debug.so, say) inside the `with` block."""
    global _lib
    saved = _lib
    _lib = _open(path)
    try:
        yield _lib
    finally:
        _lib = saved


def debug_violations(reset: bool = True) -> int:
    """Failed index checks counted by the debug build's kernels on the current
    device since the last reset (waits for the device).  Raises SwaError
    (SWA_ERR_UNSUPPORTED) in the release build."""
    n = ctypes.c_ulonglong(0)
    _check(load_library().swa_debug_violations(ctypes.byref(n), int(reset)),
           "swa_debug_violations")
    return int(n.value)


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise SwaError(-4, f"{path} is missing: build it first "
                           "(python -m sliding_window_attention_tiled_amd.build)")
    lib = ctypes.CDLL(path)
    P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.swa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, P, I, F, I, P, SZ, P]
    lib.swa_fwd.restype = I
    lib.swa_fwd_workspace_size.argtypes = [I, I, I, I, I]
    lib.swa_fwd_workspace_size.restype = SZ
    lib.swa_kv_append.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P]
    lib.swa_kv_append.restype = I
    lib.swa_kv_append_chunk.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.swa_kv_append_chunk.restype = I
    lib.swa_fwd_cached.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.swa_fwd_cached.restype = I
    lib.swa_decode.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, P, SZ, I, P]
    lib.swa_decode.restype = I
    lib.swa_decode_sinks.argtypes = [P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, F, P, SZ,
                                     I, P]
    lib.swa_decode_sinks.restype = I
    lib.swa_decode_sinks_workspace_size.argtypes = [I, I, I, I, I]
    lib.swa_decode_sinks_workspace_size.restype = SZ
    lib.swa_kv_append_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P]
    lib.swa_kv_append_paged.restype = I
    lib.swa_decode_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P, SZ, I,
                                     P]
    lib.swa_decode_paged.restype = I
    lib.swa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, I, F, I, P,
                            SZ, P]
    lib.swa_bwd.restype = I
    lib.swa_bwd_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.swa_bwd_workspace_size.restype = SZ
    lib.swa_decode_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.swa_decode_noalloc.restype = I
    lib.swa_decode_workspace_size.argtypes = [I, I, I, I]
    lib.swa_decode_workspace_size.restype = SZ
    lib.swa_status_string.argtypes = [I]
    lib.swa_status_string.restype = ctypes.c_char_p
    lib.swa_version.argtypes = []
    lib.swa_version.restype = I
    lib.swa_debug_violations.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), I]
    lib.swa_debug_violations.restype = I
    return lib


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().swa_status_string(status).decode()
        raise SwaError(status, f"{what}: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SWA_F32
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    raise SwaError(-2, f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise SwaError(-1, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise SwaError(-1, f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _buffer(t: torch.Tensor | None, name: str, shape, dtype, like: torch.Tensor):
    """A caller-supplied tensor the call reads or writes must have exactly the
    shape, dtype and device the call assumes: the C ABI receives bare pointers
    and cannot check them, so a wrong buffer would be an out-of-bounds device
    access.  Checked before any launch (and before the device check of _dev)."""
    if t is None:
        return None
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != like.device:
        raise SwaError(-1, f"{name} must be {dtype} {tuple(shape)} on {like.device}; got "
                           f"{t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _same(ref: torch.Tensor, **tensors):
    """Inputs that share the reference tensor's dtype and device."""
    for name, t in tensors.items():
        if t.dtype != ref.dtype or t.device != ref.device:
            raise SwaError(-1, f"{name} must be {ref.dtype} on {ref.device}; got {t.dtype} on "
                               f"{t.device}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def fwd_workspace_size(B: int, Hq: int, N: int, D: int, n_global: int) -> int:
    return int(load_library().swa_fwd_workspace_size(B, Hq, N, D, n_global))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, win_left: int,
        win_right: int = 0, dilation: int = 1, global_idx=None, scale: float | None = None,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
        workspace: torch.Tensor | None = None, return_lse: bool = True):
    """Sliding-window attention.  q [B,N,Hq,D], k/v [B,N,Hkv,D] (bf16 or fp32).

    Returns (out [B,N,Hq,D], lse [B,Hq,N] fp32) or out alone when
    return_lse is False.  scale=None means 1/sqrt(D).  global_idx is a
    sequence of positions (host side).
    """
    lib = load_library()
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, N, Hkv, D) or v.shape != k.shape:
        raise SwaError(-1, f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} "
                           f"v{tuple(v.shape)}")
    _same(q, k=k, v=v)
    dt = _dtype_code(q)
    _buffer(out, "out", q.shape, q.dtype, q)
    _buffer(lse, "lse", (B, Hq, N), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if global_idx is not None and len(global_idx):
        g = (ctypes.c_int32 * len(global_idx))(*[int(x) for x in global_idx])
        ng = len(global_idx)
    else:
        g, ng = None, 0
    ws_bytes = 0
    if ng:
        need = fwd_workspace_size(B, Hq, N, D, ng)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        elif workspace.device != q.device:
            raise SwaError(-1, f"workspace must be on {q.device}")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.swa_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                     _dev(lse, "lse"), B, Hq, Hkv, N, D, win_left, win_right, dilation,
                     g, ng, float(scale), dt, _dev(workspace, "workspace"), ws_bytes,
                     _stream(q))
    _check(st, "swa_fwd")
    return (out, lse) if return_lse else out


def kv_append(kcache: torch.Tensor, vcache: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, ring_head: torch.Tensor, cache_len: torch.Tensor):
    """In-place ring append.  kcache/vcache [B,Hkv,W,D]; k_new/v_new [B,Hkv,D];
    ring_head/cache_len int32 [B] on the device."""
    lib = load_library()
    B, Hkv, W, D = kcache.shape
    if vcache.shape != kcache.shape or k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D):
        raise SwaError(-1, "kv_append shape mismatch")
    _same(kcache, vcache=vcache, k_new=k_new, v_new=v_new)
    _ring_state(ring_head, cache_len, B, kcache)
    st = lib.swa_kv_append(_dev(kcache, "kcache"), _dev(vcache, "vcache"),
                           _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                           _dev(ring_head, "ring_head"), _dev(cache_len, "cache_len"),
                           B, Hkv, W, D, _dtype_code(kcache), _stream(kcache))
    _check(st, "swa_kv_append")


def _ring_state(ring_head: torch.Tensor, cache_len: torch.Tensor, B: int, like: torch.Tensor):
    for t, name in ((ring_head, "ring_head"), (cache_len, "cache_len")):
        if t.dtype != torch.int32 or t.shape != (B,) or t.device != like.device:
            raise SwaError(-1, f"{name} must be int32 [B] on {like.device}")


def kv_append_chunk(kcache: torch.Tensor, vcache: torch.Tensor, k: torch.Tensor,
                    v: torch.Tensor, ring_head: torch.Tensor, cache_len: torch.Tensor):
    """In-place append of a chunk k/v [B,n,Hkv,D] to the ring kcache/vcache
    [B,Hkv,W,D] (the same result as n single appends)."""
    lib = load_library()
    B, Hkv, W, D = kcache.shape
    n = k.shape[1]
    if vcache.shape != kcache.shape or k.shape != (B, n, Hkv, D) or v.shape != k.shape:
        raise SwaError(-1, "kv_append_chunk shape mismatch")
    _same(kcache, vcache=vcache, k=k, v=v)
    _ring_state(ring_head, cache_len, B, kcache)
    st = lib.swa_kv_append_chunk(_dev(kcache, "kcache"), _dev(vcache, "vcache"), _dev(k, "k"),
                                 _dev(v, "v"), _dev(ring_head, "ring_head"),
                                 _dev(cache_len, "cache_len"), B, Hkv, W, n, D,
                                 _dtype_code(kcache), _stream(kcache))
    _check(st, "swa_kv_append_chunk")


def fwd_cached(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kcache: torch.Tensor,
               vcache: torch.Tensor, ring_head: torch.Tensor, cache_len: torch.Tensor, *,
               win_left: int, scale: float | None = None, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None, return_lse: bool = True):
    """Causal window attention of a prompt chunk q [B,n,Hq,D], k/v [B,n,Hkv,D]
    that follows the tokens held in the ring kcache/vcache [B,Hkv,W,D].
    Returns (out [B,n,Hq,D], lse [B,Hq,n] fp32) or out alone."""
    lib = load_library()
    B, n, Hq, D = q.shape
    Hkv, W = kcache.shape[1], kcache.shape[2]
    if k.shape != (B, n, Hkv, D) or v.shape != k.shape:
        raise SwaError(-1, "fwd_cached chunk shape mismatch")
    if kcache.shape != (B, Hkv, W, D) or vcache.shape != kcache.shape:
        raise SwaError(-1, "fwd_cached ring shape mismatch")
    _same(q, k=k, v=v, kcache=kcache, vcache=vcache)
    _ring_state(ring_head, cache_len, B, q)
    _buffer(out, "out", q.shape, q.dtype, q)
    _buffer(lse, "lse", (B, Hq, n), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    st = lib.swa_fwd_cached(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(kcache, "kcache"),
                            _dev(vcache, "vcache"), _dev(ring_head, "ring_head"),
                            _dev(cache_len, "cache_len"), _dev(out, "out"), _dev(lse, "lse"),
                            B, Hq, Hkv, n, W, D, win_left, float(scale), _dtype_code(q),
                            _stream(q))
    _check(st, "swa_fwd_cached")
    return (out, lse) if return_lse else out


def decode_workspace_size(B: int, Hq: int, W: int, D: int) -> int:
    return int(load_library().swa_decode_workspace_size(B, Hq, W, D))


def decode(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
           ring_head: torch.Tensor, cache_len: torch.Tensor, *, scale: float | None = None,
           workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
           lse: torch.Tensor | None = None, return_lse: bool = True):
    """One decode step over the ring.  q [B,Hq,D] -> out [B,Hq,D] (+ lse [B,Hq])."""
    lib = load_library()
    B, Hq, D = q.shape
    Hkv, W = kcache.shape[1], kcache.shape[2]
    if kcache.shape != (B, Hkv, W, D) or vcache.shape != kcache.shape:
        raise SwaError(-1, "decode shape mismatch")
    _same(q, kcache=kcache, vcache=vcache)
    _ring_state(ring_head, cache_len, B, q)
    _buffer(out, "out", q.shape, q.dtype, q)
    _buffer(lse, "lse", (B, Hq), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_workspace_size(B, Hq, W, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device:
        raise SwaError(-1, f"workspace must be on {q.device}")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.swa_decode(_dev(q, "q"), _dev(kcache, "kcache"), _dev(vcache, "vcache"),
                        _dev(ring_head, "ring_head"), _dev(cache_len, "cache_len"),
                        _dev(out, "out"), _dev(lse, "lse"), B, Hq, Hkv, W, D, float(scale),
                        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                        _dtype_code(q), _stream(q))
    _check(st, "swa_decode")
    return (out, lse) if return_lse else out


def decode_noalloc(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                   ring_head: torch.Tensor, cache_len: torch.Tensor, *,
                   scale: float | None = None, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, return_lse: bool = True):
    """decode() without a workspace: the library keeps the split partials in
    its own per-GPU array (calls that overlap in time on one GPU race).  Pass
    out (and lse) to allocate nothing at all."""
    lib = load_library()
    B, Hq, D = q.shape
    Hkv, W = kcache.shape[1], kcache.shape[2]
    if kcache.shape != (B, Hkv, W, D) or vcache.shape != kcache.shape:
        raise SwaError(-1, "decode shape mismatch")
    _same(q, kcache=kcache, vcache=vcache)
    _ring_state(ring_head, cache_len, B, q)
    _buffer(out, "out", q.shape, q.dtype, q)
    _buffer(lse, "lse", (B, Hq), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.swa_decode_noalloc(_dev(q, "q"), _dev(kcache, "kcache"), _dev(vcache, "vcache"),
                                _dev(ring_head, "ring_head"), _dev(cache_len, "cache_len"),
                                _dev(out, "out"), _dev(lse, "lse"), B, Hq, Hkv, W, D,
                                float(scale), _dtype_code(q), _stream(q))
    _check(st, "swa_decode_noalloc")
    return (out, lse) if return_lse else out


def decode_sinks_workspace_size(B: int, Hq: int, W: int, D: int, n_sink: int) -> int:
    return int(load_library().swa_decode_sinks_workspace_size(B, Hq, W, D, n_sink))


def decode_sinks(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                 ring_head: torch.Tensor, cache_len: torch.Tensor, ksink: torch.Tensor,
                 vsink: torch.Tensor, *, scale: float | None = None,
                 workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, return_lse: bool = True):
    """One decode step over the ring and the sink entries ksink/vsink [B,Hkv,S,D]."""
    lib = load_library()
    B, Hq, D = q.shape
    Hkv, W = kcache.shape[1], kcache.shape[2]
    S = ksink.shape[2]
    if kcache.shape != (B, Hkv, W, D) or vcache.shape != kcache.shape:
        raise SwaError(-1, "decode_sinks ring shape mismatch")
    if ksink.shape != (B, Hkv, S, D) or vsink.shape != ksink.shape:
        raise SwaError(-1, "decode_sinks sink shape mismatch")
    _same(q, kcache=kcache, vcache=vcache, ksink=ksink, vsink=vsink)
    _ring_state(ring_head, cache_len, B, q)
    _buffer(out, "out", q.shape, q.dtype, q)
    _buffer(lse, "lse", (B, Hq), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_sinks_workspace_size(B, Hq, W, D, S)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device:
        raise SwaError(-1, f"workspace must be on {q.device}")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.swa_decode_sinks(_dev(q, "q"), _dev(kcache, "kcache"), _dev(vcache, "vcache"),
                              _dev(ring_head, "ring_head"), _dev(cache_len, "cache_len"),
                              _dev(ksink, "ksink") if S else None,
                              _dev(vsink, "vsink") if S else None, S,
                              _dev(out, "out"), _dev(lse, "lse"), B, Hq, Hkv, W, D,
                              float(scale), _dev(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(), _dtype_code(q),
                              _stream(q))
    _check(st, "swa_decode_sinks")
    return (out, lse) if return_lse else out


def _paged_state(kpool, vpool, block_table, seq_len, B):
    if vpool.shape != kpool.shape:
        raise SwaError(-1, "kpool and vpool must match")
    _same(kpool, vpool=vpool)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
            block_table.shape[0] != B or block_table.device != kpool.device:
        raise SwaError(-1, f"block_table must be int32 [B, nb] on {kpool.device}")
    if seq_len.dtype != torch.int32 or seq_len.shape != (B,) or seq_len.device != kpool.device:
        raise SwaError(-1, f"seq_len must be int32 [B] on {kpool.device}")


def kv_append_paged(kpool: torch.Tensor, vpool: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    block_table: torch.Tensor, seq_len: torch.Tensor, *, window: int):
    """Append k/v [B,n,Hkv,D] to a paged window cache (pool [n_pages,Hkv,P,D])."""
    lib = load_library()
    n_pages, Hkv, P, D = kpool.shape
    B, n = k.shape[0], k.shape[1]
    if k.shape != (B, n, Hkv, D) or v.shape != k.shape:
        raise SwaError(-1, "kv_append_paged shape mismatch")
    _same(kpool, k=k, v=v)
    _paged_state(kpool, vpool, block_table, seq_len, B)
    st = lib.swa_kv_append_paged(_dev(kpool, "kpool"), _dev(vpool, "vpool"),
                                 _dev(k, "k") if n else None, _dev(v, "v") if n else None,
                                 _dev(block_table, "block_table"), _dev(seq_len, "seq_len"),
                                 B, Hkv, n_pages, P, block_table.shape[1], window, n, D,
                                 _dtype_code(kpool), _stream(kpool))
    _check(st, "swa_kv_append_paged")


def decode_paged(q: torch.Tensor, kpool: torch.Tensor, vpool: torch.Tensor,
                 block_table: torch.Tensor, seq_len: torch.Tensor, *, window: int,
                 scale: float | None = None, workspace: torch.Tensor | None = None,
                 out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                 return_lse: bool = True):
    """One decode step over the last `window` positions of a paged cache."""
    lib = load_library()
    B, Hq, D = q.shape
    n_pages, Hkv, P, _ = kpool.shape
    if kpool.shape[3] != D:
        raise SwaError(-1, "decode_paged shape mismatch")
    _same(q, kpool=kpool)
    _paged_state(kpool, vpool, block_table, seq_len, B)
    _buffer(out, "out", q.shape, q.dtype, q)
    _buffer(lse, "lse", (B, Hq), torch.float32, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_workspace_size(B, Hq, window, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device:
        raise SwaError(-1, f"workspace must be on {q.device}")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.swa_decode_paged(_dev(q, "q"), _dev(kpool, "kpool"), _dev(vpool, "vpool"),
                              _dev(block_table, "block_table"), _dev(seq_len, "seq_len"),
                              _dev(out, "out"), _dev(lse, "lse"), B, Hq, Hkv, n_pages, P,
                              block_table.shape[1], window, D, float(scale),
                              _dev(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(), _dtype_code(q),
                              _stream(q))
    _check(st, "swa_decode_paged")
    return (out, lse) if return_lse else out


def bwd_workspace_size(B: int, Hq: int, Hkv: int, N: int, D: int, n_global: int = 0) -> int:
    return int(load_library().swa_bwd_workspace_size(B, Hq, Hkv, N, D, n_global))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, *, win_left: int, win_right: int = 0, dilation: int = 1,
        global_idx=None, scale: float | None = None, dq: torch.Tensor | None = None,
        dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
        workspace: torch.Tensor | None = None):
    """Gradients (dq, dk, dv) of fwd for the upstream gradient dout; out and lse
    from fwd with the same arguments (global_idx included)."""
    lib = load_library()
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, N, Hkv, D) or v.shape != k.shape or out.shape != q.shape or \
            dout.shape != q.shape or lse.shape != (B, Hq, N):
        raise SwaError(-1, "bwd shape mismatch")
    _same(q, k=k, v=v, out=out, dout=dout)
    _buffer(lse, "lse", (B, Hq, N), torch.float32, q)
    _buffer(dq, "dq", q.shape, q.dtype, q)
    _buffer(dk, "dk", k.shape, k.dtype, q)
    _buffer(dv, "dv", v.shape, v.dtype, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    g, ng = None, 0
    if global_idx is not None and len(global_idx):
        g = (ctypes.c_int32 * len(global_idx))(*[int(x) for x in global_idx])
        ng = len(global_idx)
    need = bwd_workspace_size(B, Hq, Hkv, N, D, ng)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device:
        raise SwaError(-1, f"workspace must be on {q.device}")
    st = lib.swa_bwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                     _dev(lse, "lse"), _dev(dout, "dout"), _dev(dq, "dq"), _dev(dk, "dk"),
                     _dev(dv, "dv"), B, Hq, Hkv, N, D, win_left, win_right, dilation, g, ng,
                     float(scale), _dtype_code(q), _dev(workspace, "workspace"),
                     workspace.numel() * workspace.element_size(), _stream(q))
    _check(st, "swa_bwd")
    return dq, dk, dv
