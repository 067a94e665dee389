"""fp64 CPU oracle for sliding-window attention (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and
shares no code with it.

``swa_oracle.c`` holds the arithmetic (see its header for the definition and
the passages it follows); this module only builds it with gcc and marshals
numpy arrays into it.  ``bruteforce.py`` holds a second, independent dense-mask
formulation used to pin the C oracle on tiny inputs.

Inputs are passed as numpy arrays: float32, or bfloat16 given as raw uint16
bit patterns (the oracle widens both to double exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swa_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "libswa_oracle.so")

DT_F32 = 0
DT_BF16 = 1


_LIB_NATIVE = os.path.join(_LIB_DIR, "libswa_oracle_native.so")


def build(force: bool = True, src: str = _SRC, out: str = _LIB, native: bool = False) -> str:
    """Compile the oracle C source into a shared library with gcc (OpenMP, -O3).

    native=True adds -march=native: code for the CPU this runs on, which is
    only safe to load on that machine (the CPU-baseline timing builds such a
    copy where it runs; the default copy stays portable)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    if force or not os.path.exists(out):
        tmp = out + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O3", *(["-march=native"] if native else []), "-fopenmp", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def host_info() -> dict:
    """The host the oracle runs on: logical CPUs, the CPUs this process may
    use, and the CPU model name."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x: np.ndarray) -> tuple[np.ndarray, int]:
    """float32 -> (array, DT_F32); uint16 bf16 bit patterns -> (array, DT_BF16)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, DT_F32
    if x.dtype == np.uint16:
        return x, DT_BF16
    raise TypeError(f"oracle inputs must be float32 or bf16 bits (uint16), got {x.dtype}")


def _globals(global_idx) -> tuple[np.ndarray, int]:
    if global_idx is None:
        return np.zeros(1, np.int32), 0
    g = np.ascontiguousarray(np.asarray(global_idx, dtype=np.int32).reshape(-1))
    return (g if g.size else np.zeros(1, np.int32)), int(g.size)


class OracleLib:
    """One compiled copy of the oracle (the default one, or a test's variant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_attended_set.argtypes = [I64, I64, I64, I64, I64, P, I64, P]
        lib.oracle_attended_set.restype = I64
        lib.oracle_fwd_rows.argtypes = [P, P, P, I, I64, I64, I64, I64, I64, I64, I64, I64,
                                        P, I64, D, P, I64, P, P]
        lib.oracle_fwd_rows.restype = I
        lib.oracle_fwd.argtypes = [P, P, P, I, I64, I64, I64, I64, I64, I64, I64, I64,
                                   P, I64, D, P, P]
        lib.oracle_fwd.restype = I
        lib.oracle_kv_append.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I]
        lib.oracle_kv_append.restype = I
        lib.oracle_decode.argtypes = [P, P, P, I, P, P, I64, I64, I64, I64, I64, D, P, P]
        lib.oracle_decode.restype = I
        lib.oracle_kv_append_chunk.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I]
        lib.oracle_kv_append_chunk.restype = I
        lib.oracle_fwd_cached.argtypes = [P, P, P, P, P, I, P, P, I64, I64, I64, I64, I64, I64,
                                          I64, D, P, P]
        lib.oracle_fwd_cached.restype = I
        lib.oracle_decode_sinks.argtypes = [P, P, P, P, P, I64, I, P, P, I64, I64, I64, I64,
                                            I64, D, P, P]
        lib.oracle_decode_sinks.restype = I
        lib.oracle_kv_append_paged.argtypes = [P, P, P, P, P, I64, I64, I64, P, I64, I64, I64,
                                               I64, I64, I]
        lib.oracle_kv_append_paged.restype = I
        lib.oracle_decode_paged.argtypes = [P, P, P, I, P, I64, I64, I64, P, I64, I64, I64, I64,
                                            I64, D, P, P]
        lib.oracle_decode_paged.restype = I
        lib.oracle_bwd.argtypes = [P, P, P, P, I, I64, I64, I64, I64, I64, I64, I64, I64, P,
                                   I64, D, P, P, P]
        lib.oracle_bwd.restype = I
        lib.oracle_bwd_dq_rows.argtypes = [P, P, P, P, I, I64, I64, I64, I64, I64, I64, I64,
                                           I64, P, I64, D, P, I64, P]
        lib.oracle_bwd_dq_rows.restype = I
        lib.oracle_bwd_dkv_keys.argtypes = [P, P, P, P, I, I64, I64, I64, I64, I64, I64, I64,
                                            I64, P, I64, D, P, I64, P, P]
        lib.oracle_bwd_dkv_keys.restype = I
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def attended_set(self, i: int, N: int, win_left: int, win_right: int,
                     dilation: int = 1, global_idx=None) -> list:
        """S(i) as a sorted list of key positions."""
        g, ng = _globals(global_idx)
        buf = np.zeros(N + win_left + win_right + ng + 1, np.int64)
        n = self.lib.oracle_attended_set(i, N, win_left, win_right, dilation, _ptr(g), ng,
                                         _ptr(buf))
        if n < 0:
            raise ValueError("invalid arguments to oracle_attended_set")
        return buf[:n].tolist()

    def fwd(self, q, k, v, *, win_left: int, win_right: int = 0, dilation: int = 1,
            global_idx=None, scale=None):
        """All rows.  q [B,N,Hq,D], k/v [B,N,Hkv,D] -> (out [B,N,Hq,D], lse [B,Hq,N])."""
        q, dt = _as_input(q)
        k, dtk = _as_input(k)
        v, dtv = _as_input(v)
        if not dt == dtk == dtv:
            raise TypeError("q, k and v must share one element type")
        B, N, Hq, D = q.shape
        Hkv = k.shape[2]
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        g, ng = _globals(global_idx)
        out = np.zeros((B, N, Hq, D), np.float64)
        lse = np.zeros((B, Hq, N), np.float64)
        rc = self.lib.oracle_fwd(_ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, N, D,
                                 win_left, win_right, dilation, _ptr(g), ng, float(scale),
                                 _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError("invalid arguments to oracle_fwd")
        return out, lse

    def fwd_rows(self, q, k, v, rows, *, win_left: int, win_right: int = 0,
                 dilation: int = 1, global_idx=None, scale=None):
        """Selected rows: rows is an [R,3] int array of (b, h, i).
        Returns (out [R,D], lse [R])."""
        q, dt = _as_input(q)
        k, _ = _as_input(k)
        v, _ = _as_input(v)
        B, N, Hq, D = q.shape
        Hkv = k.shape[2]
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        g, ng = _globals(global_idx)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        out = np.zeros((rows.shape[0], D), np.float64)
        lse = np.zeros(rows.shape[0], np.float64)
        rc = self.lib.oracle_fwd_rows(_ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, N, D,
                                      win_left, win_right, dilation, _ptr(g), ng,
                                      float(scale), _ptr(rows), rows.shape[0], _ptr(out),
                                      _ptr(lse))
        if rc != 0:
            raise ValueError("invalid arguments to oracle_fwd_rows")
        return out, lse

    def bwd(self, q, k, v, dout, *, win_left: int, win_right: int = 0, dilation: int = 1,
            global_idx=None, scale=None):
        """Gradients (dq [B,N,Hq,D], dk, dv [B,N,Hkv,D]) in float64 for the upstream
        gradient dout [B,N,Hq,D] of the forward with the same arguments."""
        q, dt = _as_input(q)
        k, _ = _as_input(k)
        v, _ = _as_input(v)
        dout, dt2 = _as_input(dout)
        if dt2 != dt:
            raise TypeError("dout must have the element type of q")
        B, N, Hq, D = q.shape
        Hkv = k.shape[2]
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        g, ng = _globals(global_idx)
        dq = np.zeros((B, N, Hq, D), np.float64)
        dk = np.zeros((B, N, Hkv, D), np.float64)
        dv = np.zeros((B, N, Hkv, D), np.float64)
        rc = self.lib.oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), dt, B, Hq, Hkv, N, D,
                                 win_left, win_right, dilation, _ptr(g), ng, float(scale),
                                 _ptr(dq), _ptr(dk), _ptr(dv))
        if rc != 0:
            raise ValueError("invalid arguments to oracle_bwd")
        return dq, dk, dv

    def _bwd_args(self, q, k, v, dout, scale, global_idx):
        q, dt = _as_input(q)
        k, _ = _as_input(k)
        v, _ = _as_input(v)
        dout, _ = _as_input(dout)
        B, N, Hq, D = q.shape
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        g, ng = _globals(global_idx)
        return q, k, v, dout, dt, B, N, Hq, k.shape[2], D, float(scale), g, ng

    def bwd_dq_rows(self, q, k, v, dout, rows, *, win_left: int, win_right: int = 0,
                    dilation: int = 1, global_idx=None, scale=None):
        """dq of the rows (b, h, i) listed in rows [R,3] -> [R,D] float64."""
        q, k, v, dout, dt, B, N, Hq, Hkv, D, scale, g, ng = self._bwd_args(
            q, k, v, dout, scale, global_idx)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        out = np.zeros((rows.shape[0], D), np.float64)
        rc = self.lib.oracle_bwd_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), dt, B, Hq, Hkv,
                                         N, D, win_left, win_right, dilation, _ptr(g), ng, scale,
                                         _ptr(rows), rows.shape[0], _ptr(out))
        if rc != 0:
            raise ValueError("invalid arguments to oracle_bwd_dq_rows")
        return out

    def bwd_dkv_keys(self, q, k, v, dout, keys, *, win_left: int, win_right: int = 0,
                     dilation: int = 1, global_idx=None, scale=None):
        """(dk, dv) of the keys (b, kv head, j) listed in keys [R,3] -> two [R,D]."""
        q, k, v, dout, dt, B, N, Hq, Hkv, D, scale, g, ng = self._bwd_args(
            q, k, v, dout, scale, global_idx)
        keys = np.ascontiguousarray(np.asarray(keys, dtype=np.int64).reshape(-1, 3))
        dk = np.zeros((keys.shape[0], D), np.float64)
        dv = np.zeros((keys.shape[0], D), np.float64)
        rc = self.lib.oracle_bwd_dkv_keys(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), dt, B, Hq, Hkv,
                                          N, D, win_left, win_right, dilation, _ptr(g), ng,
                                          scale, _ptr(keys), keys.shape[0], _ptr(dk), _ptr(dv))
        if rc != 0:
            raise ValueError("invalid arguments to oracle_bwd_dkv_keys")
        return dk, dv

    def ring(self, kcache, vcache, ring_head, cache_len) -> "Ring":
        return Ring(self, kcache, vcache, ring_head, cache_len)

    def paged(self, kpool, vpool, seq_len, W: int) -> "PagedCache":
        return PagedCache(self, kpool, vpool, seq_len, W)


class Ring:
    """The oracle's own copy of a ring-buffer KV cache.

    kcache/vcache [B,Hkv,W,D] (float32 or bf16 bits), ring_head/cache_len [B].
    """

    def __init__(self, orc: OracleLib, kcache, vcache, ring_head, cache_len):
        self.orc = orc
        self.k, self.dtype = _as_input(np.array(kcache, copy=True))
        self.v, _ = _as_input(np.array(vcache, copy=True))
        self.head = np.ascontiguousarray(np.asarray(ring_head, dtype=np.int64).copy())
        self.len = np.ascontiguousarray(np.asarray(cache_len, dtype=np.int64).copy())
        self.B, self.Hkv, self.W, self.D = self.k.shape

    def append(self, k_new, v_new):
        k_new, _ = _as_input(k_new)
        v_new, _ = _as_input(v_new)
        rc = self.orc.lib.oracle_kv_append(_ptr(self.k), _ptr(self.v), _ptr(k_new),
                                           _ptr(v_new), _ptr(self.head), _ptr(self.len),
                                           self.B, self.Hkv, self.W, self.D, self.dtype)
        if rc != 0:
            raise ValueError("invalid arguments to oracle_kv_append")

    def append_chunk(self, k, v):
        """Appends a chunk k, v [B,n,Hkv,D] (n single appends in token order)."""
        k, _ = _as_input(k)
        v, _ = _as_input(v)
        n = k.shape[1]
        rc = self.orc.lib.oracle_kv_append_chunk(_ptr(self.k), _ptr(self.v), _ptr(k), _ptr(v),
                                                 _ptr(self.head), _ptr(self.len), self.B,
                                                 self.Hkv, self.W, n, self.D, self.dtype)
        if rc != 0:
            raise ValueError("invalid arguments to oracle_kv_append_chunk")

    def fwd_cached(self, q, k, v, *, win_left: int, scale=None):
        """Causal window attention of a prompt chunk q [B,n,Hq,D], k/v [B,n,Hkv,D]
        that follows the tokens held in this ring.  The ring is not modified.
        Returns (out [B,n,Hq,D], lse [B,Hq,n]) fp64."""
        q, _ = _as_input(q)
        k, _ = _as_input(k)
        v, _ = _as_input(v)
        B, n, Hq, D = q.shape
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        out = np.zeros((B, n, Hq, D), np.float64)
        lse = np.zeros((B, Hq, n), np.float64)
        rc = self.orc.lib.oracle_fwd_cached(_ptr(q), _ptr(k), _ptr(v), _ptr(self.k),
                                            _ptr(self.v), self.dtype, _ptr(self.head),
                                            _ptr(self.len), B, Hq, self.Hkv, n, self.W, D,
                                            win_left, float(scale), _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError("invalid arguments to oracle_fwd_cached")
        return out, lse

    def decode(self, q, scale=None, sinks=None):
        """q [B,Hq,D] -> (out [B,Hq,D], lse [B,Hq]) fp64.  sinks = (ksink, vsink)
        [B,Hkv,S,D]: pinned entries attended in addition to the ring."""
        q, _ = _as_input(q)
        B, Hq, D = q.shape
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        out = np.zeros((B, Hq, D), np.float64)
        lse = np.zeros((B, Hq), np.float64)
        if sinks is not None:
            ks, _ = _as_input(sinks[0])
            vs, _ = _as_input(sinks[1])
            rc = self.orc.lib.oracle_decode_sinks(_ptr(q), _ptr(self.k), _ptr(self.v), _ptr(ks),
                                                  _ptr(vs), ks.shape[2], self.dtype,
                                                  _ptr(self.head), _ptr(self.len), B, Hq,
                                                  self.Hkv, self.W, D, float(scale), _ptr(out),
                                                  _ptr(lse))
            if rc != 0:
                raise ValueError("invalid arguments to oracle_decode_sinks")
            return out, lse
        rc = self.orc.lib.oracle_decode(_ptr(q), _ptr(self.k), _ptr(self.v), self.dtype,
                                        _ptr(self.head), _ptr(self.len), B, Hq, self.Hkv,
                                        self.W, D, float(scale), _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError("invalid arguments to oracle_decode")
        return out, lse


class PagedCache:
    """The oracle's copy of a paged window cache: page pool kpool/vpool
    [n_pages,Hkv,P,D], per-sequence token counts seq_len [B] and window W.
    The block table [B,nb] (int32) is passed to each call."""

    def __init__(self, orc: OracleLib, kpool, vpool, seq_len, W: int):
        self.orc = orc
        self.k, self.dtype = _as_input(np.array(kpool, copy=True))
        self.v, _ = _as_input(np.array(vpool, copy=True))
        self.len = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int64).copy())
        self.n_pages, self.Hkv, self.P, self.D = self.k.shape
        self.W = W

    def append(self, k, v, block_table):
        """k, v [B,n,Hkv,D]."""
        k, _ = _as_input(k)
        v, _ = _as_input(v)
        bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
        B, n = k.shape[0], k.shape[1]
        rc = self.orc.lib.oracle_kv_append_paged(_ptr(self.k), _ptr(self.v), _ptr(k), _ptr(v),
                                                 _ptr(bt), bt.shape[1], self.P, self.n_pages,
                                                 _ptr(self.len), B, self.Hkv, self.W, n, self.D,
                                                 self.dtype)
        if rc != 0:
            raise ValueError("invalid arguments to oracle_kv_append_paged")

    def decode(self, q, block_table, scale=None):
        q, _ = _as_input(q)
        bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
        B, Hq, D = q.shape
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        out = np.zeros((B, Hq, D), np.float64)
        lse = np.zeros((B, Hq), np.float64)
        rc = self.orc.lib.oracle_decode_paged(_ptr(q), _ptr(self.k), _ptr(self.v), self.dtype,
                                              _ptr(bt), bt.shape[1], self.P, self.n_pages,
                                              _ptr(self.len), B, Hq, self.Hkv, self.W, D,
                                              float(scale), _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError("invalid arguments to oracle_decode_paged")
        return out, lse


_default = None


def default() -> OracleLib:
    """The oracle built from swa_oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _default = OracleLib(_LIB)
    return _default


_native = None


def native() -> OracleLib:
    """A copy of the oracle built here with -march=native (rebuilt once per
    process, for the machine it runs on).  Same source, same arithmetic: used
    to time the oracle as a CPU baseline."""
    global _native
    if _native is None:
        build(force=True, out=_LIB_NATIVE, native=True)
        _native = OracleLib(_LIB_NATIVE)
    return _native


def num_threads() -> int:
    return default().num_threads()


def attended_set(*a, **kw):
    return default().attended_set(*a, **kw)


def fwd(*a, **kw):
    return default().fwd(*a, **kw)


def fwd_rows(*a, **kw):
    return default().fwd_rows(*a, **kw)


def bwd(*a, **kw):
    return default().bwd(*a, **kw)


def bwd_dq_rows(*a, **kw):
    return default().bwd_dq_rows(*a, **kw)


def bwd_dkv_keys(*a, **kw):
    return default().bwd_dkv_keys(*a, **kw)


def ring(*a, **kw) -> Ring:
    return default().ring(*a, **kw)


def paged(*a, **kw) -> PagedCache:
    return default().paged(*a, **kw)
