"""The C-ABI library: it loads, exports every declared entry point, and rejects
bad arguments before anything is enqueued.  No GPU is needed: every call here
fails validation, so no HIP runtime call is made."""
import ctypes
import os
import re

import pytest

from sliding_window_attention_tiled_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")

OK, ARG, UNSUP, WS = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libswa.so is not built (python -m sliding_window_attention_tiled_amd.build)")
    return binding.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(swa_\w+)\s*\(", src)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ["swa_fwd", "swa_fwd_workspace_size", "swa_kv_append", "swa_decode",
              "swa_decode_workspace_size", "swa_status_string", "swa_version",
              "swa_kv_append_chunk", "swa_fwd_cached", "swa_decode_sinks",
              "swa_decode_sinks_workspace_size", "swa_kv_append_paged", "swa_decode_paged",
              "swa_bwd", "swa_bwd_workspace_size"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in swa.h but not exported"


def test_status_strings(lib):
    for st in (OK, ARG, UNSUP, WS, -4):
        assert lib.swa_status_string(st)
    assert lib.swa_status_string(12345) == b"unknown status"
    assert lib.swa_version() >= 100


def test_workspace_sizes(lib):
    assert lib.swa_fwd_workspace_size(1, 8, 1024, 128, 0) == 0
    a = lib.swa_fwd_workspace_size(2, 8, 8192, 64, 16)
    assert a > 0 and a % 16 == 0
    assert lib.swa_fwd_workspace_size(2, 8, 8192, 64, 32) == 2 * a
    assert lib.swa_fwd_workspace_size(2, 8, 8192, 96, 16) == 0      # unsupported D
    assert lib.swa_decode_workspace_size(64, 32, 4096, 128) > 0
    assert lib.swa_decode_workspace_size(0, 32, 4096, 128) == 0
    assert lib.swa_decode_workspace_size(1, 1, 1, 64) > 0


P = ctypes.c_void_p(256)  # stands in for a device pointer; never dereferenced


def fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, out=P, lse=None, B=1, Hq=4, Hkv=2, N=128, D=128, wl=7, wr=0,
             dil=1, g=None, ng=0, scale=0.1, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.swa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                       a["N"], a["D"], a["wl"], a["wr"], a["dil"], a["g"], a["ng"],
                       a["scale"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ARG), (dict(k=None), ARG), (dict(v=None), ARG), (dict(out=None), ARG),
    (dict(B=0), ARG), (dict(N=0), ARG), (dict(Hq=0), ARG), (dict(Hkv=0), ARG),
    (dict(N=(1 << 28) + 1), ARG),                                # above SWA_MAX_N
    (dict(Hq=6, Hkv=4), ARG), (dict(wl=-1), ARG), (dict(wr=-2), ARG), (dict(dil=0), ARG),
    (dict(ng=-1), ARG), (dict(ng=3), ARG),                       # NULL global_idx
    (dict(D=96), UNSUP), (dict(D=32), UNSUP), (dict(dtype=7), UNSUP),
])
def test_fwd_validation(lib, kw, status):
    assert fwd(lib, **kw) == status


def test_fwd_global_validation(lib):
    g = (ctypes.c_int32 * 3)(0, 5, 128)                           # 128 is out of range
    assert fwd(lib, g=g, ng=3) == ARG
    g = (ctypes.c_int32 * 3)(0, 5, -1)
    assert fwd(lib, g=g, ng=3) == ARG
    g = (ctypes.c_int32 * 3)(0, 5, 9)
    assert fwd(lib, g=g, ng=3) == WS                             # no workspace
    need = lib.swa_fwd_workspace_size(1, 4, 128, 128, 3)
    assert fwd(lib, g=g, ng=3, ws=P, wsb=need - 1) == WS         # too small
    big = (ctypes.c_int32 * 300)(*range(300))
    assert fwd(lib, N=1000, g=big, ng=300) == UNSUP              # > 256 distinct
    dup = (ctypes.c_int32 * 300)(*([3] * 300))                   # duplicates collapse
    assert fwd(lib, N=1000, g=dup, ng=300) == WS


def test_kv_append_validation(lib):
    f = lib.swa_kv_append
    assert f(None, P, P, P, P, P, 1, 1, 8, 128, 1, None) == ARG
    assert f(P, P, P, P, None, P, 1, 1, 8, 128, 1, None) == ARG
    assert f(P, P, P, P, P, P, 0, 1, 8, 128, 1, None) == ARG
    assert f(P, P, P, P, P, P, 1, 1, 0, 128, 1, None) == ARG
    assert f(P, P, P, P, P, P, 1, 1, 8, 100, 1, None) == UNSUP
    assert f(P, P, P, P, P, P, 1, 1, 8, 128, 5, None) == UNSUP


def test_decode_validation(lib):
    f = lib.swa_decode
    need = lib.swa_decode_workspace_size(2, 8, 64, 128)
    base = [P, P, P, P, P, P, None, 2, 8, 2, 64, 128, 0.1, P, need, 1, None]
    def call(**ch):
        a = list(base)
        names = ["q", "kc", "vc", "head", "len", "out", "lse", "B", "Hq", "Hkv", "W", "D",
                 "scale", "ws", "wsb", "dtype", "stream"]
        for k_, v_ in ch.items():
            a[names.index(k_)] = v_
        return f(*a)
    assert call(q=None) == ARG
    assert call(head=None) == ARG
    assert call(out=None) == ARG
    assert call(Hq=6, Hkv=4) == ARG
    assert call(W=0) == ARG
    assert call(D=80) == UNSUP
    assert call(dtype=3) == UNSUP
    assert call(ws=None) == WS
    assert call(wsb=need - 4) == WS
    # a grid beyond 2^31 - 1 workgroups is refused before any launch
    assert call(B=1 << 20, Hq=1 << 12, Hkv=1 << 12, wsb=(1 << 63)) == ARG


def test_python_binding_requires_device_tensors(lib):
    import torch
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(binding.SwaError):
        binding.fwd(q, q, q, win_left=3)


def test_kv_append_chunk_validation(lib):
    f = lib.swa_kv_append_chunk
    # (kcache, vcache, k, v, head, len, B, Hkv, W, n, D, dtype, stream)
    assert f(None, P, P, P, P, P, 1, 1, 8, 4, 128, 1, None) == ARG
    assert f(P, P, None, P, P, P, 1, 1, 8, 4, 128, 1, None) == ARG
    assert f(P, P, P, P, P, None, 1, 1, 8, 4, 128, 1, None) == ARG
    assert f(P, P, P, P, P, P, 1, 1, 8, -1, 128, 1, None) == ARG
    assert f(P, P, P, P, P, P, 1, 1, 0, 4, 128, 1, None) == ARG
    assert f(P, P, P, P, P, P, 1, 1, 8, (1 << 28) + 1, 128, 1, None) == ARG
    assert f(P, P, P, P, P, P, 1, 1, 8, 4, 96, 1, None) == UNSUP
    assert f(P, P, P, P, P, P, 1, 1, 8, 4, 128, 9, None) == UNSUP
    assert f(P, P, P, P, P, P, 1, 1, 8, 0, 128, 1, None) == OK     # nothing to append
    assert f(P, P, None, None, P, P, 1, 1, 8, 0, 128, 1, None) == OK


def test_fwd_cached_validation(lib):
    f = lib.swa_fwd_cached
    names = ["q", "k", "v", "kc", "vc", "head", "len", "out", "lse", "B", "Hq", "Hkv", "n",
             "W", "D", "wl", "scale", "dtype", "stream"]
    base = [P, P, P, P, P, P, P, P, None, 1, 8, 2, 64, 128, 128, 127, 0.1, 1, None]

    def call(**ch):
        a = list(base)
        for k_, v_ in ch.items():
            a[names.index(k_)] = v_
        return f(*a)
    for ptr in ("q", "k", "v", "kc", "vc", "head", "len", "out"):
        assert call(**{ptr: None}) == ARG, ptr
    assert call(B=0) == ARG
    assert call(n=0) == ARG
    assert call(W=0) == ARG
    assert call(Hq=6, Hkv=4) == ARG
    assert call(wl=-1) == ARG
    assert call(wl=129) == ARG                                    # window beyond the ring
    assert call(n=(1 << 28) + 1) == ARG
    assert call(D=80) == UNSUP
    assert call(dtype=2) == UNSUP


def test_decode_sinks_validation(lib):
    f = lib.swa_decode_sinks
    need = lib.swa_decode_sinks_workspace_size(2, 8, 64, 128, 4)
    assert need > lib.swa_decode_workspace_size(2, 8, 64, 128)      # one more split
    assert lib.swa_decode_sinks_workspace_size(2, 8, 64, 128, 0) == \
        lib.swa_decode_workspace_size(2, 8, 64, 128)
    assert lib.swa_decode_sinks_workspace_size(2, 8, 64, 128, -1) == 0
    names = ["q", "kc", "vc", "head", "len", "ks", "vs", "ns", "out", "lse", "B", "Hq", "Hkv",
             "W", "D", "scale", "ws", "wsb", "dtype", "stream"]
    base = [P, P, P, P, P, P, P, 4, P, None, 2, 8, 2, 64, 128, 0.1, P, need, 1, None]

    def call(**ch):
        a = list(base)
        for k_, v_ in ch.items():
            a[names.index(k_)] = v_
        return f(*a)
    assert call(ks=None) == ARG
    assert call(vs=None) == ARG
    assert call(ns=-1) == ARG
    assert call(ns=(1 << 28) + 1) == ARG
    assert call(q=None) == ARG
    assert call(Hq=6, Hkv=4) == ARG
    assert call(D=80) == UNSUP
    assert call(wsb=need - 4) == WS
    assert call(ws=None) == WS


def test_paged_validation(lib):
    fa = lib.swa_kv_append_paged
    # (kpool, vpool, k, v, table, seq, B, Hkv, n_pages, P, nb, W, n, D, dtype, stream)
    ok = [P, P, P, P, P, P, 2, 2, 16, 16, 8, 100, 3, 128, 1, None]

    def app(**ch):
        names = ["kp", "vp", "k", "v", "bt", "sl", "B", "Hkv", "np", "P", "nb", "W", "n", "D",
                 "dt", "st"]
        a = list(ok)
        for k_, v_ in ch.items():
            a[names.index(k_)] = v_
        return fa(*a)
    assert app(kp=None) == ARG and app(bt=None) == ARG and app(sl=None) == ARG
    assert app(k=None) == ARG
    assert app(k=None, v=None, n=0) == OK
    assert app(P=24) == ARG                       # not a power of two
    assert app(nb=7) == ARG                       # 7 * 16 < 100 + 15
    assert app(nb=8, W=114) == ARG                # 8 * 16 < 114 + 15
    assert app(n=-1) == ARG and app(np=0) == ARG
    assert app(D=96) == UNSUP and app(dt=4) == UNSUP
    fd = lib.swa_decode_paged
    need = lib.swa_decode_workspace_size(2, 8, 100, 128)
    okd = [P, P, P, P, P, P, None, 2, 8, 2, 16, 16, 8, 100, 128, 0.1, P, need, 1, None]

    def dec(**ch):
        names = ["q", "kp", "vp", "bt", "sl", "out", "lse", "B", "Hq", "Hkv", "np", "P", "nb",
                 "W", "D", "scale", "ws", "wsb", "dt", "st"]
        a = list(okd)
        for k_, v_ in ch.items():
            a[names.index(k_)] = v_
        return fd(*a)
    assert dec(q=None) == ARG and dec(bt=None) == ARG and dec(out=None) == ARG
    assert dec(Hq=6, Hkv=4) == ARG and dec(P=12) == ARG and dec(nb=7) == ARG
    assert dec(D=80) == UNSUP
    assert dec(ws=None) == WS and dec(wsb=need - 1) == WS


def test_bwd_validation(lib):
    f = lib.swa_bwd
    names = ["q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv", "B", "Hq", "Hkv", "N", "D",
             "wl", "wr", "dil", "g", "ng", "scale", "dtype", "ws", "wsb", "stream"]
    need = lib.swa_bwd_workspace_size(1, 4, 2, 128, 128, 0)
    assert need >= 4 * 128 * 4 and lib.swa_bwd_workspace_size(1, 4, 2, 128, 96, 0) == 0
    assert lib.swa_bwd_workspace_size(1, 4, 2, 128, 128, -1) == 0
    # global tokens add float32 accumulators of their rows (dq) and keys (dk, dv)
    need_g = lib.swa_bwd_workspace_size(1, 4, 2, 128, 128, 2)
    assert need_g >= need + (4 * 2 * 128 + 2 * 2 * 2 * 128) * 4
    base = [P, P, P, P, P, P, P, P, P, 1, 4, 2, 128, 128, 7, 0, 1, None, 0, 0.1, 1, P, need,
            None]

    def call(**ch):
        a = list(base)
        for k_, v_ in ch.items():
            a[names.index(k_)] = v_
        return f(*a)
    for ptr in ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv"):
        assert call(**{ptr: None}) == ARG, ptr
    assert call(Hq=6, Hkv=4) == ARG and call(wl=-1) == ARG and call(dil=0) == ARG
    assert call(N=(1 << 28) + 1) == ARG
    assert call(D=80) == UNSUP and call(dtype=5) == UNSUP
    # global tokens: checked (and the workspace sized) before any launch
    assert call(g=(ctypes.c_int32 * 2)(0, 128), ng=2) == ARG        # position >= N
    assert call(g=None, ng=2) == ARG and call(ng=-1) == ARG
    many = (ctypes.c_int32 * 300)(*range(300))
    assert call(N=1024, g=many, ng=300) == UNSUP                     # > 256 distinct
    assert call(g=(ctypes.c_int32 * 2)(0, 5), ng=2) == WS            # no room for them
    assert call(ws=None) == WS and call(wsb=need - 1) == WS


BAD_SCALES = [0.0, -0.0, -0.125, float("nan"), float("inf"), float("-inf"), 3.0e38]


@pytest.mark.parametrize("scale", BAD_SCALES)
def test_scale_must_be_positive_and_finite(lib, scale):
    """The kernels mask keys with -inf on the raw scores and take the running
    max before multiplying by scale * log2(e), so every entry point that takes
    a scale refuses one that is not positive and finite (3e38 * log2(e)
    overflows float32).  The D = 80 calls show the order: a good scale passes
    on to the head-dimension check (SWA_ERR_UNSUPPORTED), a bad one stops at
    SWA_ERR_ARG before it."""
    F = ctypes.c_float
    assert fwd(lib, scale=scale) == ARG
    assert fwd(lib, scale=scale, D=80) == ARG and fwd(lib, scale=0.1, D=80) == UNSUP
    cached = lambda s, D: lib.swa_fwd_cached(P, P, P, P, P, P, P, P, None, 1, 8, 2, 64, 128,
                                             D, 127, F(s), 1, None)
    assert cached(scale, 128) == ARG and cached(scale, 80) == ARG and cached(0.1, 80) == UNSUP
    need = lib.swa_decode_workspace_size(2, 8, 64, 128)
    dec = lambda s, D: lib.swa_decode(P, P, P, P, P, P, None, 2, 8, 2, 64, D, F(s), P, need, 1,
                                      None)
    assert dec(scale, 128) == ARG and dec(scale, 80) == ARG and dec(0.1, 80) == UNSUP
    sinks = lambda s, D: lib.swa_decode_sinks(P, P, P, P, P, P, P, 4, P, None, 2, 8, 2, 64, D,
                                              F(s), P, 1 << 30, 1, None)
    assert sinks(scale, 128) == ARG and sinks(0.1, 80) == UNSUP
    need_p = lib.swa_decode_workspace_size(2, 8, 100, 128)
    paged = lambda s, D: lib.swa_decode_paged(P, P, P, P, P, P, None, 2, 8, 2, 16, 16, 8, 100,
                                              D, F(s), P, need_p, 1, None)
    assert paged(scale, 128) == ARG and paged(0.1, 80) == UNSUP
    need_b = lib.swa_bwd_workspace_size(1, 4, 2, 128, 128, 0)
    bwd = lambda s, D: lib.swa_bwd(P, P, P, P, P, P, P, P, P, 1, 4, 2, 128, D, 7, 0, 1, None, 0,
                                   F(s), 1, P, need_b, None)
    assert bwd(scale, 128) == ARG and bwd(0.1, 80) == UNSUP


def test_binding_checks_buffers_before_any_launch(lib):
    """Caller-supplied buffers of the wrong shape or dtype, and inputs whose
    dtypes disagree, raise SwaError naming the tensor before anything reaches
    the C ABI (these are host tensors: the shape checks come before the device
    check, which would otherwise be the error)."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros(1, 16, 4, 64, dtype=bf)
    k = torch.zeros(1, 16, 2, 64, dtype=bf)

    def raises(fn, name):
        with pytest.raises(binding.SwaError) as e:
            fn()
        assert f"{name} must be" in str(e.value), str(e.value)

    raises(lambda: binding.fwd(q, k, k, win_left=3, out=torch.zeros(1, 16, 4, 32, dtype=bf)),
           "out")
    raises(lambda: binding.fwd(q, k, k, win_left=3, out=torch.zeros(1, 16, 4, 64, dtype=f32)),
           "out")
    raises(lambda: binding.fwd(q, k, k, win_left=3, lse=torch.zeros(1, 4, 15)), "lse")
    raises(lambda: binding.fwd(q, k, k.float(), win_left=3), "v")
    # decode: an fp32 query over a bf16 ring would read past the ring
    kc = torch.zeros(2, 2, 32, 64, dtype=bf)
    qd = torch.zeros(2, 4, 64, dtype=bf)
    head = torch.zeros(2, dtype=torch.int32)
    raises(lambda: binding.decode(qd.float(), kc, kc, head, head), "kcache")
    raises(lambda: binding.decode(qd, kc, kc, head.long(), head), "ring_head")
    raises(lambda: binding.decode(qd, kc, kc, head, head[:1]), "cache_len")
    raises(lambda: binding.decode(qd, kc, kc, head, head, out=torch.zeros(2, 4, 32, dtype=bf)),
           "out")
    raises(lambda: binding.decode(qd, kc, kc, head, head, lse=torch.zeros(2, 5)), "lse")
    kn = torch.zeros(2, 2, 64, dtype=bf)
    raises(lambda: binding.kv_append(kc, kc, kn.float(), kn, head, head), "k_new")
    raises(lambda: binding.kv_append(kc, kc.float(), kn, kn, head, head), "vcache")
    ks = torch.zeros(2, 2, 4, 64, dtype=bf)
    raises(lambda: binding.decode_sinks(qd, kc, kc, head, head, ks, ks.float()), "vsink")
    raises(lambda: binding.decode_sinks(qd, kc, kc, head, head, ks, ks,
                                        out=torch.zeros(3, 4, 64, dtype=bf)), "out")
    qc = torch.zeros(2, 8, 4, 64, dtype=bf)
    kch = torch.zeros(2, 8, 2, 64, dtype=bf)
    raises(lambda: binding.fwd_cached(qc, kch, kch, kc, kc, head, head, win_left=4,
                                      lse=torch.zeros(2, 4, 9)), "lse")
    pool = torch.zeros(8, 2, 16, 64, dtype=bf)
    table = torch.zeros(2, 4, dtype=torch.int32)
    raises(lambda: binding.decode_paged(qd, pool, pool, table, head, window=32,
                                        out=torch.zeros(2, 4, 64, dtype=f32)), "out")
    raises(lambda: binding.decode_paged(qd.float(), pool, pool, table, head, window=32),
           "kpool")
    raises(lambda: binding.kv_append_paged(pool, pool, kch, kch.float(), table, head, window=32),
           "v")
    out = torch.zeros_like(q)
    lse = torch.zeros(1, 4, 16)
    raises(lambda: binding.bwd(q, k, k, out, lse, out, win_left=3,
                               dk=torch.zeros(1, 16, 4, 64, dtype=bf)), "dk")
    raises(lambda: binding.bwd(q, k, k, out, lse, out, win_left=3,
                               dq=torch.zeros(1, 16, 4, 64, dtype=f32)), "dq")
    with pytest.raises(binding.SwaError, match="bwd shape mismatch"):
        binding.bwd(q, k, k, out, lse[:, :, :8], out, win_left=3)
    raises(lambda: binding.bwd(q, k, k, out, lse.double(), out, win_left=3), "lse")
    raises(lambda: binding.bwd(q, k, k, out, lse, out.float(), win_left=3), "dout")
