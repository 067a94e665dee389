"""The debug build (libswa_debug.so, every source compiled with SWA_DEBUG).

In that build the kernels count failed index checks (global rows, ring slots,
sink entries, LDS tile offsets, and the device-side ring and page state they
are handed) instead of faulting, and extra workgroup barriers plus immediate
waits on every tile copy run the phases that the release kernels overlap one
after another.  The GPU tests run each entry point through both libraries on
the same seeded inputs and require

  * outputs identical bit for bit: the release kernels' overlap of loads,
    LDS writes and reads gives the same result as the serialised order (a
    missing wait or barrier would show up as a difference), and
  * no failed check.

A positive control shows that the counter sees a broken contract: a
cache_len above the ring size handed to the ring append (a value the kernel
clamps and uses for nothing but the clamped length)."""
import ctypes
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sliding_window_attention_tiled_amd import binding  # noqa: E402
from sliding_window_attention_tiled_amd import build as swa_build  # noqa: E402
from tests.gpu_util import log  # noqa: E402

SWA_ERR_UNSUPPORTED = -2


def _exports(path):
    r = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                       check=True)
    return {ln.split()[-1] for ln in r.stdout.splitlines() if ln.split()[-1].startswith("swa_")}


# ---- CPU ------------------------------------------------------------------------------

def test_debug_library_exports_the_release_abi():
    if not os.path.exists(swa_build.DEBUG_LIB):
        swa_build.build_debug()
    rel, dbg = _exports(binding.LIB_PATH), _exports(swa_build.DEBUG_LIB)
    assert "swa_debug_violations" in rel
    assert rel == dbg, rel ^ dbg


def test_release_counter_query_is_unsupported():
    lib = ctypes.CDLL(binding.LIB_PATH)
    lib.swa_debug_violations.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
    lib.swa_debug_violations.restype = ctypes.c_int
    n = ctypes.c_ulonglong(12345)
    assert lib.swa_debug_violations(ctypes.byref(n), 1) == SWA_ERR_UNSUPPORTED
    assert n.value == 12345


# ---- GPU ------------------------------------------------------------------------------

def _randn(gen, *shape, dtype=torch.bfloat16):
    return torch.randn(*shape, generator=gen).to(dtype).to("cuda")


def _fwd_case(seed, B, Hq, Hkv, N, D, wl, wr=0, dil=1, glob=None, dtype=torch.bfloat16):
    def run():
        g = torch.Generator().manual_seed(seed)
        q, k, v = (_randn(g, B, N, h, D, dtype=dtype) for h in (Hq, Hkv, Hkv))
        out, lse = binding.fwd(q, k, v, win_left=wl, win_right=wr, dilation=dil,
                               global_idx=glob)
        return [out, lse]
    return run


def _bwd_case(seed, B, Hq, Hkv, N, D, wl, wr=0, dil=1, glob=None):
    def run():
        g = torch.Generator().manual_seed(seed)
        q, k, v = (_randn(g, B, N, h, D) for h in (Hq, Hkv, Hkv))
        dout = _randn(g, B, N, Hq, D)
        out, lse = binding.fwd(q, k, v, win_left=wl, win_right=wr, dilation=dil,
                               global_idx=glob)
        dq, dk, dv = binding.bwd(q, k, v, out, lse, dout, win_left=wl, win_right=wr,
                                 dilation=dil, global_idx=glob)
        return [out, lse, dq, dk, dv]
    return run


def _ring(B, Hkv, W, D, dtype=torch.bfloat16):
    kc = torch.zeros(B, Hkv, W, D, dtype=dtype, device="cuda")
    vc = torch.zeros_like(kc)
    head = torch.zeros(B, dtype=torch.int32, device="cuda")
    length = torch.zeros(B, dtype=torch.int32, device="cuda")
    return kc, vc, head, length


def _prefill_case(seed, B, Hq, Hkv, D, W, n_before, chunk):
    def run():
        g = torch.Generator().manual_seed(seed)
        kc, vc, head, length = _ring(B, Hkv, W, D)
        k0, v0 = _randn(g, B, n_before, Hkv, D), _randn(g, B, n_before, Hkv, D)
        binding.kv_append_chunk(kc, vc, k0, v0, head, length)
        q, k, v = _randn(g, B, chunk, Hq, D), _randn(g, B, chunk, Hkv, D), \
            _randn(g, B, chunk, Hkv, D)
        out, lse = binding.fwd_cached(q, k, v, kc, vc, head, length, win_left=W - 1)
        return [out, lse, kc, vc, head, length]
    return run


def _decode_case(seed, B, Hq, Hkv, D, W, steps, n_sink=0):
    def run():
        g = torch.Generator().manual_seed(seed)
        kc, vc, head, length = _ring(B, Hkv, W, D)
        k0, v0 = _randn(g, B, W - 3, Hkv, D), _randn(g, B, W - 3, Hkv, D)
        binding.kv_append_chunk(kc, vc, k0, v0, head, length)
        if n_sink:
            ks, vs = _randn(g, B, Hkv, n_sink, D), _randn(g, B, Hkv, n_sink, D)
        res = []
        for _ in range(steps):   # the ring fills and wraps during the steps
            binding.kv_append(kc, vc, _randn(g, B, Hkv, D), _randn(g, B, Hkv, D), head, length)
            q = _randn(g, B, Hq, D)
            if n_sink:
                res += list(binding.decode_sinks(q, kc, vc, head, length, ks, vs))
            else:
                res += list(binding.decode(q, kc, vc, head, length))
        return res + [kc, vc, head, length]
    return run


def _paged_case(seed, B, Hq, Hkv, D, W, P, n_tok):
    def run():
        g = torch.Generator().manual_seed(seed)
        nb = -(-(W + P - 1) // P)
        n_pages = B * nb + 3
        perm = torch.randperm(n_pages, generator=g)[:B * nb].to(torch.int32)
        table = perm.reshape(B, nb).contiguous().to("cuda")
        kp = torch.zeros(n_pages, Hkv, P, D, dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        seq = torch.zeros(B, dtype=torch.int32, device="cuda")
        k, v = _randn(g, B, n_tok, Hkv, D), _randn(g, B, n_tok, Hkv, D)
        binding.kv_append_paged(kp, vp, k, v, table, seq, window=W)
        out, lse = binding.decode_paged(_randn(g, B, Hq, D), kp, vp, table, seq, window=W)
        return [out, lse, kp, vp, seq]
    return run


CASES = [
    # two-group forward (D = 128, four query heads per K/V head)
    ("fwd_pp_causal", _fwd_case(1, 1, 8, 2, 1100, 128, 300)),
    ("fwd_pp_dilated2_bidir", _fwd_case(2, 1, 8, 2, 650, 128, 30, 17, 2)),
    ("fwd_pp_window_ge_n", _fwd_case(3, 2, 4, 1, 300, 128, 1000, 1000)),
    # single-phase forward: two heads per K/V head, D = 64 with global tokens
    ("fwd_hpw2_causal", _fwd_case(4, 1, 4, 2, 900, 128, 200)),
    ("fwd_d64_globals", _fwd_case(5, 1, 4, 4, 1500, 64, 256, 256, 1,
                                  [0, 7, 100, 511, 512, 900, 1499])),
    ("fwd_d64_dilated_globals", _fwd_case(6, 1, 4, 2, 1000, 64, 40, 40, 3, [2, 3, 500])),
    ("fwd_f32", _fwd_case(7, 1, 4, 2, 400, 64, 70, 0, 1, None, torch.float32)),
    # chunked prefill over a ring, ring appends, decode (plain, sinks, paged)
    ("prefill_ring", _prefill_case(8, 2, 8, 2, 128, 256, 300, 100)),
    ("decode_ring", _decode_case(9, 3, 8, 2, 128, 512, 6)),
    ("decode_sinks", _decode_case(10, 2, 8, 2, 128, 256, 4, n_sink=4)),
    ("decode_paged", _paged_case(11, 3, 8, 2, 128, 256, 64, 300)),
    # backward: band only (D = 128) and with global tokens (D = 64)
    ("bwd_causal", _bwd_case(12, 1, 8, 2, 700, 128, 200)),
    ("bwd_bidir_dilated", _bwd_case(13, 1, 4, 2, 600, 64, 33, 20, 2)),
    ("bwd_globals", _bwd_case(14, 1, 4, 4, 800, 64, 128, 128, 1, [0, 5, 400, 799])),
]


# The seeded random shapes of the parity suite (GQA 1-8, asymmetric and
# degenerate windows, dilation, duplicate global tokens, both head dimensions
# and dtypes; ring sizes, fills and sink counts for decode and the chunked
# prefill) through both builds as well.
from sliding_window_attention_tiled_amd.inputs import DecodeInputs, fwd_inputs  # noqa: E402
from tests.gpu_util import to_dev  # noqa: E402
from tests.test_random_gpu import BWD_CASES as _RAND_BWD  # noqa: E402
from tests.test_random_gpu import CACHED_CASES as _RAND_CACHED  # noqa: E402
from tests.test_random_gpu import DECODE_CASES as _RAND_DECODE  # noqa: E402
from tests.test_random_gpu import FWD_CASES as _RAND_FWD  # noqa: E402
from tests.test_random_gpu import SINK_CASES as _RAND_SINKS  # noqa: E402


def _rand_fwd(case):
    name, B, Hq, Hkv, N, D, dt, wl, wr, dil, G, sc = case

    def run():
        q, k, v = (to_dev(x) for x in fwd_inputs(1000 + int(name[1:]), B, Hq, Hkv, N, D, dt))
        out, lse = binding.fwd(q, k, v, win_left=wl, win_right=wr, dilation=dil,
                               global_idx=G, scale=sc)
        return [out, lse]
    return run


def _rand_bwd(case):
    name, B, Hq, Hkv, N, D, dt, wl, wr, dil, G, sc = case

    def run():
        seed = 2000 + int(name[1:])
        q, k, v = (to_dev(x) for x in fwd_inputs(seed, B, Hq, Hkv, N, D, dt))
        g = to_dev(fwd_inputs(seed + 500, B, Hq, Hkv, N, D, dt)[0])
        kw = dict(win_left=wl, win_right=wr, dilation=dil, global_idx=G, scale=sc)
        out, lse = binding.fwd(q, k, v, **kw)
        return [out, lse, *binding.bwd(q, k, v, out, lse, g, **kw)]
    return run


def _dev_ring(gen):
    return (to_dev(gen.kcache), to_dev(gen.vcache),
            torch.from_numpy(gen.ring_head.copy()).to("cuda"),
            torch.from_numpy(gen.cache_len.copy()).to("cuda"))


def _rand_decode(case):
    name, B, Hq, Hkv, W, D, dt, fill = case

    def run():
        gen = DecodeInputs(3000 + int(name[1:]), B, Hq, Hkv, W, D, dt, fill=fill)
        kc, vc, head, length = _dev_ring(gen)
        res = []
        for _ in range(3):
            qn, kn, vn = gen.step()
            binding.kv_append(kc, vc, to_dev(kn), to_dev(vn), head, length)
            res += list(binding.decode(to_dev(qn), kc, vc, head, length))
        return res + [kc, vc, head, length]
    return run


def _rand_cached(case):
    name, B, Hq, Hkv, W, D, dt, fill, n, wl = case

    def run():
        seed = 4000 + int(name[1:])
        gen = DecodeInputs(seed, B, 1, Hkv, W, D, dt, fill=fill)
        q, k, v = (to_dev(x) for x in fwd_inputs(seed + 500, B, Hq, Hkv, n, D, dt))
        kc, vc, head, length = _dev_ring(gen)
        out, lse = binding.fwd_cached(q, k, v, kc, vc, head, length, win_left=wl)
        binding.kv_append_chunk(kc, vc, k, v, head, length)
        return [out, lse, kc, vc, head, length]
    return run


def _rand_sinks(case):
    from tests.test_sinks_gpu import _sinks
    name, B, Hq, Hkv, W, D, dt, fill, S = case

    def run():
        seed = 5000 + int(name[1:])
        gen = DecodeInputs(seed, B, Hq, Hkv, W, D, dt, fill=fill)
        ks, vs = (to_dev(x) for x in _sinks(seed + 500, B, Hkv, S, D, dt))
        kc, vc, head, length = _dev_ring(gen)
        res = []
        for _ in range(2):
            qn, kn, vn = gen.step()
            binding.kv_append(kc, vc, to_dev(kn), to_dev(vn), head, length)
            res += list(binding.decode_sinks(to_dev(qn), kc, vc, head, length, ks, vs))
        return res
    return run


CASES += [(f"random_fwd_{c[0]}", _rand_fwd(c)) for c in _RAND_FWD]
CASES += [(f"random_bwd_{c[0]}", _rand_bwd(c)) for c in _RAND_BWD]
CASES += [(f"random_decode_{c[0]}", _rand_decode(c)) for c in _RAND_DECODE]
CASES += [(f"random_cached_{c[0]}", _rand_cached(c)) for c in _RAND_CACHED]
CASES += [(f"random_sinks_{c[0]}", _rand_sinks(c)) for c in _RAND_SINKS]


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype.is_floating_point:
        iv = {2: torch.int16, 4: torch.int32}[a.element_size()]
        return torch.equal(a.view(iv), b.view(iv))
    return torch.equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_debug_build_matches_release_bit_for_bit(case):
    name, run = case
    log(f"[debug build] {name}: release")
    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    with binding.use_library(swa_build.DEBUG_LIB):
        binding.debug_violations(reset=True)
        log(f"[debug build] {name}: debug")
        got = run()
        torch.cuda.synchronize()
        n_bad = binding.debug_violations(reset=True)
    assert n_bad == 0, f"{name}: {n_bad} failed index checks"
    assert len(got) == len(ref)
    for i, (a, b) in enumerate(zip(ref, got)):
        assert a.shape == b.shape and a.dtype == b.dtype
        assert _same_bits(a, b), f"{name}: output {i} differs from the release build"


@pytest.mark.gpu
def test_debug_counter_sees_a_broken_ring_length():
    B, Hkv, W, D = 2, 2, 64, 128
    with binding.use_library(swa_build.DEBUG_LIB):
        binding.debug_violations(reset=True)
        kc, vc, head, length = _ring(B, Hkv, W, D)
        length[1] = W + 5     # above the ring size: clamped by the append
        log("[debug build] ring append with cache_len > W")
        g = torch.Generator().manual_seed(15)
        binding.kv_append(kc, vc, _randn(g, B, Hkv, D), _randn(g, B, Hkv, D), head, length)
        n_bad = binding.debug_violations(reset=True)
        assert n_bad > 0
        assert length.cpu().tolist() == [1, W]
        assert binding.debug_violations(reset=True) == 0
