"""Seeded random shapes against the fp64 oracle, every element.

The hand-picked cases elsewhere pin each feature on its own; these draw them
together (GQA group sizes 1 to 8, asymmetric and degenerate windows, dilation,
duplicate and edge global tokens, both head dimensions and both dtypes; for
the decode, with and without sinks, and the chunked prefill: batch, GQA
group, ring size and fill, sink count, chunk length and window) so that combinations nobody
listed are exercised too.  The draws come from one
fixed seed: every run checks the same shapes.
"""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding
from sliding_window_attention_tiled_amd.inputs import DecodeInputs, fwd_inputs
from tests.gpu_util import check, log, to_dev, to_host_f64
from tests.test_bwd_gpu import _check_grad

pytestmark = pytest.mark.gpu


def _draw(n_cases, seed, max_n, min_span):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for c in range(n_cases):
        group = int(rng.choice([1, 2, 3, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        B = int(rng.choice([1, 2]))
        N = int(rng.integers(1, max_n + 1))
        D = int(rng.choice([64, 128]))
        dt = "f32" if rng.random() < 0.2 else "bf16"
        wl = int(rng.integers(min_span, N + 60))
        wr = 0 if rng.random() < 0.5 else int(rng.integers(0, N + 60))
        dil = 1 if rng.random() < 0.5 else int(rng.integers(2, 7))
        G = None
        if rng.random() < 0.4:
            G = rng.integers(0, N, int(rng.integers(1, 9))).tolist()   # duplicates allowed
            if rng.random() < 0.5:
                G += [0, N - 1]
        scale = None if rng.random() < 0.7 else float(rng.uniform(0.05, 0.3))
        cases.append((f"r{c}", B, group * Hkv, Hkv, N, D, dt, wl, wr, dil, G, scale))
    return cases


FWD_CASES = _draw(40, 20261203, 700, 0)


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_random(case):
    name, B, Hq, Hkv, N, D, dt, wl, wr, dil, G, sc = case
    q, k, v = fwd_inputs(1000 + int(name[1:]), B, Hq, Hkv, N, D, dt)
    kw = dict(win_left=wl, win_right=wr, dilation=dil, global_idx=G, scale=sc)
    log(f"[fwd random] {case}")
    ref_o, ref_l = oracle.fwd(q, k, v, **kw)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, N), float("nan"), device="cuda")
    binding.fwd(qd, kd, vd, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    check(to_host_f64(out), ref_o, dt, f"{name} out")
    check(to_host_f64(lse), ref_l, dt, f"{name} lse")


# the backward's draws keep at least 8 keys of window per row (wl >= 8): with a
# handful of keys dS = P (dP - delta) nearly cancels and the rounding of the
# forward's output dominates, which the relative check would misread
BWD_CASES = _draw(12, 20261204, 320, 8)


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_random(case):
    name, B, Hq, Hkv, N, D, dt, wl, wr, dil, G, sc = case
    seed = 2000 + int(name[1:])
    q, k, v = fwd_inputs(seed, B, Hq, Hkv, N, D, dt)
    g = fwd_inputs(seed + 500, B, Hq, Hkv, N, D, dt)[0]
    log(f"[bwd random] {case}")
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    kw = dict(win_left=wl, win_right=wr, dilation=dil, global_idx=G, scale=sc)
    out, lse = binding.fwd(qd, kd, vd, **kw)
    dq, dk, dv = binding.bwd(qd, kd, vd, out, lse, gd, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd(q, k, v, g, **kw)
    _check_grad(to_host_f64(dq), rq, dt, f"{name} dq")
    _check_grad(to_host_f64(dk), rk, dt, f"{name} dk")
    _check_grad(to_host_f64(dv), rv, dt, f"{name} dv")


def _draw_decode(n_cases, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for c in range(n_cases):
        Hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4, 8, 16]))
        B = int(rng.integers(1, 7))
        W = int(rng.integers(1, 1201))
        D = int(rng.choice([64, 128]))
        dt = "f32" if rng.random() < 0.2 else "bf16"
        u = rng.random()
        fill = None if u < 0.4 else (0 if u < 0.55 else int(rng.integers(0, W + 1)))
        cases.append((f"d{c}", B, group * Hkv, Hkv, W, D, dt, fill))
    return cases


# ring sizes up to 1200 and batches of 1 to 6 take the decode through one and
# through many slot ranges per (sequence, kv head), and through the combine
DECODE_CASES = _draw_decode(16, 20261205)


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_random(case):
    from tests.test_decode_gpu import _run_steps
    name, B, Hq, Hkv, W, D, dt, fill = case
    log(f"[decode random] {case}")
    gen = DecodeInputs(3000 + int(name[1:]), B, Hq, Hkv, W, D, dt, fill=fill)
    _run_steps(gen, 5, set(range(5)), dt, name)


def _draw_cached(n_cases, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for c in range(n_cases):
        Hkv = int(rng.choice([1, 2]))
        group = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 4))
        W = int(rng.integers(1, 601))
        D = int(rng.choice([64, 128]))
        dt = "f32" if rng.random() < 0.2 else "bf16"
        u = rng.random()
        fill = None if u < 0.4 else (0 if u < 0.55 else int(rng.integers(0, W + 1)))
        n = int(rng.integers(1, 501))
        wl = int(rng.integers(0, W + 1))       # a chunk's window fits the ring: wl <= W
        cases.append((f"c{c}", B, group * Hkv, Hkv, W, D, dt, fill, n, wl))
    return cases


CACHED_CASES = _draw_cached(12, 20261206)


@pytest.mark.parametrize("case", CACHED_CASES, ids=[c[0] for c in CACHED_CASES])
def test_fwd_cached_random(case):
    name, B, Hq, Hkv, W, D, dt, fill, n, wl = case
    log(f"[fwd_cached random] {case}")
    seed = 4000 + int(name[1:])
    gen = DecodeInputs(seed, B, 1, Hkv, W, D, dt, fill=fill)
    q, k, v = fwd_inputs(seed + 500, B, Hq, Hkv, n, D, dt)
    kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
    head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
    length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
    out, lse = binding.fwd_cached(to_dev(q), to_dev(k), to_dev(v), kc, vc, head, length,
                                  win_left=wl)
    torch.cuda.synchronize()
    ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
    ref_o, ref_l = ring.fwd_cached(q, k, v, win_left=wl)
    check(to_host_f64(out), ref_o, dt, f"{name} out")
    check(to_host_f64(lse), ref_l, dt, f"{name} lse")


SINK_CASES = [(f"s{c[0][1:]}",) + c[1:] + (int(n),) for c, n in zip(
    _draw_decode(12, 20261207),
    np.random.Generator(np.random.PCG64(20261208)).integers(0, 20, 12))]


@pytest.mark.parametrize("case", SINK_CASES, ids=[c[0] for c in SINK_CASES])
def test_decode_sinks_random(case):
    from tests.test_sinks_gpu import _sinks
    name, B, Hq, Hkv, W, D, dt, fill, S = case
    log(f"[decode_sinks random] {case}")
    seed = 5000 + int(name[1:])
    gen = DecodeInputs(seed, B, Hq, Hkv, W, D, dt, fill=fill)
    ks, vs = _sinks(seed + 500, B, Hkv, S, D, dt)
    kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
    head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
    length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
    ksd, vsd = to_dev(ks), to_dev(vs)
    ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
    for t in range(3):
        qn, kn, vn = gen.step()
        binding.kv_append(kc, vc, to_dev(kn), to_dev(vn), head, length)
        out, lse = binding.decode_sinks(to_dev(qn), kc, vc, head, length, ksd, vsd)
        torch.cuda.synchronize()
        ring.append(kn, vn)
        ref_o, ref_l = ring.decode(qn, sinks=(ks, vs))
        check(to_host_f64(out), ref_o, dt, f"{name} step {t} out")
        check(to_host_f64(lse), ref_l, dt, f"{name} step {t} lse")
