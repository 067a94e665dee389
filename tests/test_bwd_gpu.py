"""GPU parity of swa_bwd (dq, dk, dv) against the oracle's backward.

The GPU forward supplies out and lse (as a training step would); the oracle
computes the exact gradients of the definition from the same inputs, so the
forward's rounding is part of what is checked.  Small shapes are compared on
every element; the full-size Mistral-shaped layer on sampled dq rows, the dv
row sums, and sampled dk/dv keys of the dilated stack (whose short window
keeps the per-key oracle cheap).
"""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding, configs
from sliding_window_attention_tiled_amd.inputs import fwd_inputs
from tests.gpu_util import check, log, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

SMALL = [
    # name, B, Hq, Hkv, N, D, dtype, wl, wr, dil, scale
    ("causal_gqa4_d128", 1, 8, 2, 300, 128, "bf16", 100, 0, 1, None),
    ("bidir_asym_mha_d64", 2, 3, 3, 257, 64, "bf16", 40, 17, 1, None),
    ("dilated3_gqa2", 1, 4, 2, 400, 128, "bf16", 30, 0, 3, None),
    ("dilated2_bidir_d64", 1, 2, 1, 333, 64, "bf16", 12, 9, 2, 0.2),
    ("window_ge_n", 1, 4, 4, 150, 64, "bf16", 500, 500, 1, None),
    ("tiny_rows", 1, 2, 2, 5, 128, "bf16", 3, 0, 1, None),
    ("f32_causal", 1, 4, 2, 200, 128, "f32", 63, 0, 1, 0.1),
    ("f32_dilated_bidir", 1, 2, 2, 150, 64, "f32", 7, 5, 4, 0.15),
]


def _run(q, k, v, g, dt, wl, wr, dil, scale, G=None):
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    out, lse = binding.fwd(qd, kd, vd, win_left=wl, win_right=wr, dilation=dil, scale=scale,
                           global_idx=G)
    dq, dk, dv = binding.bwd(qd, kd, vd, out, lse, gd, win_left=wl, win_right=wr,
                             dilation=dil, global_idx=G, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check_grad(got, ref, dt, what, long_rows=None):
    """Gradients scale with the number of attended rows; compare in units of
    the largest reference entry (at least 1).  long_rows (a boolean per
    sampled row) limits the relative-RMS part of the bf16 check to rows that
    attend at least 8 keys: on a row with a handful of keys dS = P (dP - delta)
    nearly cancels, and delta = dout . out carries the bf16 rounding of the
    forward's output, so such rows carry up to a few 1e-2 relative error at
    the same small absolute error (the max-abs part still covers them)."""
    s = max(1.0, float(np.max(np.abs(ref))))
    got, ref = got / s, ref / s
    if long_rows is None or dt != "bf16":
        return check(got, ref, dt, what)
    mx = float(np.max(np.abs(got - ref)))
    assert mx <= 2e-2, f"{what}: max-abs {mx:.3e}"
    return check(got[long_rows], ref[long_rows], dt, what + " (rows with >= 8 keys)")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_bwd_small(case):
    name, B, Hq, Hkv, N, D, dt, wl, wr, dil, scale = case
    q, k, v = fwd_inputs(91, B, Hq, Hkv, N, D, dt)
    g = fwd_inputs(92, B, Hq, Hkv, N, D, dt)[0]
    log(f"[bwd] {name}")
    dq, dk, dv = _run(q, k, v, g, dt, wl, wr, dil, scale)
    rq, rk, rv = oracle.bwd(q, k, v, g, win_left=wl, win_right=wr, dilation=dil, scale=scale)
    _check_grad(to_host_f64(dq), rq, dt, f"{name} dq")
    _check_grad(to_host_f64(dk), rk, dt, f"{name} dk")
    _check_grad(to_host_f64(dv), rv, dt, f"{name} dv")


GLOBAL_CASES = [
    # name, B, Hq, Hkv, N, D, dtype, wl, wr, dil, scale, global positions
    ("g_bidir_gqa4_d128", 1, 8, 2, 300, 128, "bf16", 40, 40, 1, None, [0, 7, 150, 299]),
    ("g_causal_mha_d64", 2, 4, 4, 257, 64, "bf16", 30, 0, 1, None, [0, 100, 256]),
    ("g_dilated3_gqa2", 1, 4, 2, 400, 128, "bf16", 20, 0, 3, None, [3, 5, 200, 201, 399]),
    ("g_many_bidir", 1, 2, 1, 700, 64, "bf16", 16, 16, 1, None, list(range(0, 700, 7))),
    ("g_f32_dilated_bidir", 1, 2, 2, 150, 64, "f32", 7, 5, 2, 0.3, [0, 1, 2, 75, 149]),
    ("g_f32_causal_d128", 1, 4, 1, 333, 128, "f32", 50, 0, 1, None, [10, 20, 330, 20]),
    # every token global: no non-global rows, every pair outside the band is a global row's
    ("g_all_global_f32", 1, 2, 1, 70, 64, "f32", 5, 0, 1, None, list(range(70))),
    # window covering the sequence: the global tokens add no pair
    ("g_window_ge_n", 1, 4, 2, 90, 128, "bf16", 200, 200, 1, None, [0, 45, 89]),
    # three tokens, one global, causal
    ("g_tiny_n", 1, 2, 2, 3, 64, "bf16", 1, 0, 1, None, [1]),
    # D = 64 bf16, where the band passes take the global pairs themselves:
    # causal with dilation (global rows and keys in every residue class), and
    # 84 globals (two gathered tiles per head in both passes)
    ("g_causal_dil3_gqa2_d64", 1, 4, 2, 420, 64, "bf16", 25, 0, 3, None,
     [0, 1, 2, 64, 65, 200, 301, 419]),
    ("g_many_causal_dil2_d64", 1, 4, 2, 500, 64, "bf16", 40, 0, 2, None,
     list(range(1, 500, 6))),
    # D = 128 bf16, where rows_dkdv adds the global rows' terms to every key and
    # sums the global keys' partials before its one rounding: many globals, so
    # that each global key gathers terms from most rows of the sequence
    ("g_many_bidir_gqa4_d128", 1, 8, 2, 900, 128, "bf16", 48, 48, 1, None,
     list(range(0, 900, 9))),
    ("g_many_causal_d128", 1, 4, 1, 800, 128, "bf16", 64, 0, 1, None,
     list(range(3, 800, 8))),
]


@pytest.mark.parametrize("case", GLOBAL_CASES, ids=[c[0] for c in GLOBAL_CASES])
def test_bwd_global_tokens_small(case):
    """Global rows attend every key and every row attends the global keys: the
    backward's pairs outside the band, every element against the oracle."""
    name, B, Hq, Hkv, N, D, dt, wl, wr, dil, scale, G = case
    q, k, v = fwd_inputs(95, B, Hq, Hkv, N, D, dt)
    g = fwd_inputs(96, B, Hq, Hkv, N, D, dt)[0]
    log(f"[bwd] {name}")
    dq, dk, dv = _run(q, k, v, g, dt, wl, wr, dil, scale, G)
    rq, rk, rv = oracle.bwd(q, k, v, g, win_left=wl, win_right=wr, dilation=dil,
                            global_idx=G, scale=scale)
    _check_grad(to_host_f64(dq), rq, dt, f"{name} dq")
    _check_grad(to_host_f64(dk), rk, dt, f"{name} dk")
    _check_grad(to_host_f64(dv), rv, dt, f"{name} dv")


def test_bwd_full_size_global_tokens_sampled():
    """The bidirectional encoder layer with 16 global tokens at full size:
    sampled dq rows and dk/dv keys, global ones included."""
    c = configs.FWD["bidir_encoder_globals"]
    B, Hq, Hkv, N, D, dt = c["B"], c["Hq"], c["Hkv"], c["N"], c["D"], c["dtype"]
    G = c["global_idx"]
    wl, wr = c["win_left"], c["win_right"]
    q, k, v = fwd_inputs(c["seed"], B, Hq, Hkv, N, D, dt)
    g = fwd_inputs(c["seed"] + 100, B, Hq, Hkv, N, D, dt)[0]
    log("[bwd] bidirectional encoder with globals, full size")
    dq, dk, dv = _run(q, k, v, g, dt, wl, wr, 1, None, G)
    rng = np.random.Generator(np.random.PCG64(97))
    picks = [0, 512, 4096, 8192 - 512, 1, 511, 513, N - 1] + rng.integers(0, N, 4).tolist()
    rows = np.array([[int(rng.integers(0, B)), int(rng.integers(0, Hq)), int(i)] for i in picks])
    ref = oracle.bwd_dq_rows(q, k, v, g, rows, win_left=wl, win_right=wr, global_idx=G)
    got = to_host_f64(dq)
    _check_grad(np.stack([got[b, i, h] for b, h, i in rows]), ref, dt, "globals sampled dq")
    sel = np.array([[int(rng.integers(0, B)), int(rng.integers(0, Hkv)), int(j)] for j in picks])
    rk, rv = oracle.bwd_dkv_keys(q, k, v, g, sel, win_left=wl, win_right=wr, global_idx=G)
    gk, gv = to_host_f64(dk), to_host_f64(dv)
    _check_grad(np.stack([gk[b, j, h] for b, h, j in sel]), rk, dt, "globals sampled dk")
    _check_grad(np.stack([gv[b, j, h] for b, h, j in sel]), rv, dt, "globals sampled dv")


def test_bwd_full_size_mistral_sampled():
    c = configs.FWD["mistral_causal_w4096"]
    B, Hq, Hkv, N, D, dt = c["B"], c["Hq"], c["Hkv"], c["N"], c["D"], c["dtype"]
    q, k, v = fwd_inputs(c["seed"], B, Hq, Hkv, N, D, dt)
    g = fwd_inputs(c["seed"] + 100, B, Hq, Hkv, N, D, dt)[0]
    log("[bwd] mistral full size")
    dq, dk, dv = _run(q, k, v, g, dt, c["win_left"], 0, 1, None)
    rng = np.random.Generator(np.random.PCG64(93))
    rows = np.array([[0, int(rng.integers(0, Hq)), int(i)] for i in
                     [0, 1, 4094, 4095, 4096, 8191, N - 1] + rng.integers(0, N, 9).tolist()])
    ref = oracle.bwd_dq_rows(q, k, v, g, rows, win_left=c["win_left"])
    got = to_host_f64(dq)
    _check_grad(np.stack([got[b, i, h] for b, h, i in rows]), ref, dt, "mistral sampled dq",
                long_rows=rows[:, 2] >= 7)
    # every row of P sums to one: the dv rows of a kv head add up to the dout
    # rows of its query heads
    from oracle.bruteforce import widen
    gsum = widen(g).reshape(B, N, Hkv, Hq // Hkv, D).sum(axis=(1, 3))
    _check_grad(to_host_f64(dv).sum(axis=1), gsum, dt, "mistral dv row sums")


@pytest.mark.parametrize("d", [1, 8])
def test_bwd_full_size_dilated_sampled(d):
    c = configs.DILATED_STACK
    B, H, N, D, dt = c["B"], c["Hq"], c["N"], c["D"], c["dtype"]
    q, k, v = fwd_inputs(c["seed"], B, H, H, N, D, dt)
    g = fwd_inputs(c["seed"] + 100, B, H, H, N, D, dt)[0]
    log(f"[bwd] dilated stack d={d} full size")
    dq, dk, dv = _run(q, k, v, g, dt, c["win_left"], 0, d, None)
    rng = np.random.Generator(np.random.PCG64(94 + d))
    rows = np.array([[int(rng.integers(0, B)), int(rng.integers(0, H)), int(i)] for i in
                     [0, d, 511 * d, N - 1] + rng.integers(0, N, 6).tolist()])
    ref = oracle.bwd_dq_rows(q, k, v, g, rows, win_left=c["win_left"], dilation=d)
    got = to_host_f64(dq)
    _check_grad(np.stack([got[b, i, h] for b, h, i in rows]), ref, dt, f"d={d} sampled dq",
                long_rows=rows[:, 2] >= 7 * d)
    sel = np.array([[int(rng.integers(0, B)), int(rng.integers(0, H)), int(j)] for j in
                    [0, N - 1, N - 1 - 511 * d, N // 2] + rng.integers(0, N, 2).tolist()])
    rk, rv = oracle.bwd_dkv_keys(q, k, v, g, sel, win_left=c["win_left"], dilation=d)
    gk, gv = to_host_f64(dk), to_host_f64(dv)
    _check_grad(np.stack([gk[b, j, h] for b, h, j in sel]), rk, dt, f"d={d} sampled dk")
    _check_grad(np.stack([gv[b, j, h] for b, h, j in sel]), rv, dt, f"d={d} sampled dv")


REPEAT_CASES = [
    # name, B, Hq, Hkv, N, D, dtype, wl, wr, global positions
    ("rep_bidir_globals_d64", 2, 6, 6, 2048, 64, "bf16", 128, 128, list(range(0, 2048, 256))),
    ("rep_causal_gqa4_d128", 1, 8, 2, 1500, 128, "bf16", 300, 0, [0, 1, 700, 1499]),
    ("rep_many_globals_d64", 1, 4, 2, 1200, 64, "bf16", 32, 32, list(range(3, 1200, 37))),
    ("rep_f32_bidir", 1, 4, 4, 700, 64, "f32", 50, 50, [0, 350, 699]),
]


@pytest.mark.parametrize("case", REPEAT_CASES, ids=[c[0] for c in REPEAT_CASES])
def test_bwd_with_globals_is_bitwise_repeatable(case):
    """Every sum of the backward, those over the global tokens' split partials
    included, has a fixed order: repeated calls give the same bits (and match
    the oracle)."""
    name, B, Hq, Hkv, N, D, dt, wl, wr, G = case
    q, k, v = fwd_inputs(95, B, Hq, Hkv, N, D, dt)
    g = fwd_inputs(96, B, Hq, Hkv, N, D, dt)[0]
    log(f"[bwd repeat] {name}")
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    kw = dict(win_left=wl, win_right=wr, global_idx=G)
    out, lse = binding.fwd(qd, kd, vd, **kw)
    first = None
    for rep in range(3):
        grads = binding.bwd(qd, kd, vd, out, lse, gd, **kw)
        torch.cuda.synchronize()
        bits_now = [t.view(torch.int16 if dt == "bf16" else torch.int32).cpu().clone()
                    for t in grads]
        if first is None:
            first = bits_now
        else:
            for a, b_, nm in zip(first, bits_now, ("dq", "dk", "dv")):
                assert torch.equal(a, b_), f"{name}: {nm} differs on call {rep + 1}"
    rq, rk, rv = oracle.bwd(q, k, v, g, **kw)
    _check_grad(to_host_f64(grads[0]), rq, dt, f"{name} dq")
    _check_grad(to_host_f64(grads[1]), rk, dt, f"{name} dk")
    _check_grad(to_host_f64(grads[2]), rv, dt, f"{name} dv")
