"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every function here takes an ``OracleLib`` and raises AssertionError when the
oracle disagrees with what the pages or the mathematics fix:

* values the pages print (index sets, the ring-buffer rule, the demo's window),
  stored under tests/golden/ with their citations;
* the dense-mask brute force (a different formulation of the same definition);
* closed forms and special cases that reduce to a library routine
  (torch's scaled_dot_product_attention in float64 on the CPU);
* invariants (dilation = strided undilated problems, GQA = repeated heads,
  ring rotation, partial rings).

The same functions run against deliberately broken copies of the oracle in
test_oracle_mutations.py, to show that each plausible mistake is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle import bruteforce
from sliding_window_attention_tiled_amd.inputs import fwd_inputs, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


def _sdpa(q, k, v, causal, scale):
    """Library attention in float64: q/k/v [B,N,H,D] float64 numpy (H equal)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3)))
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v),
                                                         is_causal=causal, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


# ---- values printed on the pages -------------------------------------------

def pin_dilated_index_sets(orc):
    g = _golden("dilated_index_sets.json")
    i, N = 40, 100
    for c in g["cases"]:
        got = orc.attended_set(i, N, g["win_left"], g["win_right"], c["dilation"])
        assert got == [i + o for o in c["offsets"]], (c, got)


def pin_dilated_span(orc):
    g = _golden("dilated_span.json")
    i, N = 50, 100
    got = orc.attended_set(i, N, g["win_left"], g["win_right"], g["dilation"])
    assert len(got) == g["keys"], got
    assert got[-1] - got[0] + 1 == g["span"], got


def pin_edge_truncation(orc):
    g = _golden("edge_truncation.json")
    half = g["W"] // 2
    for c in g["cases"]:
        got = orc.attended_set(c["i"], g["N"], half, half, 1)
        assert got == c["keys"], (c, got)


def pin_decode_demo_window(orc):
    g = _golden("decode_demo_window.json")
    n, w = g["n"], g["window_size"]
    # as a causal forward window of w keys for the last token
    assert orc.attended_set(n - 1, n, w - 1, 0, 1) == g["keys"]
    # as a decode step: a ring of w slots after appending n tokens one by one,
    # scale 1 as in the demo.  The demo draws K, V, q from seed 42.
    rs = np.random.RandomState(42)
    d = 8
    K = rs.randn(n, d).astype(np.float32)
    V = rs.randn(n, d).astype(np.float32)
    q = rs.randn(d).astype(np.float32)
    ring = orc.ring(np.zeros((1, 1, w, d), np.float32), np.zeros((1, 1, w, d), np.float32),
                    [0], [0])
    for t in range(n):
        ring.append(K[t][None, None, :], V[t][None, None, :])
    out, lse = ring.decode(q[None, None, :], scale=1.0)
    keys = g["keys"]
    ref = _sdpa(q[None, None, None, :].astype(np.float64),
                K[keys][None, :, None, :].astype(np.float64),
                V[keys][None, :, None, :].astype(np.float64), False, 1.0)
    _close(out[0, 0], ref[0, 0, 0], 1e-12, "decode demo window")
    s = K[keys].astype(np.float64) @ q.astype(np.float64)
    _close(lse[0, 0], np.log(np.exp(s).sum()), 1e-12, "decode demo lse")


def pin_ring_buffer_trace(orc):
    g = _golden("ring_buffer_trace.json")
    W = g["size"]
    ring = orc.ring(np.zeros((1, 1, W, 1), np.float32), np.zeros((1, 1, W, 1), np.float32),
                    [0], [0])
    for item in g["appended"]:
        x = np.full((1, 1, 1), float(item), np.float32)
        ring.append(x, x)
    assert ring.k[0, 0, :, 0].tolist() == [float(x) for x in g["buffer"]], ring.k
    assert int(ring.head[0]) == g["next_slot"]
    assert int(ring.len[0]) == W
    # q = 0: uniform weights over the held items -> their mean, lse = ln(count)
    out, lse = ring.decode(np.zeros((1, 1, 1), np.float32), scale=1.0)
    _close(out[0, 0, 0], np.mean(g["held_items"]), 1e-12, "ring mean")
    _close(lse[0, 0], math.log(len(g["held_items"])), 1e-12, "ring lse")


# ---- the dense-mask brute force ---------------------------------------------

BRUTE_CASES = [
    # (B, Hq, Hkv, N, D, wl, wr, dil, globals, dtype, scale)
    (1, 2, 2, 1, 8, 3, 0, 1, None, "f32", None),
    (1, 2, 2, 2, 8, 3, 0, 1, None, "f32", None),
    (2, 2, 1, 63, 16, 7, 0, 1, None, "bf16", None),
    (1, 4, 2, 70, 8, 5, 3, 1, None, "f32", 0.37),           # asymmetric window
    (1, 2, 2, 65, 8, 4, 4, 1, [0, 17, 17, 64], "bf16", None),  # bidir + globals
    (1, 2, 2, 64, 8, 9, 0, 1, [0, 31, 40], "f32", None),      # causal + globals
    (1, 2, 2, 77, 8, 5, 0, 3, None, "bf16", None),            # dilated causal
    (1, 2, 2, 81, 8, 2, 3, 2, [5, 6], "f32", None),           # dilated bidir + globals
    (1, 4, 1, 257, 16, 20, 0, 4, None, "bf16", 0.2),          # GQA 4, dilated
    (1, 2, 2, 40, 8, 100, 100, 1, None, "f32", None),         # window > N
]


def pin_bruteforce(orc):
    for n, (B, Hq, Hkv, N, D, wl, wr, dil, G, dt, sc) in enumerate(BRUTE_CASES):
        q, k, v = fwd_inputs(100 + n, B, Hq, Hkv, N, D, dt)
        o1, l1 = orc.fwd(q, k, v, win_left=wl, win_right=wr, dilation=dil, global_idx=G,
                         scale=sc)
        o2, l2 = bruteforce.fwd(q, k, v, win_left=wl, win_right=wr, dilation=dil,
                                global_idx=G, scale=sc)
        _close(o1, o2, 1e-12, f"brute force case {n} out")
        _close(l1, l2, 1e-12, f"brute force case {n} lse")
        # the row-sampled entry point agrees with the full one
        rows = np.array([[B - 1, Hq - 1, N - 1], [0, 0, 0], [0, Hq // 2, N // 2]])
        o3, l3 = orc.fwd_rows(q, k, v, rows, win_left=wl, win_right=wr, dilation=dil,
                              global_idx=G, scale=sc)
        for r, (b, h, i) in enumerate(rows):
            _close(o3[r], o1[b, i, h], 0.0, "fwd_rows out")
            _close(l3[r], l1[b, h, i], 0.0, "fwd_rows lse")


def pin_bruteforce_mask_is_page_mask(orc):
    """bruteforce's mask for odd W equals the page's |j - i| > W // 2 rule."""
    del orc
    for N, W in [(10, 5), (33, 9), (7, 1)]:
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        page_masked = np.abs(j - i) > W // 2
        assert np.array_equal(~page_masked, bruteforce.mask_matrix(N, W // 2, W // 2))


# ---- closed forms and special cases -------------------------------------------

def pin_full_window(orc):
    """A window covering the whole sequence is ordinary (causal) attention."""
    for causal in (False, True):
        B, H, N, D = 2, 3, 37, 16
        q, k, v = fwd_inputs(7, B, H, H, N, D, "f32")
        wr = 0 if causal else N
        out, lse = orc.fwd(q, k, v, win_left=N + 5, win_right=wr, scale=0.3)
        ref = _sdpa(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                    causal, 0.3)
        _close(out, ref, 1e-12, f"full window causal={causal}")
        s = 0.3 * np.einsum("bihd,bjhd->bhij", q.astype(np.float64), k.astype(np.float64))
        if causal:
            s = s + np.triu(np.full((N, N), -np.inf), 1)
        ref_lse = np.log(np.exp(s).sum(-1))
        _close(lse, ref_lse, 1e-12, f"full window lse causal={causal}")


def pin_zero_window(orc):
    """wl = wr = 0: each query attends only itself -> out_i = v_i, lse_i = s_ii."""
    B, Hq, Hkv, N, D = 1, 4, 2, 19, 8
    q, k, v = fwd_inputs(8, B, Hq, Hkv, N, D, "bf16")
    out, lse = orc.fwd(q, k, v, win_left=0, win_right=0, scale=0.5)
    qf, kf, vf = (bruteforce.widen(x) for x in (q, k, v))
    for h in range(Hq):
        kh = h // (Hq // Hkv)
        _close(out[:, :, h], vf[:, :, kh], 0.0, "zero window out")
        s = 0.5 * np.sum(qf[:, :, h] * kf[:, :, kh], axis=-1)
        _close(lse[:, h], s, 1e-12, "zero window lse")


def _count_band(i, N, wl, wr, d):
    tmin = max(-wl, -(i // d))
    tmax = min(wr, (N - 1 - i) // d)
    return list(range(i + tmin * d, i + tmax * d + 1, d))


def pin_q_zero(orc):
    """q = 0: uniform weights -> out = mean of v over S(i), lse = ln |S(i)|."""
    for (N, wl, wr, d, G) in [(50, 6, 0, 1, None), (50, 3, 4, 3, None),
                              (60, 5, 0, 2, [0, 13, 14]), (45, 2, 2, 1, [7, 44])]:
        B, H, D = 1, 2, 4
        _, k, v = fwd_inputs(9, B, H, H, N, D, "f32")
        q = np.zeros((B, N, H, D), np.float32)
        out, lse = orc.fwd(q, k, v, win_left=wl, win_right=wr, dilation=d, global_idx=G)
        causal = wr == 0
        gset = set(G or [])
        for i in range(N):
            if i in gset:
                S = [j for j in range(N) if not causal or j <= i]
            else:
                S = sorted(set(_count_band(i, N, wl, wr, d)) |
                           {g for g in gset if not causal or g <= i})
            _close(out[0, i], v[0, S].astype(np.float64).mean(axis=0), 1e-12, "q=0 mean")
            _close(lse[0, :, i], math.log(len(S)), 1e-12, "q=0 lse")


def pin_dilation_strided(orc):
    """Dilation d equals d undilated problems on the residue subsequences r::d."""
    B, H, N, D = 1, 2, 90, 8
    q, k, v = fwd_inputs(10, B, H, H, N, D, "bf16")
    for (wl, wr, d) in [(5, 0, 2), (4, 3, 3), (7, 0, 4)]:
        out, lse = orc.fwd(q, k, v, win_left=wl, win_right=wr, dilation=d)
        for r in range(d):
            o_r, l_r = orc.fwd(q[:, r::d], k[:, r::d], v[:, r::d], win_left=wl,
                               win_right=wr, dilation=1, scale=1 / math.sqrt(D))
            _close(out[:, r::d], o_r, 1e-12, "dilation strided out")
            _close(lse[:, :, r::d], l_r, 1e-12, "dilation strided lse")
        # and each residue subsequence against the library routine when the
        # window covers it entirely
        o_all, _ = orc.fwd(q, k, v, win_left=N, win_right=0, dilation=d)
        for r in range(d):
            ref = _sdpa(*(bruteforce.widen(x[:, r::d]) for x in (q, k, v)), True,
                        1 / math.sqrt(D))
            _close(o_all[:, r::d], ref, 1e-12, "dilated full window")


def pin_gqa(orc):
    """Grouped KV heads equal running with k, v repeated per query head."""
    B, Hq, Hkv, N, D = 1, 6, 2, 33, 8
    q, k, v = fwd_inputs(11, B, Hq, Hkv, N, D, "f32")
    out, lse = orc.fwd(q, k, v, win_left=4, win_right=2)
    kr = np.repeat(k, Hq // Hkv, axis=2)
    vr = np.repeat(v, Hq // Hkv, axis=2)
    out2, lse2 = orc.fwd(q, kr, vr, win_left=4, win_right=2)
    _close(out, out2, 0.0, "gqa out")
    _close(lse, lse2, 0.0, "gqa lse")
    ref = _sdpa(*(x.astype(np.float64) for x in (q, kr, vr)), True, 1 / math.sqrt(D))
    out3, _ = orc.fwd(q, k, v, win_left=N, win_right=0)
    _close(out3, ref, 1e-12, "gqa full causal")


def pin_globals(orc):
    """A global row is a full attention row; with a full window globals change nothing."""
    B, H, N, D = 1, 2, 48, 8
    q, k, v = fwd_inputs(12, B, H, H, N, D, "f32")
    G = [0, 5, 47]
    for causal in (False, True):
        wr = 0 if causal else 3
        out, _ = orc.fwd(q, k, v, win_left=3, win_right=wr, global_idx=G)
        ref = _sdpa(*(x.astype(np.float64) for x in (q, k, v)), causal, 1 / math.sqrt(D))
        for g in G:
            _close(out[:, g], ref[:, g], 1e-12, f"global row {g} causal={causal}")
        full, _ = orc.fwd(q, k, v, win_left=N, win_right=0 if causal else N, global_idx=G)
        _close(full, ref, 1e-12, "full window with globals")
    # causal visibility of a global column: row 2 must not see global key 5
    assert orc.attended_set(2, N, 1, 0, 1, G) == [0, 1, 2]
    assert orc.attended_set(10, N, 1, 0, 1, G) == [0, 5, 9, 10]
    # bidirectional: row 2 sees key 5 and 47 as well
    assert orc.attended_set(2, N, 1, 1, 1, G) == [0, 1, 2, 3, 5, 47]


# ---- decode ---------------------------------------------------------------------

def _logical_sequence(ring_k, ring_v, head, length):
    """Oldest-to-newest rows of one ring (numpy copy, [length, H, D])."""
    W = ring_k.shape[1]
    slots = [(head - length + a) % W for a in range(length)]
    return ring_k[:, slots].transpose(1, 0, 2), ring_v[:, slots].transpose(1, 0, 2)


def pin_decode(orc):
    """A decode step equals the last row of a causal forward with win_left = W-1
    over the logical sequence; partial rings equal full causal attention over the
    filled part; rotating the ring changes nothing."""
    B, Hq, Hkv, W, D = 3, 4, 2, 8, 8
    rng = np.random.Generator(np.random.PCG64(13))
    kc = rng.standard_normal((B, Hkv, W, D), dtype=np.float32)
    vc = rng.standard_normal((B, Hkv, W, D), dtype=np.float32)
    head = np.array([0, 3, 7])
    length = np.array([W, 2, 0])            # full, partial, empty rings
    ring = orc.ring(to_bf16_bits(kc), to_bf16_bits(vc), head, length)
    for step in range(11):
        qt = to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32))
        kt = to_bf16_bits(rng.standard_normal((B, Hkv, D), dtype=np.float32))
        vt = to_bf16_bits(rng.standard_normal((B, Hkv, D), dtype=np.float32))
        ring.append(kt, vt)
        out, lse = ring.decode(qt, scale=0.25)
        for b in range(B):
            n = int(ring.len[b])
            assert n == min(W, int(length[b]) + step + 1)
            ks, vs = _logical_sequence(ring.k[b], ring.v[b], int(ring.head[b]), n)
            # newest entry is the one just appended
            assert np.array_equal(ks[-1], kt[b]) and np.array_equal(vs[-1], vt[b])
            qs = np.zeros((1, n, Hq, D), np.uint16)
            qs[0, -1] = qt[b]
            o_f, l_f = orc.fwd(qs, ks[None], vs[None], win_left=W - 1, win_right=0,
                               scale=0.25)
            _close(out[b], o_f[0, -1], 1e-12, "decode vs causal fwd last row")
            _close(lse[b], l_f[0, :, -1], 1e-12, "decode lse vs causal fwd")
            kr = np.repeat(bruteforce.widen(ks), Hq // Hkv, axis=1)
            vr = np.repeat(bruteforce.widen(vs), Hq // Hkv, axis=1)
            ref = _sdpa(bruteforce.widen(qt[b])[None, None], kr[None], vr[None], False, 0.25)
            _close(out[b], ref[0, 0], 1e-12, "decode vs library attention")
    # rotation: the same logical content at another physical offset
    out_a, lse_a = ring.decode(qt, scale=0.25)
    rot = 5
    ring2 = orc.ring(np.roll(ring.k, rot, axis=2), np.roll(ring.v, rot, axis=2),
                     (ring.head + rot) % W, ring.len)
    out_b, lse_b = ring2.decode(qt, scale=0.25)
    _close(out_a, out_b, 1e-12, "ring rotation out")
    _close(lse_a, lse_b, 1e-12, "ring rotation lse")


# ---- chunked prefill handed to the ring --------------------------------------

def _empty_ring(orc, B, Hkv, W, D, dtype, head):
    z = np.zeros((B, Hkv, W, D), np.uint16 if dtype == "bf16" else np.float32)
    return orc.ring(z, z.copy(), head, [0] * B)


def pin_append_chunk(orc):
    """A chunk append leaves the ring exactly as that many single appends."""
    B, Hkv, W, D = 2, 2, 8, 4
    rng = np.random.Generator(np.random.PCG64(21))
    for n in (0, 1, 5, 8, 11, 19, 27):
        kc = to_bf16_bits(rng.standard_normal((B, Hkv, W, D), dtype=np.float32))
        vc = to_bf16_bits(rng.standard_normal((B, Hkv, W, D), dtype=np.float32))
        head, length = [3, 6], [2, W]
        a = orc.ring(kc, vc, head, length)
        b = orc.ring(kc, vc, head, length)
        k = to_bf16_bits(rng.standard_normal((B, n, Hkv, D), dtype=np.float32))
        v = to_bf16_bits(rng.standard_normal((B, n, Hkv, D), dtype=np.float32))
        a.append_chunk(k, v)
        for t in range(n):
            b.append(np.ascontiguousarray(k[:, t]), np.ascontiguousarray(v[:, t]))
        assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v), f"n={n} contents"
        assert a.head.tolist() == b.head.tolist(), f"n={n} head"
        assert a.len.tolist() == b.len.tolist(), f"n={n} len"


CHUNK_CASES = [
    # (B, Hq, Hkv, D, W, wl, chunk lengths, dtype)
    (1, 2, 2, 8, 16, 15, [40], "f32"),                  # one chunk, empty ring
    (1, 2, 1, 8, 16, 15, [7, 1, 30, 9], "bf16"),        # GQA 2, chunks < and > W
    (2, 4, 2, 8, 12, 5, [3, 20, 1, 1, 14], "bf16"),     # ring wider than the window
    (1, 2, 2, 8, 9, 9, [9, 9, 9], "f32"),               # wl == W, chunk == W
]


def pin_chunked_prefill(orc):
    """Running a prompt chunk by chunk through the ring (attend, then append)
    gives the causal window attention of the whole prompt (dense-mask brute
    force over the full sequence)."""
    for n_case, (B, Hq, Hkv, D, W, wl, chunks, dt) in enumerate(CHUNK_CASES):
        N = sum(chunks)
        q, k, v = fwd_inputs(300 + n_case, B, Hq, Hkv, N, D, dt)
        ref_o, ref_l = bruteforce.fwd(q, k, v, win_left=wl, win_right=0, scale=0.3)
        ring = _empty_ring(orc, B, Hkv, W, D, dt, [n_case % W] * B)
        p0 = 0
        for n in chunks:
            sl = slice(p0, p0 + n)
            cq, ck, cv = (np.ascontiguousarray(x[:, sl]) for x in (q, k, v))
            o, l = ring.fwd_cached(cq, ck, cv, win_left=wl, scale=0.3)
            _close(o, ref_o[:, sl], 1e-12, f"chunked prefill case {n_case} out @{p0}")
            _close(l, ref_l[:, :, sl], 1e-12, f"chunked prefill case {n_case} lse @{p0}")
            ring.append_chunk(ck, cv)
            p0 += n
        assert ring.len.tolist() == [min(N, W)] * B


def pin_prefill_then_decode(orc):
    """Chunked prefill of a prompt, then decode steps on the same ring: every
    step equals the causal window-W attention row of the whole sequence."""
    B, Hq, Hkv, D, W = 1, 4, 2, 8, 10
    chunks, steps = [6, 13], 5
    N = sum(chunks) + steps
    q, k, v = fwd_inputs(310, B, Hq, Hkv, N, D, "bf16")
    ref_o, ref_l = bruteforce.fwd(q, k, v, win_left=W - 1, win_right=0, scale=0.4)
    ring = _empty_ring(orc, B, Hkv, W, D, "bf16", [4])
    p0 = 0
    for n in chunks:
        sl = slice(p0, p0 + n)
        cq, ck, cv = (np.ascontiguousarray(x[:, sl]) for x in (q, k, v))
        o, _ = ring.fwd_cached(cq, ck, cv, win_left=W - 1, scale=0.4)
        _close(o, ref_o[:, sl], 1e-12, "prefill chunk")
        ring.append_chunk(ck, cv)
        p0 += n
    for t in range(p0, N):
        ring.append(np.ascontiguousarray(k[:, t]), np.ascontiguousarray(v[:, t]))
        o, l = ring.decode(np.ascontiguousarray(q[:, t]), scale=0.4)
        _close(o, ref_o[:, t], 1e-12, f"decode step at {t}")
        _close(l, ref_l[:, :, t], 1e-12, f"decode lse at {t}")


def pin_decode_sinks(orc):
    """Decode with the first S tokens pinned as sinks (the ring holding the
    tokens after them) equals the causal window-W forward with global tokens
    0..S-1 at every decode row (dense-mask brute force); q = 0 gives the mean
    over sinks and held ring entries; no sinks is plain decode."""
    B, Hq, Hkv, D, W, S = 2, 4, 2, 8, 6, 3
    N = 20
    q, k, v = fwd_inputs(320, B, Hq, Hkv, N, D, "bf16")
    ref_o, ref_l = bruteforce.fwd(q, k, v, win_left=W - 1, win_right=0,
                                  global_idx=list(range(S)), scale=0.35)
    ks = np.ascontiguousarray(k[:, :S].transpose(0, 2, 1, 3))
    vs = np.ascontiguousarray(v[:, :S].transpose(0, 2, 1, 3))
    ring = _empty_ring(orc, B, Hkv, W, D, "bf16", [2, 5])
    for t in range(S, N):
        ring.append(np.ascontiguousarray(k[:, t]), np.ascontiguousarray(v[:, t]))
        o, l = ring.decode(np.ascontiguousarray(q[:, t]), scale=0.35, sinks=(ks, vs))
        _close(o, ref_o[:, t], 1e-12, f"decode with sinks at {t}")
        _close(l, ref_l[:, :, t], 1e-12, f"decode with sinks lse at {t}")
    # q = 0: uniform weights over sinks and the held ring entries
    o, l = ring.decode(np.zeros((B, Hq, D), np.uint16), scale=1.0, sinks=(ks, vs))
    for b in range(B):
        held = [(int(ring.head[b]) - 1 - a) % W for a in range(int(ring.len[b]))]
        vals = np.concatenate([bruteforce.widen(vs[b]), bruteforce.widen(ring.v[b][:, held])],
                              axis=1)                         # [Hkv, S + len, D]
        for h in range(Hq):
            _close(o[b, h], vals[h // (Hq // Hkv)].mean(axis=0), 1e-12, "sinks q=0 mean")
        _close(l[b], math.log(vals.shape[1]), 1e-12, "sinks q=0 lse")
    # no sinks: the plain decode
    z = np.zeros((B, Hkv, 0, D), np.uint16)
    qd = np.ascontiguousarray(q[:, N - 1])
    o1, l1 = ring.decode(qd, scale=0.35, sinks=(z, z))
    o2, l2 = ring.decode(qd, scale=0.35)
    _close(o1, o2, 0.0, "zero sinks out")
    _close(l1, l2, 0.0, "zero sinks lse")


class _PagePool:
    """Host bookkeeping of a paged window cache: a free list shared by all
    sequences and, per sequence, the block held by each table entry.  Before
    an append it points the entries of the blocks about to be written at
    pages; a block that left the window gives its page back first."""

    def __init__(self, n_pages, B, nb, P, W, order):
        self.free = list(order)
        self.table = np.full((B, nb), -1, np.int32)
        self.block = np.full((B, nb), -1, np.int64)
        self.nb, self.P, self.W = nb, P, W

    def reserve(self, b, L, n):
        first = L + max(0, n - self.W)
        for blk in range(first // self.P, (L + n - 1) // self.P + 1):
            j = blk % self.nb
            if self.block[b, j] != blk:
                if self.table[b, j] >= 0:
                    self.free.append(int(self.table[b, j]))    # out of every window now
                self.table[b, j] = self.free.pop(0)
                self.block[b, j] = blk

    def release(self, b):
        for j in range(self.nb):
            if self.table[b, j] >= 0:
                self.free.append(int(self.table[b, j]))
        self.table[b] = -1
        self.block[b] = -1


def pin_paged_stream(orc):
    """Three sequences share a page pool smaller than their blocks; pages of
    blocks that left the window go back to the pool and are reused, also by
    other sequences.  Every decode step equals the dense-mask brute force of
    the causal window-W forward of that sequence's tokens."""
    B, Hq, Hkv, D, W, P, nb, n_pages = 3, 4, 2, 8, 10, 4, 4, 9
    N = 40
    q, k, v = fwd_inputs(330, B, Hq, Hkv, N, D, "bf16")
    ref_o, _ = bruteforce.fwd(q, k, v, win_left=W - 1, win_right=0, scale=0.3)
    rng = np.random.Generator(np.random.PCG64(331))
    pool = _PagePool(n_pages, B, nb, P, W, rng.permutation(n_pages))
    z = np.zeros((n_pages, Hkv, P, D), np.uint16)
    cache = orc.paged(z, z, [0] * B, W)
    # sequence 0 prefilled with a chunk longer than the window; 1 and 2 start empty
    plan = {0: [23, 1, 1, 1], 1: [1] * 12, 2: [5, 1, 1]}
    pos = [0] * B
    for step in range(12):
        for b in range(B):
            if step >= len(plan[b]):
                continue
            n = plan[b][step]
            pool.reserve(b, pos[b], n)
            kb = np.zeros((B, n, Hkv, D), np.uint16)
            vb = np.zeros_like(kb)
            kb[b], vb[b] = k[b, pos[b]:pos[b] + n], v[b, pos[b]:pos[b] + n]
            # one sequence per append call: the other rows append nothing
            lens = cache.len.copy()
            sub = orc.paged(cache.k, cache.v, [cache.len[b]], W)
            sub.append(kb[b:b + 1], vb[b:b + 1], pool.table[b:b + 1])
            cache.k, cache.v = sub.k, sub.v
            cache.len = lens
            cache.len[b] += n
            pos[b] += n
            qb = np.zeros((1, Hq, D), np.uint16)
            qb[0] = q[b, pos[b] - 1]
            sub = orc.paged(cache.k, cache.v, [cache.len[b]], W)
            o, _ = sub.decode(qb, pool.table[b:b + 1], scale=0.3)
            _close(o[0], ref_o[b, pos[b] - 1], 1e-12, f"paged seq {b} position {pos[b] - 1}")
        if step == 4:
            pool.release(2)                      # sequence 2 finished: all its pages return
            assert len(set(pool.free)) == len(pool.free)
    used = {int(x) for x in pool.table.reshape(-1) if x >= 0}
    assert len(used) + len(pool.free) == n_pages and not used & set(pool.free)


def pin_paged_equals_ring(orc):
    """The same token stream through a W-slot ring and through the paged cache
    gives the same decode rows; a batched paged append of several sequences at
    once equals appending them one by one."""
    B, Hq, Hkv, D, W, P, nb = 2, 2, 1, 8, 12, 8, 3
    N = 30
    q, k, v = fwd_inputs(332, B, Hq, Hkv, N, D, "f32")
    ring = _empty_ring(orc, B, Hkv, W, D, "f32", [5, 0])
    n_pages = B * nb
    cache = orc.paged(np.zeros((n_pages, Hkv, P, D), np.float32),
                      np.zeros((n_pages, Hkv, P, D), np.float32), [0] * B, W)
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)[:, ::-1].copy()  # in-place reuse
    p0 = 0
    for n in [17, 1, 1, 9, 1, 1]:
        sl = slice(p0, p0 + n)
        cache.append(np.ascontiguousarray(k[:, sl]), np.ascontiguousarray(v[:, sl]), table)
        ring.append_chunk(np.ascontiguousarray(k[:, sl]), np.ascontiguousarray(v[:, sl]))
        p0 += n
        qt = np.ascontiguousarray(q[:, p0 - 1])
        o1, l1 = cache.decode(qt, table, scale=0.2)
        o2, l2 = ring.decode(qt, scale=0.2)
        _close(o1, o2, 1e-12, f"paged vs ring at {p0}")
        _close(l1, l2, 1e-12, f"paged vs ring lse at {p0}")


# ---- backward ----------------------------------------------------------------------

BWD_CASES = [
    # (B, Hq, Hkv, N, D, wl, wr, dil, globals, dtype, scale)
    (1, 2, 2, 23, 8, 5, 0, 1, None, "f32", 0.4),            # causal
    (2, 4, 2, 31, 8, 3, 6, 1, None, "bf16", None),          # asymmetric bidirectional, GQA
    (1, 2, 1, 40, 8, 4, 0, 3, None, "bf16", 0.3),           # dilated causal, GQA 2
    (1, 2, 2, 33, 8, 2, 2, 1, [0, 9, 32], "f32", None),     # bidirectional + globals
    (1, 2, 2, 30, 8, 3, 0, 2, [4, 5, 17], "f32", 0.5),      # dilated causal + globals
]


def _torch_grads(q, k, v, dout, wl, wr, dil, G, scale):
    """Gradients by torch autograd (float64, CPU) of the dense-masked attention."""
    qf, kf, vf, gf = (torch.from_numpy(bruteforce.widen(x)) for x in (q, k, v, dout))
    qf.requires_grad_(True)
    kf.requires_grad_(True)
    vf.requires_grad_(True)
    Hq, Hkv, N = q.shape[2], k.shape[2], q.shape[1]
    rep = Hq // Hkv
    allowed = torch.from_numpy(bruteforce.mask_matrix(N, wl, wr, dil, G))
    kr = kf.repeat_interleave(rep, dim=2)
    vr = vf.repeat_interleave(rep, dim=2)
    s = scale * torch.einsum("bihd,bjhd->bhij", qf, kr)
    s = s.masked_fill(~allowed, float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), vr)
    (o * gf).sum().backward()
    return qf.grad.numpy(), kf.grad.numpy(), vf.grad.numpy()


def pin_bwd_autograd(orc):
    """Oracle gradients equal torch autograd through the dense-masked softmax."""
    for n, (B, Hq, Hkv, N, D, wl, wr, dil, G, dt, sc) in enumerate(BWD_CASES):
        q, k, v = fwd_inputs(400 + n, B, Hq, Hkv, N, D, dt)
        dout = fwd_inputs(450 + n, B, Hq, Hkv, N, D, dt)[0]
        scale = sc if sc is not None else 1 / math.sqrt(D)
        dq, dk, dv = orc.bwd(q, k, v, dout, win_left=wl, win_right=wr, dilation=dil,
                             global_idx=G, scale=scale)
        tq, tk, tv = _torch_grads(q, k, v, dout, wl, wr, dil, G, scale)
        _close(dq, tq, 1e-10, f"bwd case {n} dq")
        _close(dk, tk, 1e-10, f"bwd case {n} dk")
        _close(dv, tv, 1e-10, f"bwd case {n} dv")


def pin_bwd_finite_differences(orc):
    """Directional derivatives of L = sum(dout * out) by central differences of
    the oracle's own forward (step 2^-12 on exactly representable inputs)."""
    B, Hq, Hkv, N, D, wl, wr, dil, G = 1, 2, 1, 9, 4, 2, 1, 1, [7]
    q, k, v = fwd_inputs(460, B, Hq, Hkv, N, D, "f32")
    q, k, v = (np.round(x * 64) / 64 for x in (q, k, v))      # room for exact steps
    q, k, v = (x.astype(np.float32) for x in (q, k, v))
    dout = fwd_inputs(461, B, Hq, Hkv, N, D, "f32")[0]
    dq, dk, dv = orc.bwd(q, k, v, dout, win_left=wl, win_right=wr, dilation=dil, global_idx=G,
                         scale=0.7)
    rng = np.random.Generator(np.random.PCG64(462))
    h = 2.0 ** -12

    def loss(q_, k_, v_):
        o, _ = orc.fwd(q_, k_, v_, win_left=wl, win_right=wr, dilation=dil, global_idx=G,
                       scale=0.7)
        return float(np.sum(o * dout))

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(3):
            u = rng.integers(-1, 2, size=x.shape).astype(np.float32)   # entries in {-1, 0, 1}
            args = {"q": q, "k": k, "v": v}
            args[name] = x + h * u
            fp = loss(args["q"], args["k"], args["v"])
            args[name] = x - h * u
            fm = loss(args["q"], args["k"], args["v"])
            fd = (fp - fm) / (2 * h)
            an = float(np.sum(g * u))
            assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, fd, an)


def pin_bwd_closed_forms(orc):
    """A zero window: each query sees only itself, so P = 1, dq = dk = 0 and
    dv_i = the sum of dout_i over the kv head's query heads.  In general the
    dv rows of a kv head sum to the dout rows of its query heads (each row of
    P sums to 1)."""
    B, Hq, Hkv, N, D = 1, 4, 2, 13, 8
    q, k, v = fwd_inputs(470, B, Hq, Hkv, N, D, "bf16")
    dout = fwd_inputs(471, B, Hq, Hkv, N, D, "bf16")[0]
    dq, dk, dv = orc.bwd(q, k, v, dout, win_left=0, win_right=0)
    g = bruteforce.widen(dout).reshape(B, N, Hkv, Hq // Hkv, D).sum(axis=3)
    _close(dq, 0.0 * dq, 0.0, "zero window dq")
    _close(dk, 0.0 * dk, 0.0, "zero window dk")
    _close(dv, g, 1e-12, "zero window dv")
    dq, dk, dv = orc.bwd(q, k, v, dout, win_left=4, win_right=2, dilation=2, global_idx=[3])
    _close(dv.sum(axis=1), g.sum(axis=1), 1e-10, "dv rows sum to dout rows")


def pin_bwd_sampled(orc):
    """The row- and key-sampled backward entry points agree with the full one."""
    for n, (B, Hq, Hkv, N, D, wl, wr, dil, G, dt, sc) in enumerate(BWD_CASES[:4]):
        q, k, v = fwd_inputs(400 + n, B, Hq, Hkv, N, D, dt)
        dout = fwd_inputs(450 + n, B, Hq, Hkv, N, D, dt)[0]
        kw = dict(win_left=wl, win_right=wr, dilation=dil, global_idx=G, scale=sc)
        dq, dk, dv = orc.bwd(q, k, v, dout, **kw)
        rows = np.array([[0, 0, 0], [B - 1, Hq - 1, N - 1], [0, Hq // 2, N // 2]])
        got = orc.bwd_dq_rows(q, k, v, dout, rows, **kw)
        for r, (b, h, i) in enumerate(rows):
            _close(got[r], dq[b, i, h], 1e-12, f"sampled dq case {n}")
        sel = np.array([[0, 0, 0], [B - 1, Hkv - 1, N - 1], [0, Hkv - 1, N // 3]])
        gk, gv = orc.bwd_dkv_keys(q, k, v, dout, sel, **kw)
        for r, (b, kh, j) in enumerate(sel):
            _close(gk[r], dk[b, j, kh], 1e-12, f"sampled dk case {n}")
            _close(gv[r], dv[b, j, kh], 1e-12, f"sampled dv case {n}")


ALL_PINS = [
    pin_dilated_index_sets, pin_dilated_span, pin_edge_truncation, pin_decode_demo_window,
    pin_ring_buffer_trace, pin_bruteforce, pin_bruteforce_mask_is_page_mask, pin_full_window,
    pin_zero_window, pin_q_zero, pin_dilation_strided, pin_gqa, pin_globals, pin_decode,
    pin_append_chunk, pin_chunked_prefill, pin_prefill_then_decode, pin_decode_sinks,
    pin_paged_stream, pin_paged_equals_ring, pin_bwd_autograd, pin_bwd_finite_differences,
    pin_bwd_closed_forms, pin_bwd_sampled,
]
