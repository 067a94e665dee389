"""GPU parity of swa_fwd against the fp64 CPU oracle.

* small and ragged shapes (several tiles plus a ragged tail) compared element
  by element on every row;
* the full-size workloads compared on sampled rows (edges, ramps, global rows
  and a seeded uniform sample), in the launch configuration the bench times;
* attended index sets checked bit-exactly through the production kernels with
  a one-hot value probe (q = 0 makes every weight 1/|S(i)|, so out[i][c] is
  non-zero exactly when key j0 + c is attended);
* every output row written, and results bitwise reproducible.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding, configs
from sliding_window_attention_tiled_amd.inputs import fwd_inputs, to_bf16_bits
from tests.gpu_util import bits, check, log, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

# name, B, Hq, Hkv, N, D, dtype, win_left, win_right, dilation, globals, scale
SMALL = [
    ("tiny_causal_w64_f32", 1, 2, 2, 256, 64, "f32", 63, 0, 1, None, 1 / 8),
    ("causal_gqa4", 1, 8, 2, 1000, 128, "bf16", 299, 0, 1, None, None),
    ("causal_gqa4_d64_b2", 2, 4, 1, 515, 64, "bf16", 130, 0, 1, None, None),
    ("bidir_globals_d64", 2, 3, 3, 777, 64, "bf16", 50, 50, 1, [0, 100, 776, 100, 333], None),
    ("bidir_asym_gqa2", 1, 4, 2, 650, 128, "bf16", 37, 90, 1, None, 0.05),
    ("dilated3_causal", 1, 2, 2, 1500, 128, "bf16", 100, 0, 3, None, None),
    ("dilated4_bidir_globals", 1, 4, 4, 1201, 64, "bf16", 20, 20, 4, [0, 5, 600, 1200], None),
    ("causal_globals_gqa4", 1, 4, 1, 900, 128, "bf16", 64, 0, 1, [0, 7, 450, 899], None),
    ("window_ge_n", 1, 2, 2, 300, 128, "bf16", 1000, 1000, 1, None, None),
    ("causal_window_ge_n", 1, 2, 2, 300, 64, "bf16", 5000, 0, 1, None, None),
    ("zero_window", 1, 2, 2, 130, 64, "bf16", 0, 0, 1, None, None),
    ("n1", 1, 4, 4, 1, 128, "bf16", 5, 0, 1, None, None),
    ("n2_bidir_global", 2, 2, 1, 2, 64, "bf16", 5, 5, 1, [1], None),
    ("gqa8", 1, 16, 2, 300, 128, "bf16", 50, 0, 1, None, None),
    ("bidir_dilated2_gqa4", 1, 8, 2, 1100, 128, "bf16", 70, 45, 2, None, None),
    ("window_ge_n_gqa4", 2, 4, 1, 300, 128, "bf16", 1000, 1000, 1, None, None),
    ("n3_causal_gqa4", 1, 4, 1, 3, 128, "bf16", 8, 0, 1, None, None),
    ("zero_window_gqa4", 1, 8, 2, 200, 128, "bf16", 0, 0, 1, None, None),
    ("gqa3", 1, 6, 2, 300, 64, "bf16", 50, 10, 1, None, None),
    ("many_globals_256", 1, 2, 2, 2048, 64, "bf16", 16, 16, 1, list(range(0, 2048, 8)), None),
    ("dilation_gt_n", 1, 2, 2, 100, 64, "bf16", 3, 3, 150, [7], None),
    ("f32_bidir_globals", 1, 3, 3, 333, 128, "f32", 40, 40, 1, [0, 100], None),
    ("f32_dilated_gqa", 1, 4, 2, 400, 64, "f32", 30, 0, 2, None, None),
    ("f32_causal_globals", 1, 2, 1, 257, 128, "f32", 17, 0, 1, [0, 128, 256], None),
]


def _run(q, k, v, **kw):
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"), device="cuda")
    binding.fwd(qd, kd, vd, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fwd_small_all_rows(case):
    name, B, Hq, Hkv, N, D, dt, wl, wr, dil, G, sc = case
    q, k, v = fwd_inputs(zlib.crc32(name.encode()) % 1000, B, Hq, Hkv, N, D, dt)
    kw = dict(win_left=wl, win_right=wr, dilation=dil, global_idx=G, scale=sc)
    ref_o, ref_l = oracle.fwd(q, k, v, **kw)
    log(f"[fwd small] {name} B={B} Hq={Hq} Hkv={Hkv} N={N} D={D} {dt} wl={wl} wr={wr} d={dil} G={G}")
    out, lse = _run(q, k, v, **kw)
    check(to_host_f64(out), ref_o, dt, f"{name} out")
    check(to_host_f64(lse), ref_l, dt, f"{name} lse")


def _sample_rows(B, Hq, N, seed, extra_positions=(), n_random=192):
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = set([0, 1, 2, N // 2, N - 2, N - 1]) | set(int(x) for x in extra_positions if 0 <= x < N)
    rows = []
    for i in sorted(pos):
        for b in {0, B - 1}:
            for h in {0, Hq // 2, Hq - 1}:
                rows.append((b, h, i))
    rb = rng.integers(0, B, n_random)
    rh = rng.integers(0, Hq, n_random)
    ri = rng.integers(0, N, n_random)
    rows += list(zip(rb.tolist(), rh.tolist(), ri.tolist()))
    return np.array(rows, np.int64)


def _check_rows(out, lse, q, k, v, rows, dt, what, **kw):
    ref_o, ref_l = oracle.fwd_rows(q, k, v, rows, **kw)
    o = out[rows[:, 0], rows[:, 2], rows[:, 1]]     # out is [B,N,Hq,D]
    l = lse[rows[:, 0], rows[:, 1], rows[:, 2]]     # lse is [B,Hq,N]
    print(check(to_host_f64(o), ref_o, dt, f"{what} out"))
    print(check(to_host_f64(l), ref_l, dt, f"{what} lse"))


def test_fwd_full_mistral_causal_w4096():
    c = configs.FWD["mistral_causal_w4096"]
    q, k, v = fwd_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["D"], c["dtype"])
    kw = dict(win_left=c["win_left"], win_right=c["win_right"], dilation=c["dilation"])
    log("[fwd full] mistral_causal_w4096")
    out, lse = _run(q, k, v, **kw)
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    rows = _sample_rows(c["B"], c["Hq"], c["N"], 21,
                        extra_positions=[31, 32, 4094, 4095, 4096, 4097, 8191, 12000])
    _check_rows(out, lse, q, k, v, rows, "bf16", "mistral", **kw)


def test_fwd_full_bidir_encoder_globals():
    c = configs.FWD["bidir_encoder_globals"]
    q, k, v = fwd_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["D"], c["dtype"])
    kw = dict(win_left=c["win_left"], win_right=c["win_right"], dilation=c["dilation"],
              global_idx=c["global_idx"])
    log("[fwd full] bidir_encoder_globals")
    out, lse = _run(q, k, v, **kw)
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    G = c["global_idx"]
    rows = _sample_rows(c["B"], c["Hq"], c["N"], 31,
                        extra_positions=G + [255, 256, 257, 511, 513, 7935, 7936, 8190])
    _check_rows(out, lse, q, k, v, rows, "bf16", "bidir", **kw)


@pytest.mark.parametrize("dil", configs.DILATED_STACK["dilations"])
def test_fwd_full_dilated_stack(dil):
    c = configs.DILATED_STACK
    q, k, v = fwd_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["D"], c["dtype"])
    kw = dict(win_left=c["win_left"], win_right=c["win_right"], dilation=dil)
    log(f"[fwd full] dilated stack d={dil}")
    out, lse = _run(q, k, v, **kw)
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    rows = _sample_rows(c["B"], c["Hq"], c["N"], 40 + dil, n_random=128,
                        extra_positions=[dil - 1, dil, 511 * dil, 511 * dil + 1, 32767 - dil])
    _check_rows(out, lse, q, k, v, rows, "bf16", f"dilated d={dil}", **kw)


# ---- attended index sets, bit-exact ------------------------------------------------

PROBES = [
    # name, N, Hq, Hkv, D, win_left, win_right, dilation, globals
    ("causal", 700, 2, 1, 128, 100, 0, 1, None),
    ("causal_gqa4", 700, 4, 1, 128, 100, 0, 1, None),
    ("dilated2_bidir_gqa4", 650, 4, 1, 128, 30, 17, 2, None),
    ("bidir_globals", 600, 1, 1, 64, 40, 40, 1, [0, 300, 599]),
    ("dilated3_globals", 650, 1, 1, 128, 30, 10, 3, [5, 400]),
    ("dilated8_causal_sink", 513, 4, 1, 128, 20, 0, 8, [0]),
    ("causal_globals", 400, 1, 1, 64, 33, 0, 1, [3, 200, 201]),
]


@pytest.mark.parametrize("probe", PROBES, ids=[p[0] for p in PROBES])
def test_attended_sets_bit_exact(probe):
    name, N, Hq, Hkv, D, wl, wr, dil, G = probe
    q = torch.zeros(1, N, Hq, D, dtype=torch.bfloat16, device="cuda")
    k = to_dev(fwd_inputs(5, 1, Hq, Hkv, N, D, "bf16")[1])
    got = [[set() for _ in range(N)] for _ in range(Hq)]
    log(f"[index probe] {name}")
    lse_all = None
    for j0 in range(0, N, D):
        v = torch.zeros(1, N, Hkv, D, dtype=torch.bfloat16, device="cuda")
        n = min(D, N - j0)
        v[0, j0:j0 + n, :, :n] = torch.eye(n, dtype=torch.bfloat16, device="cuda")[:, None, :]
        out, lse = binding.fwd(q, k, v, win_left=wl, win_right=wr, dilation=dil, global_idx=G)
        torch.cuda.synchronize()
        nz = (out[0, :, :, :n] != 0).cpu().numpy()       # [N, Hq, n]
        for h in range(Hq):
            ii, cc = np.nonzero(nz[:, h, :])
            for i, cidx in zip(ii.tolist(), cc.tolist()):
                got[h][i].add(j0 + cidx)
        lse_all = lse.cpu().numpy()
    for i in range(N):
        want = set(oracle.attended_set(i, N, wl, wr, dil, G))
        for h in range(Hq):
            assert got[h][i] == want, f"{name} row {i} head {h}: " \
                f"extra {sorted(got[h][i] - want)[:8]} missing {sorted(want - got[h][i])[:8]}"
            assert abs(lse_all[0, h, i] - math.log(len(want))) < 1e-5


def test_fwd_deterministic():
    B, Hq, Hkv, N, D = 1, 8, 2, 1200, 128
    q, k, v = (to_dev(x) for x in fwd_inputs(77, B, Hq, Hkv, N, D, "bf16"))
    log("[fwd determinism]")
    G = [0, 600]
    o1, l1 = binding.fwd(q, k, v, win_left=200, win_right=30, global_idx=G)
    o2, l2 = binding.fwd(q, k, v, win_left=200, win_right=30, global_idx=G)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))
    assert torch.equal(l1, l2)


def test_fwd_nan_propagation():
    """A NaN in v reaches every row whose window holds that key; rows of other
    heads and rows far from the key stay finite.  (A masked key still meets a
    zero weight inside its tile, and 0 * NaN is NaN, so rows sharing the tile
    may see it too: inputs are expected to be finite.)"""
    B, Hq, Hkv, N, D = 1, 2, 2, 1000, 64
    q, k, v = fwd_inputs(78, B, Hq, Hkv, N, D, "bf16")
    v = v.copy()
    v[0, 150, 0, 3] = to_bf16_bits(np.array([np.nan], np.float32))[0]
    log("[fwd nan propagation]")
    out, _ = _run(q, k, v, win_left=10, win_right=0, scale=0.3)
    o = to_host_f64(out)
    for i in range(150, 161):
        assert np.isnan(o[0, i, 0, 3]), i
    assert not np.isnan(o[0, 600:, 0]).any()
    assert not np.isnan(o[0, :, 1]).any()
