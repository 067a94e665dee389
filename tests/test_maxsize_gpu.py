"""The largest sizes the C ABI accepts: N = SWA_MAX_N (2^28) positions for the
forward, a 2^28-slot ring for append and decode (one head dimension of 64,
one kv head, so that q, k, v and out fit in HBM: 32 GiB each).

Inputs are drawn on the device from a seeded generator.  The oracle checks
sampled rows: a row's window is translation invariant away from the
sequence ends, so each sampled row is evaluated on the slice of the
sequence that holds its window (the true ends included where the window
reaches them), copied to the host.  The decode check gives the oracle the
live entries of the ring in age order.  Index arithmetic that overflowed 32
bits anywhere on these paths would show up as wrong rows near the end."""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding
from tests.gpu_util import check, log, to_host_f64

pytestmark = pytest.mark.gpu

SWA_MAX_N = 1 << 28


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _normal_bf16(shape, gen):
    x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    step = 1 << 26
    flat = x.view(-1)
    for i in range(0, flat.numel(), step):
        flat[i:i + step].normal_(generator=gen)
    return x


# (the ring test runs first and frees its 64 GiB before the forward tests draw
# their 96 GiB of inputs, so that at most about 130 GiB are held at once)
def test_append_and_decode_on_max_ring():
    torch.cuda.empty_cache()
    B, Hq, Hkv, W, D = 1, 8, 1, SWA_MAX_N, 64
    gen = torch.Generator(device="cuda").manual_seed(77)
    log("[maxsize] ring of 2^28 slots: drawing K and V")
    kc = _normal_bf16((B, Hkv, W, D), gen)
    vc = _normal_bf16((B, Hkv, W, D), gen)
    head = torch.tensor([2000], dtype=torch.int32, device="cuda")
    length = torch.tensor([4999], dtype=torch.int32, device="cuda")
    k_new = _normal_bf16((B, Hkv, D), gen)
    v_new = _normal_bf16((B, Hkv, D), gen)
    binding.kv_append(kc, vc, k_new, v_new, head, length)
    torch.cuda.synchronize()
    assert head.cpu().tolist() == [2001] and length.cpu().tolist() == [5000]
    assert torch.equal(kc[0, 0, 2000].view(torch.int16), k_new[0, 0].view(torch.int16))
    assert torch.equal(vc[0, 0, 2000].view(torch.int16), v_new[0, 0].view(torch.int16))
    q = _normal_bf16((B, Hq, D), gen)
    log("[maxsize] decode over 5000 live entries wrapping slot 0 of a 2^28-slot ring")
    out, lse = binding.decode(q, kc, vc, head, length)
    torch.cuda.synchronize()
    # the live entries in age order (age a at slot (head - 1 - a) mod W), as a
    # ring of their own: W' = 5000, head' = 0, age a at slot 4999 - a
    L = 5000
    ages = torch.arange(L, device="cuda")
    slots = (2001 - 1 - ages) % W
    order = torch.flip(slots, [0])          # slot of age L-1-j at position j
    ks = _bits(kc[:, :, order])
    vs = _bits(vc[:, :, order])
    ring = oracle.ring(ks, vs, np.array([0], np.int32), np.array([L], np.int32))
    ref_o, ref_l = ring.decode(_bits(q))
    check(to_host_f64(out), ref_o, "bf16", "2^28-slot ring decode out")
    check(to_host_f64(lse), ref_l, "bf16", "2^28-slot ring decode lse")
    del kc, vc
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def big_qkv():
    torch.cuda.empty_cache()
    gen = torch.Generator(device="cuda").manual_seed(2024)
    shape = (1, SWA_MAX_N, 1, 64)
    log("[maxsize] drawing q, k, v at N = 2^28, D = 64")
    q, k, v = (_normal_bf16(shape, gen) for _ in range(3))
    yield q, k, v
    del q, k, v
    torch.cuda.empty_cache()


def _check_rows(q, k, v, out, lse, rows, wl, wr, dil, what):
    N = q.shape[1]
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for i in rows:
        s = max(0, i - wl * dil)
        e = min(N - 1, i + wr * dil)
        qs, ks, vs = (_bits(t[:, s:e + 1]) for t in (q, k, v))
        o, lv = oracle.fwd_rows(qs, ks, vs, np.array([[0, 0, i - s]], np.int64),
                                win_left=wl, win_right=wr, dilation=dil)
        ref_o.append(o[0])
        ref_l.append(lv[0])
        got_o.append(to_host_f64(out[0, i, 0]))
        got_l.append(float(lse[0, 0, i]))
    check(np.stack(got_o), np.stack(ref_o), "bf16", f"{what} out")
    check(np.array(got_l), np.array(ref_l), "bf16", f"{what} lse")


def _rows(N, seed, n_random=40):
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 2, 100, 101, (1 << 27) - 1, 1 << 27, (1 << 27) + 1, N - 101, N - 3, N - 2,
             N - 1]
    return sorted(set(fixed + rng.integers(0, N, n_random).tolist()))


def test_fwd_at_max_sequence_length_causal(big_qkv):
    q, k, v = big_qkv
    log("[maxsize] fwd causal window 101 at N = 2^28")
    out, lse = binding.fwd(q, k, v, win_left=100)
    torch.cuda.synchronize()
    _check_rows(q, k, v, out, lse, _rows(SWA_MAX_N, 1), 100, 0, 1, "N = 2^28 causal")
    del out, lse


def test_fwd_at_max_sequence_length_dilated_bidirectional(big_qkv):
    q, k, v = big_qkv
    log("[maxsize] fwd bidirectional 40 + 30, dilation 3, at N = 2^28")
    out, lse = binding.fwd(q, k, v, win_left=40, win_right=30, dilation=3)
    torch.cuda.synchronize()
    _check_rows(q, k, v, out, lse, _rows(SWA_MAX_N, 2), 40, 30, 3, "N = 2^28 dilated")
    del out, lse
