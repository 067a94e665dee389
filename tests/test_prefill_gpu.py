"""GPU parity of the prefill-to-ring hand-off: swa_kv_append_chunk and
swa_fwd_cached against the oracle's ring.

A chunk append must leave the ring and its counters bit-identical to the
oracle's; a cached forward (a prompt chunk attending to the ring's tokens and
to itself) must match the oracle's definition within the dtype tolerance.
Chains of chunks followed by decode steps check the whole hand-off, and the
full-size case compares sampled rows with the oracle's row evaluation of the
same keys laid out as one contiguous sequence.
"""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding, configs
from sliding_window_attention_tiled_amd.inputs import DecodeInputs, fwd_inputs
from tests.gpu_util import bits, check, log, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _device_ring(gen):
    return (to_dev(gen.kcache), to_dev(gen.vcache),
            torch.from_numpy(gen.ring_head.copy()).to("cuda"),
            torch.from_numpy(gen.cache_len.copy()).to("cuda"))


def _assert_ring_equal(kc, vc, head, length, ring, dt, what):
    torch.cuda.synchronize()
    if dt == "bf16":
        assert np.array_equal(bits(kc), ring.k), f"{what}: K ring differs"
        assert np.array_equal(bits(vc), ring.v), f"{what}: V ring differs"
    else:
        assert np.array_equal(kc.cpu().numpy(), ring.k), f"{what}: K ring differs"
        assert np.array_equal(vc.cpu().numpy(), ring.v), f"{what}: V ring differs"
    assert np.array_equal(head.cpu().numpy(), ring.head), f"{what}: ring_head"
    assert np.array_equal(length.cpu().numpy(), ring.len), f"{what}: cache_len"


APPEND = [
    # name, B, Hkv, W, D, dtype, initial fill, chunk lengths
    ("bf16_mixed", 3, 2, 100, 128, "bf16", 40, [1, 37, 100, 0, 263, 5]),
    ("f32_d64", 2, 4, 64, 64, "f32", 0, [64, 3, 130]),
    ("one_slot_ring", 2, 1, 1, 128, "bf16", 1, [1, 4]),
]


@pytest.mark.parametrize("case", APPEND, ids=[c[0] for c in APPEND])
def test_kv_append_chunk(case):
    name, B, Hkv, W, D, dt, fill, chunks = case
    gen = DecodeInputs(21, B, 1, Hkv, W, D, dt, fill=fill)
    kc, vc, head, length = _device_ring(gen)
    ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
    for i, n in enumerate(chunks):
        _, k, v = fwd_inputs(400 + i, B, 1, Hkv, n, D, dt)
        log(f"[append_chunk] {name} chunk {i} n={n}")
        binding.kv_append_chunk(kc, vc, to_dev(k), to_dev(v), head, length)
        ring.append_chunk(k, v)
        _assert_ring_equal(kc, vc, head, length, ring, dt, f"{name} chunk {i}")


CACHED = [
    # name, B, Hq, Hkv, W, D, dtype, fill, n, win_left
    ("gqa4_full_ring", 2, 8, 2, 300, 128, "bf16", None, 200, 300),
    ("gqa4_partial_ring", 2, 8, 2, 300, 128, "bf16", 77, 131, 299),
    ("gqa2_empty_ring", 1, 4, 2, 256, 64, "bf16", 0, 190, 255),
    ("mha_short_window", 2, 3, 3, 500, 64, "bf16", 450, 260, 70),
    ("gqa4_chunk_longer_than_ring", 1, 4, 1, 96, 128, "bf16", 96, 333, 96),
    ("f32_gqa2", 2, 4, 2, 160, 128, "f32", 100, 150, 159),
    ("f32_d64_full", 1, 2, 2, 64, 64, "f32", None, 97, 64),
    ("window_zero", 1, 4, 4, 32, 64, "bf16", 32, 70, 0),
]


@pytest.mark.parametrize("case", CACHED, ids=[c[0] for c in CACHED])
def test_fwd_cached(case):
    name, B, Hq, Hkv, W, D, dt, fill, n, wl = case
    gen = DecodeInputs(31, B, 1, Hkv, W, D, dt, fill=fill)
    q, k, v = fwd_inputs(32, B, Hq, Hkv, n, D, dt)
    kc, vc, head, length = _device_ring(gen)
    scale = 0.1 if dt == "f32" else None
    log(f"[fwd_cached] {name}")
    out, lse = binding.fwd_cached(to_dev(q), to_dev(k), to_dev(v), kc, vc, head, length,
                                  win_left=wl, scale=scale)
    torch.cuda.synchronize()
    ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
    ref_o, ref_l = ring.fwd_cached(q, k, v, win_left=wl, scale=scale)
    check(to_host_f64(out), ref_o, dt, f"{name} out")
    check(to_host_f64(lse), ref_l, dt, f"{name} lse")
    # the ring is read only
    _assert_ring_equal(kc, vc, head, length, ring, dt, f"{name} ring untouched")


def test_chunked_prefill_then_decode():
    """Prompt in uneven chunks (attend, then append), then decode steps; each
    stage against the oracle running the same chain on its own ring."""
    B, Hq, Hkv, W, D, dt = 2, 8, 2, 192, 128, "bf16"
    gen = DecodeInputs(41, B, Hq, Hkv, W, D, dt, fill=0)
    kc, vc, head, length = _device_ring(gen)
    ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
    ws = torch.empty(binding.decode_workspace_size(B, Hq, W, D), dtype=torch.uint8,
                     device="cuda")
    for i, n in enumerate([130, 64, 1, 250]):
        q, k, v = fwd_inputs(500 + i, B, Hq, Hkv, n, D, dt)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        log(f"[prefill chain] chunk {i} n={n}")
        out, lse = binding.fwd_cached(qd, kd, vd, kc, vc, head, length, win_left=W - 1)
        binding.kv_append_chunk(kc, vc, kd, vd, head, length)
        torch.cuda.synchronize()
        ref_o, ref_l = ring.fwd_cached(q, k, v, win_left=W - 1)
        ring.append_chunk(k, v)
        check(to_host_f64(out), ref_o, dt, f"chunk {i} out")
        check(to_host_f64(lse), ref_l, dt, f"chunk {i} lse")
        _assert_ring_equal(kc, vc, head, length, ring, dt, f"chunk {i}")
    for t in range(6):
        qn, kn, vn = gen.step()
        log(f"[prefill chain] decode step {t}")
        binding.kv_append(kc, vc, to_dev(kn), to_dev(vn), head, length)
        out, lse = binding.decode(to_dev(qn), kc, vc, head, length, workspace=ws)
        torch.cuda.synchronize()
        ring.append(kn, vn)
        ref_o, ref_l = ring.decode(qn)
        check(to_host_f64(out), ref_o, dt, f"decode {t} out")
        check(to_host_f64(lse), ref_l, dt, f"decode {t} lse")


def test_fwd_cached_full_size_sampled():
    """A 4096-token chunk after a full 4096-slot ring, Mistral-shaped heads:
    sampled rows against the oracle evaluating them over the ring's tokens and
    the chunk laid out as one contiguous sequence."""
    c = configs.PREFILL_CHUNK
    B, Hq, Hkv, W, D, dt, n, wl = (c[x] for x in ("B", "Hq", "Hkv", "W", "D", "dtype",
                                                   "chunk", "win_left"))
    gen = DecodeInputs(c["seed"], B, Hq, Hkv, W, D, dt)
    q, k, v = fwd_inputs(c["seed"] + 100, B, Hq, Hkv, n, D, dt)
    kc, vc, head, length = _device_ring(gen)
    log("[fwd_cached] full-size chunk")
    out, lse = binding.fwd_cached(to_dev(q), to_dev(k), to_dev(v), kc, vc, head, length,
                                  win_left=wl)
    torch.cuda.synchronize()
    # logical sequence: ring entries oldest first, then the chunk
    L = int(gen.cache_len[0])
    slots = [(int(gen.ring_head[0]) - L + a) % W for a in range(L)]
    k_seq = np.concatenate([gen.kcache[:, :, slots].transpose(0, 2, 1, 3), k], axis=1)
    v_seq = np.concatenate([gen.vcache[:, :, slots].transpose(0, 2, 1, 3), v], axis=1)
    q_seq = np.concatenate([np.zeros((B, L, Hq, D), q.dtype), q], axis=1)
    rng = np.random.Generator(np.random.PCG64(7))
    ts = sorted(set([0, 1, 63, 64, 2047, n - 1] + rng.integers(0, n, 40).tolist()))
    rows = np.array([[0, int(rng.integers(0, Hq)), L + t] for t in ts] +
                    [[0, Hq - 1, L + t] for t in (0, n - 1)])
    ref_o, ref_l = oracle.fwd_rows(np.ascontiguousarray(q_seq), np.ascontiguousarray(k_seq),
                                   np.ascontiguousarray(v_seq), rows, win_left=wl, win_right=0)
    o = to_host_f64(out)
    l = to_host_f64(lse)
    got_o = np.stack([o[b, i - L, h] for b, h, i in rows])
    got_l = np.array([l[b, h, i - L] for b, h, i in rows])
    check(got_o, ref_o, dt, "full-size chunk sampled out")
    check(got_l, ref_l, dt, "full-size chunk sampled lse")
