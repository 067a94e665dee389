"""GPU parity of swa_kv_append + swa_decode against the oracle's own ring.

Each step appends one token per sequence on the device and attends the new
query over the valid ring slots; the oracle applies the same append to its
copy and evaluates the definition in fp64.  The ring contents and the
head/length counters must match bit for bit; out and lse within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding, configs
from sliding_window_attention_tiled_amd.inputs import DecodeInputs
from tests.gpu_util import bits, check, log, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _ring_on_device(gen):
    kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
    head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
    length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
    return kc, vc, head, length


def _run_steps(gen, steps, check_steps, dt, what, scale=None):
    kc, vc, head, length = _ring_on_device(gen)
    ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
    ws = torch.empty(binding.decode_workspace_size(gen.B, gen.Hq, gen.W, gen.D),
                     dtype=torch.uint8, device="cuda")
    for t in range(steps):
        qn, kn, vn = gen.step()
        qd, kd, vd = to_dev(qn), to_dev(kn), to_dev(vn)
        binding.kv_append(kc, vc, kd, vd, head, length)
        out, lse = binding.decode(qd, kc, vc, head, length, scale=scale, workspace=ws)
        ring.append(kn, vn)
        if t in check_steps:
            torch.cuda.synchronize()
            log(f"[decode] {what} step {t}")
            ref_o, ref_l = ring.decode(qn, scale=scale)
            check(to_host_f64(out), ref_o, dt, f"{what} step {t} out")
            check(to_host_f64(lse), ref_l, dt, f"{what} step {t} lse")
            assert np.array_equal(head.cpu().numpy(), ring.head)
            assert np.array_equal(length.cpu().numpy(), ring.len)
    torch.cuda.synchronize()
    if dt == "bf16":
        assert np.array_equal(bits(kc), ring.k) and np.array_equal(bits(vc), ring.v)
    else:
        assert np.array_equal(kc.cpu().numpy(), ring.k) and np.array_equal(vc.cpu().numpy(), ring.v)


SMALL = [
    # name, B, Hq, Hkv, W, D, dtype, initial fill (None = full)
    ("full_gqa4", 3, 8, 2, 256, 128, "bf16", None),
    ("partial_gqa4", 4, 8, 2, 300, 128, "bf16", 5),
    ("empty_start_d64", 2, 4, 4, 200, 64, "bf16", 0),
    ("gqa16", 2, 16, 1, 512, 128, "bf16", 100),
    ("gqa32_two_head_blocks", 1, 32, 1, 256, 64, "bf16", None),
    ("f32_partial", 3, 4, 2, 130, 128, "f32", 7),
    ("f32_full_d64", 2, 6, 3, 64, 64, "f32", None),
    ("tiny_ring", 2, 2, 1, 3, 128, "bf16", 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_decode_small(case):
    name, B, Hq, Hkv, W, D, dt, fill = case
    gen = DecodeInputs(11, B, Hq, Hkv, W, D, dt, fill=fill)
    steps = 12
    _run_steps(gen, steps, set(range(steps)), dt, name, scale=0.1 if dt == "f32" else None)


def test_decode_full_rolling_cache():
    c = configs.DECODE
    gen = DecodeInputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["W"], c["D"], c["dtype"])
    steps = c["steps"]
    _run_steps(gen, steps, {0, 1, 100, 200, steps - 1}, c["dtype"], "rolling cache")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_never_reads_stale_slots(dt):
    """Slots that hold no entry (age >= cache_len) may contain anything,
    NaN and infinities included: the result must equal the oracle's, which
    attends only the live entries.  Live ranges wrap around slot 0, and one
    sequence holds a single entry."""
    B, Hq, Hkv, W, D = 3, 8, 2, 300, 128
    rng = np.random.Generator(np.random.PCG64(81))
    ring_head = np.array([5, 290, 0], np.int32)
    cache_len = np.array([37, 299, 1], np.int32)
    shape = (B, Hkv, W, D)
    kc = rng.standard_normal(shape, dtype=np.float32)
    vc = rng.standard_normal(shape, dtype=np.float32)
    q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    poison = np.array([np.nan, np.inf, -np.inf], np.float32)
    for b in range(B):
        for s in range(W):
            age = (ring_head[b] - 1 - s) % W
            if age >= cache_len[b]:
                kc[b, :, s] = poison[s % 3]
                vc[b, :, s] = poison[(s + 1) % 3]
    if dt == "bf16":
        from sliding_window_attention_tiled_amd.inputs import to_bf16_bits
        kc, vc, q = to_bf16_bits(kc), to_bf16_bits(vc), to_bf16_bits(q)
    log(f"[decode] stale slots poisoned, {dt}")
    ring = oracle.ring(kc, vc, ring_head, cache_len)
    ref_o, ref_l = ring.decode(q)
    out, lse = binding.decode(to_dev(q), to_dev(kc), to_dev(vc),
                              torch.from_numpy(ring_head).to("cuda"),
                              torch.from_numpy(cache_len).to("cuda"))
    torch.cuda.synchronize()
    check(to_host_f64(out), ref_o, dt, f"stale-slot decode {dt} out")
    check(to_host_f64(lse), ref_l, dt, f"stale-slot decode {dt} lse")
