"""GPU parity of swa_decode_sinks: decode over the ring plus attention-sink
entries kept beside it, against the oracle's ring with the same sinks.

Covers rings that are empty, partial and full next to the sinks, fp32 and
bf16, GQA groups up to 16, no sinks (the plain decode), the full-size rolling
cache with four sinks, and the whole stream: a prompt prefilled with its first
tokens as global positions, the sinks and the ring filled by chunk appends,
then decode steps.
"""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding, configs
from sliding_window_attention_tiled_amd.inputs import DecodeInputs, fwd_inputs
from tests.gpu_util import check, log, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _sinks(seed, B, Hkv, S, D, dt):
    _, k, v = fwd_inputs(seed, B, 1, Hkv, S, D, dt)
    return (np.ascontiguousarray(k.transpose(0, 2, 1, 3)),
            np.ascontiguousarray(v.transpose(0, 2, 1, 3)))


CASES = [
    # name, B, Hq, Hkv, W, D, dtype, fill, n_sink
    ("gqa4_partial", 3, 8, 2, 200, 128, "bf16", 37, 4),
    ("gqa4_empty_ring", 2, 8, 2, 256, 128, "bf16", 0, 4),
    ("gqa16_full", 2, 16, 1, 300, 64, "bf16", None, 7),
    ("mha_many_sinks", 2, 4, 4, 128, 64, "bf16", 100, 130),
    ("no_sinks", 2, 8, 2, 200, 128, "bf16", 150, 0),
    ("f32_partial", 2, 4, 2, 96, 128, "f32", 50, 3),
    ("f32_empty_ring", 1, 2, 1, 64, 64, "f32", 0, 5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_sinks(case):
    name, B, Hq, Hkv, W, D, dt, fill, S = case
    gen = DecodeInputs(51, B, Hq, Hkv, W, D, dt, fill=fill)
    ks, vs = _sinks(52, B, Hkv, S, D, dt)
    kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
    head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
    length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
    ksd, vsd = to_dev(ks), to_dev(vs)
    ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
    scale = 0.1 if dt == "f32" else None
    for t in range(4):
        qn, kn, vn = gen.step()
        log(f"[decode_sinks] {name} step {t}")
        binding.kv_append(kc, vc, to_dev(kn), to_dev(vn), head, length)
        out, lse = binding.decode_sinks(to_dev(qn), kc, vc, head, length, ksd, vsd, scale=scale)
        torch.cuda.synchronize()
        ring.append(kn, vn)
        ref_o, ref_l = ring.decode(qn, scale=scale, sinks=(ks, vs))
        check(to_host_f64(out), ref_o, dt, f"{name} step {t} out")
        check(to_host_f64(lse), ref_l, dt, f"{name} step {t} lse")


def test_decode_sinks_full_size():
    c = configs.DECODE
    B, Hq, Hkv, W, D, dt = c["B"], c["Hq"], c["Hkv"], c["W"], c["D"], c["dtype"]
    gen = DecodeInputs(c["seed"], B, Hq, Hkv, W, D, dt)
    ks, vs = _sinks(53, B, Hkv, 4, D, dt)
    kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
    head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
    length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
    ksd, vsd = to_dev(ks), to_dev(vs)
    ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
    ws = torch.empty(binding.decode_sinks_workspace_size(B, Hq, W, D, 4), dtype=torch.uint8,
                     device="cuda")
    for t in range(3):
        qn, kn, vn = gen.step()
        log(f"[decode_sinks] full size step {t}")
        binding.kv_append(kc, vc, to_dev(kn), to_dev(vn), head, length)
        out, lse = binding.decode_sinks(to_dev(qn), kc, vc, head, length, ksd, vsd, workspace=ws)
        torch.cuda.synchronize()
        ring.append(kn, vn)
        ref_o, ref_l = ring.decode(qn, sinks=(ks, vs))
        check(to_host_f64(out), ref_o, dt, f"full size step {t} out")
        check(to_host_f64(lse), ref_l, dt, f"full size step {t} lse")


def test_stream_with_sinks():
    """Prompt of N tokens: swa_fwd with global positions 0..S-1 (the sinks);
    the first S tokens' K/V into the sink buffers, the rest into the ring (chunk
    appends); then decode steps over ring + sinks.  Every stage against the
    oracle; the decode rows also against the oracle's forward over the whole
    sequence with the same global positions."""
    B, Hq, Hkv, D, W, S, N, steps, dt = 2, 8, 2, 128, 160, 4, 300, 5, "bf16"
    q, k, v = fwd_inputs(61, B, Hq, Hkv, N + steps, D, dt)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sinks = list(range(S))
    log("[stream with sinks] prefill")
    out, lse = binding.fwd(qd[:, :N].contiguous(), kd[:, :N].contiguous(),
                           vd[:, :N].contiguous(), win_left=W - 1, global_idx=sinks)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd(np.ascontiguousarray(q[:, :N]), np.ascontiguousarray(k[:, :N]),
                              np.ascontiguousarray(v[:, :N]), win_left=W - 1, global_idx=sinks)
    check(to_host_f64(out), ref_o, dt, "prefill out")
    check(to_host_f64(lse), ref_l, dt, "prefill lse")
    # sink buffers: a ring of S slots from head 0 receives tokens 0..S-1 in order
    ksd = torch.empty((B, Hkv, S, D), dtype=torch.bfloat16, device="cuda")
    vsd = torch.empty_like(ksd)
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    binding.kv_append_chunk(ksd, vsd, kd[:, :S].contiguous(), vd[:, :S].contiguous(),
                            zero.clone(), zero.clone())
    kc = torch.zeros((B, Hkv, W, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    head = torch.tensor([7, 100], dtype=torch.int32, device="cuda")
    length = torch.zeros(B, dtype=torch.int32, device="cuda")
    binding.kv_append_chunk(kc, vc, kd[:, S:N].contiguous(), vd[:, S:N].contiguous(), head,
                            length)
    ks = np.ascontiguousarray(k[:, :S].transpose(0, 2, 1, 3))
    vs = np.ascontiguousarray(v[:, :S].transpose(0, 2, 1, 3))
    z = np.zeros((B, Hkv, W, D), np.uint16)
    ring = oracle.ring(z, z, [7, 100], [0, 0])
    ring.append_chunk(np.ascontiguousarray(k[:, S:N]), np.ascontiguousarray(v[:, S:N]))
    torch.cuda.synchronize()
    from tests.gpu_util import bits
    assert np.array_equal(bits(ksd), ks) and np.array_equal(bits(vsd), vs)
    full_o, full_l = oracle.fwd(q, k, v, win_left=W - 1, global_idx=sinks)
    for t in range(N, N + steps):
        log(f"[stream with sinks] decode position {t}")
        binding.kv_append(kc, vc, kd[:, t].contiguous(), vd[:, t].contiguous(), head, length)
        o, l = binding.decode_sinks(qd[:, t].contiguous(), kc, vc, head, length, ksd, vsd)
        torch.cuda.synchronize()
        ring.append(np.ascontiguousarray(k[:, t]), np.ascontiguousarray(v[:, t]))
        ref_o, ref_l = ring.decode(np.ascontiguousarray(q[:, t]), sinks=(ks, vs))
        check(to_host_f64(o), ref_o, dt, f"decode {t} out")
        check(to_host_f64(l), ref_l, dt, f"decode {t} lse")
        check(to_host_f64(o), full_o[:, t], dt, f"decode {t} vs whole-sequence forward")
