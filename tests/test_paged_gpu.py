"""GPU parity of the paged window cache: swa_kv_append_paged and
swa_decode_paged against the oracle's paged cache.

Sequences share a page pool smaller than their blocks; pages of blocks that
left the window return to a free list and are reused, also by other
sequences (the bookkeeping a serving loop does on the host).  After every
append the whole pool must be bit-identical to the oracle's and every decode
within tolerance.  The full-size case runs the rolling-cache decode shape
through a paged pool with randomly placed pages.
"""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding, configs
from sliding_window_attention_tiled_amd.inputs import DecodeInputs, fwd_inputs
from tests.gpu_util import bits, check, log, to_dev, to_host_f64
from tests.oracle_pins import _PagePool

pytestmark = pytest.mark.gpu


def _pool_equal(kp, vp, cache, dt, what):
    torch.cuda.synchronize()
    if dt == "bf16":
        assert np.array_equal(bits(kp), cache.k) and np.array_equal(bits(vp), cache.v), what
    else:
        assert np.array_equal(kp.cpu().numpy(), cache.k) and \
            np.array_equal(vp.cpu().numpy(), cache.v), what


CASES = [
    # name, B, Hq, Hkv, D, W, P, n_pages, dtype, per-sequence append plans
    ("bf16_gqa4_p16", 3, 8, 2, 128, 100, 16, 24, "bf16",
     {0: [150, 1, 1, 1, 1], 1: [1] * 5 + [40, 1], 2: [33, 1, 70, 1, 1, 20]}),
    ("f32_mha_p32", 2, 2, 2, 64, 64, 32, 8, "f32", {0: [1] * 6, 1: [90, 1, 1, 1]}),
    ("bf16_gqa16_p64", 2, 16, 1, 64, 200, 64, 10, "bf16", {0: [300, 1, 1], 1: [10, 1, 1]}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_stream(case):
    name, B, Hq, Hkv, D, W, P, n_pages, dt, plan = case
    nb = -(-(W + P - 1) // P)
    N = max(sum(v) for v in plan.values())
    q, k, v = fwd_inputs(71, B, Hq, Hkv, N, D, dt)
    rng = np.random.Generator(np.random.PCG64(72))
    pool = _PagePool(n_pages, B, nb, P, W, rng.permutation(n_pages))
    shape = (n_pages, Hkv, P, D)
    z = np.zeros(shape, np.uint16 if dt == "bf16" else np.float32)
    cache = oracle.paged(z, z, [0] * B, W)
    kp, vp = to_dev(z), to_dev(z)
    seq = torch.zeros(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(binding.decode_workspace_size(B, Hq, W, D), dtype=torch.uint8,
                     device="cuda")
    scale = 0.1 if dt == "f32" else None
    pos = [0] * B
    for step in range(max(len(p_) for p_ in plan.values())):
        # one batched append: sequences with nothing to append this step get n = 0
        # through a per-step batch of the sequences that do append
        active = [b for b in range(B) if step < len(plan[b])]
        for b in active:
            n = plan[b][step]
            pool.reserve(b, pos[b], n)
            table = torch.from_numpy(pool.table[b:b + 1].copy()).to("cuda")
            kb = np.ascontiguousarray(k[b:b + 1, pos[b]:pos[b] + n])
            vb = np.ascontiguousarray(v[b:b + 1, pos[b]:pos[b] + n])
            log(f"[paged] {name} step {step} seq {b} append {n}")
            seq_b = seq[b:b + 1].clone()
            binding.kv_append_paged(kp, vp, to_dev(kb), to_dev(vb), table, seq_b, window=W)
            seq[b] = seq_b[0]
            sub = oracle.paged(cache.k, cache.v, [cache.len[b]], W)
            sub.append(kb, vb, pool.table[b:b + 1])
            cache.k, cache.v = sub.k, sub.v
            cache.len[b] += n
            pos[b] += n
        _pool_equal(kp, vp, cache, dt, f"{name} pool after step {step}")
        assert seq.cpu().numpy().tolist() == cache.len.tolist()
        # decode every sequence that has tokens, batched over B with the full table
        if min(pos) == 0:
            continue
        qt = np.ascontiguousarray(np.stack([q[b, pos[b] - 1] for b in range(B)]))
        table = torch.from_numpy(pool.table.copy()).to("cuda")
        out, lse = binding.decode_paged(to_dev(qt), kp, vp, table, seq, window=W, scale=scale,
                                        workspace=ws)
        torch.cuda.synchronize()
        ref_o, ref_l = cache.decode(qt, pool.table, scale=scale)
        check(to_host_f64(out), ref_o, dt, f"{name} step {step} out")
        check(to_host_f64(lse), ref_l, dt, f"{name} step {step} lse")
        if step == 2 and B > 2:
            # sequence 2 finishes and returns all its pages; a new sequence takes
            # its batch slot and draws pages from the shared free list
            pool.release(2)
            pos[2] = 0
            seq[2] = 0
            cache.len[2] = 0


def test_paged_full_size():
    """The rolling-cache decode shape (64 sequences, Hq=32, Hkv=8, D=128,
    window 4096) through pages of 64 positions placed at random in the pool,
    sequences at different lengths past the window: append + decode steps."""
    c = configs.DECODE
    B, Hq, Hkv, W, D, dt = c["B"], c["Hq"], c["Hkv"], c["W"], c["D"], c["dtype"]
    P = 64
    nb = (W + P - 1 + P - 1) // P
    n_pages = B * nb
    g = np.random.Generator(np.random.PCG64(81))
    gen = DecodeInputs(82, n_pages, Hq, Hkv, P, D, dt)      # pool contents ~ N(0,1)
    kpool, vpool = gen.kcache, gen.vcache                    # [n_pages, Hkv, P, D]
    table = g.permutation(n_pages).astype(np.int32).reshape(B, nb)
    seq_len = g.integers(W, 3 * W, size=B).astype(np.int32)
    cache = oracle.paged(kpool, vpool, seq_len, W)
    kp, vp = to_dev(kpool), to_dev(vpool)
    tdev = torch.from_numpy(table).to("cuda")
    seq = torch.from_numpy(seq_len.copy()).to("cuda")
    ws = torch.empty(binding.decode_workspace_size(B, Hq, W, D), dtype=torch.uint8,
                     device="cuda")
    for t in range(3):
        qn, kn, vn = DecodeInputs(83 + t, B, Hq, Hkv, 1, D, dt).step()
        log(f"[paged] full size step {t}")
        binding.kv_append_paged(kp, vp, to_dev(kn[:, None]), to_dev(vn[:, None]), tdev, seq,
                                window=W)
        out, lse = binding.decode_paged(to_dev(qn), kp, vp, tdev, seq, window=W, workspace=ws)
        torch.cuda.synchronize()
        cache.append(kn[:, None], vn[:, None], table)
        ref_o, ref_l = cache.decode(qn, table)
        check(to_host_f64(out), ref_o, dt, f"full size step {t} out")
        check(to_host_f64(lse), ref_l, dt, f"full size step {t} lse")
    _pool_equal(kp, vp, cache, dt, "full size pool")
