"""swa_decode_noalloc (the decode entry point that allocates nothing: its split
partials live in the library's own per-GPU array) against swa_decode with a
caller workspace.  Both run the same kernels with the same split plan, so the
outputs must agree bit for bit; each is also checked against the oracle's ring.

The calls go through the C ABI directly (ctypes), two in a row with the second
on a smaller input, so the second reads a scratch array that still holds the
first call's partials.  A launch that needs more scratch than the array holds
is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_tiled_amd import binding
from sliding_window_attention_tiled_amd.inputs import DecodeInputs
from tests.gpu_util import check, log, to_dev, to_host_f64

P = ctypes.c_void_p
SCRATCH = 16 << 20     # SWA_NOALLOC_SCRATCH_BYTES


def _ptr(t):
    return P(t.data_ptr()) if t is not None else None


def _noalloc(lib, q, kc, vc, head, length, out, lse, dt):
    B, Hq, D = q.shape
    Hkv, W = kc.shape[1], kc.shape[2]
    return lib.swa_decode_noalloc(_ptr(q), _ptr(kc), _ptr(vc), _ptr(head), _ptr(length),
                                  _ptr(out), _ptr(lse), B, Hq, Hkv, W, D,
                                  ctypes.c_float(1.0 / np.sqrt(D)), dt,
                                  P(torch.cuda.current_stream().cuda_stream))


# larger first, then smaller: (name, B, Hq, Hkv, W, D, dtype, fill)
CASES = [
    [("bf16_split", 4, 16, 2, 2000, 128, "bf16", 1500),
     ("bf16_split_smaller", 2, 8, 8, 300, 64, "bf16", 170)],
    [("f32_split", 3, 8, 2, 700, 128, "f32", None),
     ("f32_split_smaller", 1, 4, 4, 130, 64, "f32", 9)],
    [("bf16_one_range_per_ring", 64, 8, 8, 256, 128, "bf16", None),
     ("bf16_split_after_direct", 1, 4, 1, 640, 64, "bf16", 600)],
]


@pytest.mark.gpu
@pytest.mark.parametrize("pair", CASES, ids=[c[0][0] for c in CASES])
def test_decode_noalloc_matches_decode(pair):
    lib = binding.load_library()
    for name, B, Hq, Hkv, W, D, dt, fill in pair:
        log(f"[noalloc] {name}: B={B} Hq={Hq} Hkv={Hkv} W={W} D={D} {dt} fill={fill}")
        gen = DecodeInputs(23, B, Hq, Hkv, W, D, dt, fill=fill)
        kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
        head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
        length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
        qn, kn, vn = gen.step()
        q = to_dev(qn)
        binding.kv_append(kc, vc, to_dev(kn), to_dev(vn), head, length)
        ref_out, ref_lse = binding.decode(q, kc, vc, head, length)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        code = binding.SWA_BF16 if dt == "bf16" else binding.SWA_F32
        assert _noalloc(lib, q, kc, vc, head, length, out, lse, code) == 0
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if dt == "bf16" else out.view(torch.int32),
                           ref_out.view(torch.int16) if dt == "bf16" else
                           ref_out.view(torch.int32)), name
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), name
        ring = oracle.ring(gen.kcache, gen.vcache, gen.ring_head, gen.cache_len)
        ring.append(kn, vn)
        o, l_ = ring.decode(qn)
        check(to_host_f64(out), o, dt, f"{name} out")
        check(to_host_f64(lse), l_, dt, f"{name} lse")


def test_decode_noalloc_refuses_more_than_its_scratch():
    """Refused before any HIP call (runs without a GPU; the pointers are never
    dereferenced).  float32, 1024 sequences x 32 query heads, D = 128: one
    slot range per ring, 1024 * 32 * (128 + 4) * 4 = 17.3 MB of partials, more
    than the 16 MiB array."""
    lib = binding.load_library()
    fake = P(256)
    assert 1024 * 32 * 132 * 4 > SCRATCH
    st = lib.swa_decode_noalloc(fake, fake, fake, fake, fake, fake, None, 1024, 32, 1, 4096,
                                128, ctypes.c_float(0.1), binding.SWA_F32, None)
    assert st == -3
    # argument errors come first, as in swa_decode
    st = lib.swa_decode_noalloc(None, fake, fake, fake, fake, fake, None, 1024, 32, 1, 4096,
                                128, ctypes.c_float(0.1), binding.SWA_F32, None)
    assert st == -1
    st = lib.swa_decode_noalloc(fake, fake, fake, fake, fake, fake, None, 1024, 32, 1, 4096,
                                128, ctypes.c_float(0.0), binding.SWA_F32, None)
    assert st == -1
