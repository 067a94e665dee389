"""Seeded synthetic inputs, shared by the tests, the smoke check and the bench.

This module only draws random numbers; it holds none of the attention
arithmetic, so both the GPU library and the CPU oracle can be fed from it
without sharing any of the method's code.

Recipe: numpy ``Generator(PCG64(seed))``, ``standard_normal(dtype=float32)``,
drawn in a fixed order (forward: q, k, v; decode: kcache, vcache, ring_head,
then per step q_t, k_t, v_t).  bfloat16 tensors are the float32 draws rounded
to nearest-even, returned as raw uint16 bit patterns so that both sides read
the identical bits.
"""
from __future__ import annotations

import numpy as np


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN inputs keep a quiet NaN pattern; this generator never produces them.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def fwd_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, D: int, dtype: str):
    """(q [B,N,Hq,D], k [B,N,Hkv,D], v [B,N,Hkv,D]) ~ N(0,1); float32 or bf16 bits."""
    g = _rng(seed)
    q = g.standard_normal((B, N, Hq, D), dtype=np.float32)
    k = g.standard_normal((B, N, Hkv, D), dtype=np.float32)
    v = g.standard_normal((B, N, Hkv, D), dtype=np.float32)
    return _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)


class DecodeInputs:
    """Initial ring state plus a stream of per-step (q_t, k_t, v_t).

    kcache/vcache [B,Hkv,W,D] ~ N(0,1); ring_head[b] ~ U[0, W) (random head
    offsets); cache_len[b] = fill (W for a full ring).  Steps are drawn in order
    from the same generator, so step t is reproducible only by drawing steps
    0..t-1 first.
    """

    def __init__(self, seed: int, B: int, Hq: int, Hkv: int, W: int, D: int,
                 dtype: str, fill: int | None = None):
        self.B, self.Hq, self.Hkv, self.W, self.D, self.dtype = B, Hq, Hkv, W, D, dtype
        self._g = _rng(seed)
        self.kcache = _cast(self._g.standard_normal((B, Hkv, W, D), dtype=np.float32), dtype)
        self.vcache = _cast(self._g.standard_normal((B, Hkv, W, D), dtype=np.float32), dtype)
        self.ring_head = self._g.integers(0, W, size=B).astype(np.int32)
        self.cache_len = np.full(B, W if fill is None else fill, np.int32)

    def step(self):
        g = self._g
        q = g.standard_normal((self.B, self.Hq, self.D), dtype=np.float32)
        k = g.standard_normal((self.B, self.Hkv, self.D), dtype=np.float32)
        v = g.standard_normal((self.B, self.Hkv, self.D), dtype=np.float32)
        return _cast(q, self.dtype), _cast(k, self.dtype), _cast(v, self.dtype)
