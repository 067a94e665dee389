"""The workloads the library is measured and checked on.

Window conventions (explicit left/right extents in dilated steps):
  * causal window of W keys  -> win_left = W - 1, win_right = 0
  * symmetric 256 + 256      -> win_left = win_right = 256
  * dilated causal, 512 keys -> win_left = 511, win_right = 0, dilation d
"""
from __future__ import annotations

FWD = {
    "tiny_causal": dict(B=1, Hq=2, Hkv=2, N=256, D=64, dtype="f32",
                        win_left=63, win_right=0, dilation=1, global_idx=None, seed=1),
    "mistral_causal_w4096": dict(B=1, Hq=32, Hkv=8, N=16384, D=128, dtype="bf16",
                                 win_left=4095, win_right=0, dilation=1, global_idx=None,
                                 seed=2),
    "bidir_encoder_globals": dict(B=4, Hq=12, Hkv=12, N=8192, D=64, dtype="bf16",
                                  win_left=256, win_right=256, dilation=1,
                                  global_idx=list(range(0, 8192, 512)), seed=3),
}

# four layers of one dilated stack: same q/k/v, dilation 1, 2, 4, 8
DILATED_STACK = dict(B=2, Hq=16, Hkv=16, N=32768, D=128, dtype="bf16",
                     win_left=511, win_right=0, dilations=(1, 2, 4, 8), global_idx=None,
                     seed=4)

DECODE = dict(B=64, Hq=32, Hkv=8, W=4096, D=128, dtype="bf16", steps=256, seed=5)

# chunked prefill: one 4096-token chunk of a Mistral-shaped prompt attending to
# a full 4096-slot ring (the tokens before it) and to itself, window 4096
PREFILL_CHUNK = dict(B=1, Hq=32, Hkv=8, W=4096, D=128, dtype="bf16", chunk=4096,
                     win_left=4095, seed=6)
