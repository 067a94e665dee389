"""Dense-mask brute force for sliding-window attention (test infrastructure only).

This is the O(N^2) formulation the mask-implementation section of the
bmjup.com page "Sliding window attention" describes (section 2 "mask
implementation"): form every score q_i.k_j / sqrt(d), set the scores outside
the window to -infinity, apply softmax, multiply by V.  It is deliberately
written differently from the C oracle: the window is a boolean N x N matrix
built from the offset j - i (a multiple of the dilation whose step count lies
in [-wl, wr]) instead of an enumeration of i + t*d, and globals are whole
rows/columns of that matrix.  It exists to pin the C oracle on tiny inputs.
"""
from __future__ import annotations

import numpy as np


def widen(x: np.ndarray) -> np.ndarray:
    """float32, or bf16 held as uint16 bit patterns, to float64 (exact)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def mask_matrix(N: int, win_left: int, win_right: int, dilation: int = 1,
                global_idx=None) -> np.ndarray:
    """allowed[i, j] is True when query i attends key j."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    off = j - i
    steps = off // dilation
    allowed = (off % dilation == 0) & (steps >= -win_left) & (steps <= win_right)
    causal = win_right == 0
    if global_idx is not None and len(global_idx):
        g = np.unique(np.asarray(global_idx, dtype=np.int64))
        visible = np.ones((N, N), bool) if not causal else (j <= i)
        allowed[:, g] |= visible[:, g]      # every row sees the global keys
        allowed[g, :] = visible[g, :]       # global rows see every key
    return allowed


def fwd(q, k, v, *, win_left: int, win_right: int = 0, dilation: int = 1,
        global_idx=None, scale: float | None = None):
    """q [B,N,Hq,D], k/v [B,N,Hkv,D] -> (out [B,N,Hq,D], lse [B,Hq,N]) in float64."""
    q, k, v = widen(q), widen(k), widen(v)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    allowed = mask_matrix(N, win_left, win_right, dilation, global_idx)
    out = np.zeros((B, N, Hq, D))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            s = scale * (q[b, :, h, :] @ k[b, :, kh, :].T)       # [N, N]
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (e / l) @ v[b, :, kh, :]
            lse[b, h, :] = (m + np.log(l))[:, 0]
    return out, lse


def full_attention(q, k, v, *, causal: bool, scale: float | None = None):
    """Ordinary softmax attention (no window), for the window >= N special case."""
    q, k, v = widen(q), widen(k), widen(v)
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, N, Hq, D))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            s = scale * q[b, :, h, :] @ k[b, :, h // group, :].T
            if causal:
                s = s + np.triu(np.full((N, N), -np.inf), 1)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            out[b, :, h, :] = (e / e.sum(axis=1, keepdims=True)) @ v[b, :, h // group, :]
            lse[b, h, :] = (m + np.log(e.sum(axis=1, keepdims=True)))[:, 0]
    return out, lse
