"""Helpers for the GPU parity tests: moving seeded inputs to the device and the
tolerance checks (float32: max-abs 1e-4; bfloat16: max-abs 2e-2 and relative
RMS 5e-3, for both out and lse)."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {
    "f32": dict(max_abs=1e-4, rel_rms=None),
    "bf16": dict(max_abs=2e-2, rel_rms=5e-3),
}


def log(msg: str):
    """Name the case on stdout before a GPU step, flushed."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    """float32 array or bf16 bit patterns (uint16) -> device tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(x).to("cuda")


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    tol = TOL[dtype]
    mx = float(err.max()) if err.size else 0.0
    msg = f"{what}: max-abs {mx:.3e}"
    if tol["rel_rms"] is not None:
        rr = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
        msg += f", rel-rms {rr:.3e}"
        assert rr <= tol["rel_rms"], msg
    assert mx <= tol["max_abs"], msg
    log("  " + msg)
    return msg
