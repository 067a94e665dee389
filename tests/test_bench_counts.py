"""bench.py on the CPU: its refusal of more than one GPU, and the exact work
counts its TFLOP/s figures divide by, checked against the oracle's
brute-force attended-set matrix (bruteforce.mask_matrix) on small shapes."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import bruteforce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("N,W", [(1, 1), (7, 1), (7, 3), (10, 10), (10, 40), (300, 64)])
def test_exact_pairs_causal(N, W):
    assert bench.exact_pairs_causal(N, W) == int(bruteforce.mask_matrix(N, W - 1, 0).sum())


@pytest.mark.parametrize("N,wl,d", [(50, 5, 1), (50, 5, 2), (97, 7, 4), (64, 40, 8), (9, 3, 16)])
def test_dilated_causal_pairs(N, wl, d):
    assert bench.dilated_causal_pairs(N, wl, d) == int(
        bruteforce.mask_matrix(N, wl, 0, d).sum())


@pytest.mark.parametrize("n,wl,ring", [(20, 7, 8), (5, 7, 8), (30, 15, 16), (1, 0, 4)])
def test_prefill_pairs(n, wl, ring):
    # the chunk's rows of one causal window over the cached tokens and the chunk
    m = bruteforce.mask_matrix(ring + n, wl, 0)
    assert bench.prefill_pairs(n, wl, ring) == int(m[ring:].sum())


@pytest.mark.parametrize("wl,wr,G", [(16, 16, [0, 50, 50, 199]), (3, 40, [7]),
                                     (8, 8, [])])
def test_encoder_pairs(wl, wr, G):
    N = 200
    c = dict(N=N, win_left=wl, win_right=wr, global_idx=G)
    m = bruteforce.mask_matrix(N, wl, wr, 1, G if G else None)
    assert bench.encoder_pairs(c) == int(m.sum())


def test_headline_traffic_profile_matches_the_kernel_sources():
    """The HBM traffic the bench reports comes from the committed counter
    summary of the headline kernel, keyed by a hash of the sources it is
    compiled from; after a change to them the counters must be taken again
    (or the key renewed when the kernel's code is shown unchanged)."""
    import bench
    assert bench.measured_traffic() is not None
