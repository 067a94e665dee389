"""Benchmark: sliding-window attention on one MI355X.

One step = one swa_fwd call on the Mistral-shaped causal layer (B=1, Hq=32,
Hkv=8, N=16384, D=128, bf16, window W=4096 keys [i-4095, i]) with inputs
already resident in HBM.  The headline value is in-window TFLOP/s by the
nominal count 4*B*Hq*N*W*D per call; the exact count (sum over rows of the
attended keys times 4*D) is reported beside it and is what the roofline
fraction uses.  The same JSON line carries the decode leg (64 sequences,
Hq=32, Hkv=8, D=128, W=4096 ring, append + attend per step) as HBM GB/s of
K+V streamed, and the fp64 CPU oracle timed on bounded samples of both
(forward rows as TFLOP/s, decode steps as GB/s), with the host's CPU count
and model.

Also reported: socket power and shader clock while the forward runs in a
loop for 3 s (amd-smi), with the MFMA peak at that clock.  Per call: the
bidirectional encoder with global tokens, the
four layers of the dilated stack and one 4096-token chunk of a chunked prefill
(exact TFLOP/s against min(MFMA peak, HBM peak x arithmetic intensity)), and
the decode shape with four attention sinks and through a paged pool (GB/s),
and the backward of the headline layer (TFLOP/s at 10*D flop per pair).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-decode]
                    [--no-others]
    python bench.py --power     # board power and shader clock under load (amd-smi)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


# the sources the headline kernel (swa_fwd_pp_kernel) is compiled from
FWD_SOURCES = ["sliding_window_attention_tiled_amd/csrc/fwd_pp.hip",
               "sliding_window_attention_tiled_amd/csrc/tile_common.h",
               "sliding_window_attention_tiled_amd/csrc/fwd_common.h",
               "sliding_window_attention_tiled_amd/csrc/device_common.h",
               "sliding_window_attention_tiled_amd/csrc/swa_kernels.h"]
FWD_PROFILE = "profiles/swa_fwd_pp_mistral_causal_w4096.md"


def measured_traffic():
    """HBM bytes per forward launch from the committed counter summary, or None
    when the kernel sources changed after the counters were taken."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, FWD_PROFILE)).read()
        h = hashlib.sha256()
        for f in FWD_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic-bytes-per-launch: ", "source-sha256: ")))
    if fields.get("source-sha256", "").strip() != h.hexdigest():
        return None
    return float(fields["traffic-bytes-per-launch"])


def exact_pairs_causal(N: int, W: int) -> int:
    """Sum over i of |[max(0, i-W+1), i]|."""
    full = max(0, N - (W - 1))
    ramp = min(N, W - 1)
    return full * W + ramp * (ramp + 1) // 2


def dilated_causal_pairs(N: int, wl: int, d: int) -> int:
    """Attended pairs of a causal dilated window: query i sees i, i - d, ...,
    down to max(i - wl*d, i mod d)."""
    return int((np.minimum(wl, np.arange(N) // d) + 1).sum())


def prefill_pairs(n: int, wl: int, ring_len: int) -> int:
    """Attended pairs of an n-token chunk after ring_len cached tokens, causal
    window wl + 1: chunk token t sees min(ring_len, max(wl - t, 0)) ring entries
    and chunk tokens max(0, t - wl) .. t."""
    t = np.arange(n)
    return int((np.minimum(ring_len, np.maximum(wl - t, 0)) + np.minimum(t, wl) + 1).sum())


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode leg")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the per-call timings of the other workloads")
    ap.add_argument("--cpu-rows", type=int, default=393216)
    ap.add_argument("--cpu-decode-steps", type=int, default=256)
    ap.add_argument("--only", choices=["fwd", "decode", "others"], default=None,
                    help="run one leg only (for profiling)")
    ap.add_argument("--power", action="store_true",
                    help="run only the board-power leg: each workload in a loop for a few "
                         "seconds while amd-smi samples socket power and shader clocks")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy, the reference "
                         "kernel for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def copy_calibration(reps: int = 3):
    """A plain copy of 2^30 bytes, repeated: the counter reading of one dispatch
    divided by 2^20 KiB read (and written) gives the scale factor of the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "reps": reps}))


def to_dev(x):
    import torch
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")


def bench_fwd(args):
    import torch
    from sliding_window_attention_tiled_amd import binding, configs
    from sliding_window_attention_tiled_amd.inputs import fwd_inputs

    c = configs.FWD["mistral_causal_w4096"]
    B, Hq, Hkv, N, D = c["B"], c["Hq"], c["Hkv"], c["N"], c["D"]
    W = c["win_left"] + 1
    qh, kh, vh = fwd_inputs(c["seed"], B, Hq, Hkv, N, D, c["dtype"])
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    kw = dict(win_left=c["win_left"], win_right=c["win_right"], dilation=c["dilation"],
              out=out, lse=lse)
    stream = torch.cuda.current_stream()
    # settle the clocks (about 0.3 s of the same work), then the counted warm-up
    t_settle = time.perf_counter() + 0.3
    while time.perf_counter() < t_settle:
        binding.fwd(q, k, v, **kw)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        binding.fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        starts[s].record(stream)
        binding.fwd(q, k, v, **kw)
        ends[s].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]  # ms, one launch each
    ms_event = float(np.mean(per))
    ms_step = wall * 1e3 / args.steps
    nominal = 4.0 * B * Hq * N * W * D
    exact = 4.0 * B * Hq * exact_pairs_causal(N, W) * D
    return dict(ms_step=ms_step, ms_kernel=ms_event, ms_kernel_min=float(np.min(per)),
                nominal_flop=nominal, exact_flop=exact, inputs=(qh, kh, vh), cfg=c)


def bench_decode(args):
    import torch
    from sliding_window_attention_tiled_amd import binding, configs
    from sliding_window_attention_tiled_amd.inputs import DecodeInputs

    c = configs.DECODE
    gen = DecodeInputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["W"], c["D"], c["dtype"])
    kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
    head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
    length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
    steps = c["steps"]
    qs, ks, vs = [], [], []
    for _ in range(steps):
        a, b_, c_ = gen.step()
        qs.append(a), ks.append(b_), vs.append(c_)
    qd = to_dev(np.stack(qs))
    kd = to_dev(np.stack(ks))
    vd = to_dev(np.stack(vs))
    ws = torch.empty(binding.decode_workspace_size(c["B"], c["Hq"], c["W"], c["D"]),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qd[0])
    lse = torch.empty((c["B"], c["Hq"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(t):
        binding.kv_append(kc, vc, kd[t], vd[t], head, length)
        binding.decode(qd[t], kc, vc, head, length, workspace=ws, out=out, lse=lse)

    for t in range(min(3, steps)):  # warm-up on a copy-free prefix; ring state moves on
        step(t)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for t in range(steps):
        e0, e1, e2 = ev[t]
        e0.record(stream)
        binding.kv_append(kc, vc, kd[t], vd[t], head, length)
        e1.record(stream)
        binding.decode(qd[t], kc, vc, head, length, workspace=ws, out=out, lse=lse)
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = float(np.mean([a.elapsed_time(b) for _, a, b in ev]))
    step_ms = float(np.mean([a.elapsed_time(b) for a, _, b in ev]))
    kv_bytes = 2.0 * c["B"] * c["Hkv"] * c["W"] * c["D"] * 2
    host = dict(kcache=gen.kcache, vcache=gen.vcache, ring_head=gen.ring_head,
                cache_len=gen.cache_len, q=qs, k=ks, v=vs)
    return dict(workload="rolling_cache_decode", B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], W=c["W"],
                D=c["D"], steps=steps, ms_per_step_wall=wall * 1e3 / steps,
                ms_append_plus_decode=step_ms, ms_decode=dec_ms,
                kv_bytes_per_step=kv_bytes,
                decode_gbs=kv_bytes / (dec_ms * 1e-3) / 1e9,
                decode_frac_hbm=kv_bytes / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                step_gbs=kv_bytes / (step_ms * 1e-3) / 1e9), host


def _time_calls(fn, reps=10, warmup=3):
    """Mean and min device time (ms) of fn() over reps launches, HIP events on
    the current stream, after a short clock-settling warm-up."""
    import torch
    stream = torch.cuda.current_stream()
    t_settle = time.perf_counter() + 0.1
    while time.perf_counter() < t_settle:
        fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return float(np.mean(per)), float(np.min(per))


def _bound(flop, bytes_):
    """Roofline bound of a launch: min(MFMA peak, HBM peak x arithmetic intensity)."""
    return min(PEAK_BF16_TFLOPS, PEAK_HBM_GBS * 1e9 * flop / bytes_ / 1e12)


def _report(name, ms, ms_min, flop, bytes_, extra=None):
    tf = flop / (ms * 1e-3) / 1e12
    bound = _bound(flop, bytes_)
    r = {"workload": name, "kernel_ms": round(ms, 4), "kernel_ms_min": round(ms_min, 4),
         "tflops_exact": round(tf, 2), "bound_tflops": round(bound, 1),
         "frac_of_bound": round(tf / bound, 4), "algorithmic_bytes": int(bytes_)}
    if extra:
        r.update(extra)
    return r


def encoder_pairs(c) -> int:
    """Exact attended pairs per (b, h) of the bidirectional encoder with global
    tokens: the band, the global keys outside it, and whole rows for the
    global queries."""
    N = c["N"]
    G = np.array(sorted(set(c["global_idx"])))
    i = np.arange(N)
    band = np.minimum(i, c["win_left"]) + np.minimum(N - 1 - i, c["win_right"]) + 1
    far = ((G[None, :] < i[:, None] - c["win_left"]) |
           (G[None, :] > i[:, None] + c["win_right"])).sum(1)
    return int(np.where(np.isin(i, G), N, band + far).sum())


def bench_other_workloads():
    """The bidirectional encoder with global tokens, the four layers of the
    dilated stack and one chunk of a chunked prefill, each timed per call and
    reported as exact TFLOP/s against min(MFMA, HBM x intensity)."""
    import torch
    from sliding_window_attention_tiled_amd import binding, configs
    from sliding_window_attention_tiled_amd.inputs import DecodeInputs, fwd_inputs

    res = []
    # bidirectional encoder, window 256 + 256, 16 global tokens
    c = configs.FWD["bidir_encoder_globals"]
    B, H, N, D = c["B"], c["Hq"], c["N"], c["D"]
    q, k, v = (to_dev(x) for x in fwd_inputs(c["seed"], B, H, H, N, D, c["dtype"]))
    G = np.array(sorted(set(c["global_idx"])))
    pairs = encoder_pairs(c)
    flop = 4.0 * B * H * D * float(pairs)
    bytes_ = 4.0 * B * N * H * D * 2 + 4.0 * B * H * N
    ws = torch.empty(binding.fwd_workspace_size(B, H, N, D, len(G)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ms, mn = _time_calls(lambda: binding.fwd(q, k, v, win_left=c["win_left"],
                                             win_right=c["win_right"], global_idx=c["global_idx"],
                                             out=out, lse=lse, workspace=ws))
    res.append(_report("bidir_encoder_globals", ms, mn, flop, bytes_))
    del q, k, v, out, lse, ws

    # dilated stack: one call per dilation on the same q/k/v
    c = configs.DILATED_STACK
    B, H, N, D = c["B"], c["Hq"], c["N"], c["D"]
    q, k, v = (to_dev(x) for x in fwd_inputs(c["seed"], B, H, H, N, D, c["dtype"]))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    bytes_ = 4.0 * B * N * H * D * 2 + 4.0 * B * H * N
    for d in c["dilations"]:
        flop = 4.0 * B * H * D * float(dilated_causal_pairs(N, c["win_left"], d))
        ms, mn = _time_calls(lambda: binding.fwd(q, k, v, win_left=c["win_left"], win_right=0,
                                                 dilation=d, out=out, lse=lse))
        res.append(_report(f"dilated_stack_d{d}", ms, mn, flop, bytes_))
    del q, k, v, out, lse

    # chunked prefill: a 4096-token chunk after a full 4096-slot ring
    c = configs.PREFILL_CHUNK
    B, Hq, Hkv, W, D, n = c["B"], c["Hq"], c["Hkv"], c["W"], c["D"], c["chunk"]
    gen = DecodeInputs(c["seed"], B, Hq, Hkv, W, D, c["dtype"])
    q, k, v = (to_dev(x) for x in fwd_inputs(c["seed"] + 100, B, Hq, Hkv, n, D, c["dtype"]))
    kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
    head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
    length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
    wl = c["win_left"]
    flop = 4.0 * B * Hq * D * float(prefill_pairs(n, wl, W))
    bytes_ = (2.0 * B * n * Hq * D * 2 + 2.0 * B * n * Hkv * D * 2 + 2.0 * B * Hkv * W * D * 2
              + 4.0 * B * Hq * n)
    ms, mn = _time_calls(lambda: binding.fwd_cached(q, k, v, kc, vc, head, length,
                                                    win_left=wl, out=out, lse=lse))
    # the hand-off copy of the chunk into a scratch ring (state restored each time)
    kc2, vc2 = kc.clone(), vc.clone()
    h2, l2 = head.clone(), length.clone()
    ams, amn = _time_calls(lambda: binding.kv_append_chunk(kc2, vc2, k, v, h2, l2))
    append_bytes = 2.0 * 2 * B * min(n, W) * Hkv * D * 2   # read chunk + write ring, K and V
    res.append(_report("prefill_chunk4096_after_full_ring", ms, mn, flop, bytes_,
                       {"append_chunk_ms": round(ams, 4),
                        "append_chunk_gbs": round(append_bytes / (ams * 1e-3) / 1e9, 1)}))
    del q, k, v, kc, vc, kc2, vc2, out, lse
    res.extend(bench_decode_variants())
    res.append(bench_bwd())
    res.append(bench_bwd_globals())
    return res


def bench_bwd_globals():
    """Backward of the bidirectional encoder with 16 global tokens: the band
    passes plus the passes over the global tokens' pairs outside the band."""
    import torch
    from sliding_window_attention_tiled_amd import binding, configs
    from sliding_window_attention_tiled_amd.inputs import fwd_inputs

    c = configs.FWD["bidir_encoder_globals"]
    B, H, N, D = c["B"], c["Hq"], c["N"], c["D"]
    G = c["global_idx"]
    q, k, v = (to_dev(x) for x in fwd_inputs(c["seed"], B, H, H, N, D, c["dtype"]))
    g = to_dev(fwd_inputs(c["seed"] + 100, B, H, H, N, D, c["dtype"])[0])
    kw = dict(win_left=c["win_left"], win_right=c["win_right"], global_idx=G)
    out, lse = binding.fwd(q, k, v, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(binding.bwd_workspace_size(B, H, H, N, D, len(G)), dtype=torch.uint8,
                     device="cuda")
    ms, mn = _time_calls(lambda: binding.bwd(q, k, v, out, lse, g, dq=dq, dk=dk, dv=dv,
                                             workspace=ws, **kw))
    flop = 10.0 * B * H * D * float(encoder_pairs(c))
    bytes_ = (4.0 * B * N * H * D + 4.0 * B * N * H * D) * 2 + 8.0 * B * H * N
    return _report("bwd_bidir_encoder_globals", ms, mn, flop, bytes_,
                   {"flop_per_pair": "10*D algorithmic"})


def bench_bwd():
    """Backward of the Mistral-shaped causal layer (config of the headline):
    one swa_bwd call (delta, dq pass, dk/dv pass).  Algorithmic work 10*D flop
    per attended pair (recomputed q.k, dP, dv, dk, dq: 2*D each); the kernels
    execute 14*D (the query-major and key-major passes each form q.k and dP)."""
    import torch
    from sliding_window_attention_tiled_amd import binding, configs
    from sliding_window_attention_tiled_amd.inputs import fwd_inputs

    c = configs.FWD["mistral_causal_w4096"]
    B, Hq, Hkv, N, D = c["B"], c["Hq"], c["Hkv"], c["N"], c["D"]
    W = c["win_left"] + 1
    q, k, v = (to_dev(x) for x in fwd_inputs(c["seed"], B, Hq, Hkv, N, D, c["dtype"]))
    g = to_dev(fwd_inputs(c["seed"] + 100, B, Hq, Hkv, N, D, c["dtype"])[0])
    out, lse = binding.fwd(q, k, v, win_left=c["win_left"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(binding.bwd_workspace_size(B, Hq, Hkv, N, D), dtype=torch.uint8, device="cuda")
    ms, mn = _time_calls(lambda: binding.bwd(q, k, v, out, lse, g, win_left=c["win_left"],
                                             dq=dq, dk=dk, dv=dv, workspace=ws))
    pairs = exact_pairs_causal(N, W)
    flop = 10.0 * B * Hq * D * pairs
    bytes_ = (4.0 * B * N * Hq * D + 4.0 * B * N * Hkv * D) * 2 + 8.0 * B * Hq * N
    return _report("bwd_mistral_causal_w4096", ms, mn, flop, bytes_,
                   {"flop_per_pair": "10*D algorithmic (14*D executed)"})


def _decode_report(name, ms, ms_min, kv_bytes, extra=None):
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    r = {"workload": name, "kernel_ms": round(ms, 4), "kernel_ms_min": round(ms_min, 4),
         "kv_bytes": int(kv_bytes), "gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    if extra:
        r.update(extra)
    return r


def bench_decode_variants():
    """The rolling-cache decode shape (64 sequences, Hq=32, Hkv=8, D=128, window
    4096) with four attention-sink entries, and through a paged pool of
    64-position pages placed at random: one decode call timed per step, K+V
    bytes of the attended entries per call."""
    import torch
    from sliding_window_attention_tiled_amd import binding, configs
    from sliding_window_attention_tiled_amd.inputs import DecodeInputs

    c = configs.DECODE
    B, Hq, Hkv, W, D = c["B"], c["Hq"], c["Hkv"], c["W"], c["D"]
    res = []
    gen = DecodeInputs(c["seed"], B, Hq, Hkv, W, D, c["dtype"])
    kc, vc = to_dev(gen.kcache), to_dev(gen.vcache)
    head = torch.from_numpy(gen.ring_head.copy()).to("cuda")
    length = torch.from_numpy(gen.cache_len.copy()).to("cuda")
    qd = to_dev(gen.step()[0])
    S = 4
    sk = DecodeInputs(c["seed"] + 10, B, Hq, Hkv, S, D, c["dtype"])
    ks, vs = to_dev(sk.kcache), to_dev(sk.vcache)
    ws = torch.empty(binding.decode_sinks_workspace_size(B, Hq, W, D, S), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(qd)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ms, mn = _time_calls(lambda: binding.decode_sinks(qd, kc, vc, head, length, ks, vs,
                                                      workspace=ws, out=out, lse=lse))
    res.append(_decode_report("decode_ring4096_sinks4", ms, mn,
                              2.0 * B * Hkv * (W + S) * D * 2))
    del kc, vc
    P = 64
    nb = (W + P - 1 + P - 1) // P
    n_pages = B * nb
    pg = DecodeInputs(c["seed"] + 20, n_pages, Hq, Hkv, P, D, c["dtype"])
    kp, vp = to_dev(pg.kcache), to_dev(pg.vcache)
    g = np.random.Generator(np.random.PCG64(c["seed"] + 21))
    table = torch.from_numpy(g.permutation(n_pages).astype(np.int32).reshape(B, nb)).to("cuda")
    seq = torch.from_numpy(g.integers(W, 3 * W, size=B).astype(np.int32)).to("cuda")
    ms, mn = _time_calls(lambda: binding.decode_paged(qd, kp, vp, table, seq, window=W,
                                                      workspace=ws, out=out, lse=lse))
    res.append(_decode_report("decode_paged_p64_window4096", ms, mn,
                              2.0 * B * Hkv * W * D * 2, {"page_size": P}))
    return res


def cpu_baseline(inputs, cfg, n_rows):
    """The oracle (built here with -O3 -march=native, OpenMP over rows) on a
    seeded uniform sample of the forward's rows, as exact TFLOP/s."""
    import oracle

    orc = oracle.native()
    qh, kh, vh = inputs
    N, Hq, B = cfg["N"], cfg["Hq"], cfg["B"]
    rng = np.random.Generator(np.random.PCG64(99))
    rows = np.stack([rng.integers(0, B, n_rows), rng.integers(0, Hq, n_rows),
                     rng.integers(0, N, n_rows)], axis=1).astype(np.int64)
    W = cfg["win_left"] + 1
    pairs = np.minimum(rows[:, 2] + 1, W).sum()
    t0 = time.perf_counter()
    orc.fwd_rows(qh, kh, vh, rows, win_left=cfg["win_left"], win_right=cfg["win_right"])
    dt = time.perf_counter() - t0
    flop = 4.0 * cfg["D"] * float(pairs)
    r = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(),
         "kind": "oracle",
         "sample": f"{n_rows} seeded uniform (b, h, i) rows of the same workload, "
                   f"exact in-window flop / wall time ({dt:.1f} s)",
         "build": "gcc -O3 -march=native -fopenmp, fp64"}
    r.update(oracle.host_info())
    return r


def cpu_baseline_decode(host, n_steps):
    """The oracle's ring (append, then attend over the valid slots) on the first
    n_steps steps of the decode workload's stream, as K+V GB/s: the K+V bytes
    a step attends over (the whole 4096-slot ring of every sequence and kv
    head) divided by the wall time per step."""
    import oracle

    orc = oracle.native()
    ring = orc.ring(host["kcache"], host["vcache"], host["ring_head"], host["cache_len"])
    B, Hkv, W, D = host["kcache"].shape
    n = min(n_steps, len(host["q"]))
    t0 = time.perf_counter()
    for t in range(n):
        ring.append(host["k"][t], host["v"][t])
        ring.decode(host["q"][t])
    dt = time.perf_counter() - t0
    kv_bytes = 2.0 * B * Hkv * W * D * 2
    r = {"value": kv_bytes * n / dt / 1e9, "unit": "GB/s", "cores": orc.num_threads(),
         "kind": "oracle",
         "sample": f"steps 0..{n - 1} of the 256-step rolling-cache stream (append + decode "
                   f"each), {kv_bytes:.4g} B of K+V per step / wall time ({dt:.1f} s)",
         "build": "gcc -O3 -march=native -fopenmp, fp64"}
    r.update(oracle.host_info())
    return r


def _smi_sample():
    """Socket power (W) and the shader clock of each XCD (MHz) from amd-smi, or
    None where the tool is missing or its output has another shape."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"],
                           capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        g = (d["gpu_data"] if isinstance(d, dict) else d)[0]
        watts = float(g["power"]["socket_power"]["value"])
        clks = [float(v["clk"]["value"]) for k, v in g["clock"].items()
                if k.startswith("gfx_") and isinstance(v, dict)]
        return watts, clks
    except Exception:
        return None


def _power_cap():
    """The board's power cap in W (rocm-smi --showmaxpower), or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showmaxpower"], capture_output=True, text=True,
                           timeout=20)
        m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", r.stdout)
        return float(m.group(1)) if m else None
    except Exception:
        return None


def _power_of(name, fn, seconds=5.0, settle=1.0):
    """Run fn in a loop for `seconds` while a thread samples amd-smi; samples of
    the first `settle` seconds (clock ramp) are dropped."""
    import threading
    import time
    import torch
    fn()
    torch.cuda.synchronize()
    samples, stop = [], []
    t0 = time.time()

    def sampler():
        while not stop:
            s = _smi_sample()
            if s is not None and time.time() - t0 >= settle:
                samples.append(s)
            time.sleep(0.25)

    th = threading.Thread(target=sampler)
    th.start()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    n = 0
    while time.time() - t0 < seconds:
        for _ in range(20):
            fn()
        n += 20
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    stop.append(1)
    th.join()
    rec = {"workload": name, "calls": n, "ms_per_call": round(e0.elapsed_time(e1) / n, 4),
           "samples": len(samples)}
    if samples:
        w = [s[0] for s in samples]
        c = [sum(s[1]) / len(s[1]) for s in samples if s[1]]
        rec["socket_power_w"] = round(sum(w) / len(w), 1)
        rec["socket_power_w_max"] = max(w)
        if c:
            rec["gfx_clock_mhz"] = round(sum(c) / len(c), 1)
            rec["gfx_clock_mhz_min"] = round(min(min(s[1]) for s in samples if s[1]), 1)
    return rec


def bench_power():
    """Board power and shader clock under each heavy workload: the headline
    forward, its backward and the bidirectional encoder forward with global
    tokens; and the idle board for reference."""
    import time
    import torch
    from sliding_window_attention_tiled_amd import binding, configs
    from sliding_window_attention_tiled_amd.inputs import fwd_inputs

    out = [{"power_cap_w": _power_cap()}]
    idle = _smi_sample()
    if idle is not None:
        out.append({"workload": "idle", "socket_power_w": idle[0],
                    "gfx_clock_mhz": round(sum(idle[1]) / max(1, len(idle[1])), 1)})
    for name in ("mistral_causal_w4096", "bidir_encoder_globals"):
        c = configs.FWD[name]
        q, k, v = (to_dev(x) for x in fwd_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"],
                                                 c["D"], c["dtype"]))
        kw = dict(win_left=c["win_left"], win_right=c["win_right"], dilation=c["dilation"],
                  global_idx=c.get("global_idx"))
        o = torch.empty_like(q)
        lse = torch.empty((c["B"], c["Hq"], c["N"]), dtype=torch.float32, device="cuda")
        out.append(_power_of(name, lambda: binding.fwd(q, k, v, out=o, lse=lse, **kw)))
        if name == "mistral_causal_w4096":
            g = to_dev(fwd_inputs(c["seed"] + 100, c["B"], c["Hq"], c["Hkv"], c["N"], c["D"],
                                  c["dtype"])[0])
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            out.append(_power_of("bwd_" + name,
                                 lambda: binding.bwd(q, k, v, o, lse, g, dq=dq, dk=dk, dv=dv,
                                                     **kw)))
        del q, k, v, o, lse
        torch.cuda.empty_cache()
        time.sleep(1.0)
    return out


def board_under_fwd(seconds=3.0):
    """Socket power and shader clock while the headline forward runs in a loop,
    and the bf16 MFMA peak at that clock (the published peak is counted at
    2.4 GHz); empty where amd-smi gives nothing."""
    import torch
    from sliding_window_attention_tiled_amd import binding, configs
    from sliding_window_attention_tiled_amd.inputs import fwd_inputs

    c = configs.FWD["mistral_causal_w4096"]
    q, k, v = (to_dev(x) for x in fwd_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"],
                                             c["D"], c["dtype"]))
    o = torch.empty_like(q)
    lse = torch.empty((c["B"], c["Hq"], c["N"]), dtype=torch.float32, device="cuda")
    rec = _power_of("mistral_causal_w4096",
                    lambda: binding.fwd(q, k, v, win_left=c["win_left"], out=o, lse=lse),
                    seconds=seconds)
    if "gfx_clock_mhz" not in rec:
        return {}
    peak = PEAK_BF16_TFLOPS * rec["gfx_clock_mhz"] / 2400.0
    W = c["win_left"] + 1
    exact = 4.0 * c["B"] * c["Hq"] * exact_pairs_causal(c["N"], W) * c["D"]
    tf = exact / (rec["ms_per_call"] * 1e-3) / 1e12
    return {"socket_power_w": rec["socket_power_w"], "power_cap_w": _power_cap(),
            "gfx_clock_mhz": rec["gfx_clock_mhz"], "ms_per_call": rec["ms_per_call"],
            "mfma_peak_at_clock_tflops": round(peak, 1),
            "frac_of_peak_at_clock": round(tf / peak, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.power:
        print(json.dumps({"power": bench_power()}))
        return
    if args.only == "decode":
        print(json.dumps({"decode": bench_decode(args)[0]}))
        return
    if args.only == "others":
        print(json.dumps({"other_workloads": bench_other_workloads()}))
        return
    f = bench_fwd(args)
    ms = f["ms_kernel"]
    value = f["nominal_flop"] / (ms * 1e-3) / 1e12
    exact_tf = f["exact_flop"] / (ms * 1e-3) / 1e12
    res = {
        "metric": "in-window TFLOP/s, causal SWA W=4096 N=16k bf16; decode HBM GB/s (1 GPU)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) q/k/v from a seeded PCG64 generator",
        "config": {"workload": "mistral_causal_w4096", "B": 1, "Hq": 32, "Hkv": 8,
                   "N": 16384, "D": 128, "window": 4096, "causal": True},
        "tflops_exact": round(exact_tf, 2),
        "kernel_ms": round(ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(exact_tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(exact_tf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic()},
    }
    if args.only is None:
        board = board_under_fwd()
        if board:
            res["board_under_fwd"] = board
    dec_host = None
    if not args.no_decode and args.only is None:
        res["decode"], dec_host = bench_decode(args)
    if not args.no_others and args.only is None:
        res["other_workloads"] = bench_other_workloads()
    if not args.no_cpu and args.only is None:
        res["cpu_baseline"] = cpu_baseline(f["inputs"], f["cfg"], args.cpu_rows)
        if dec_host is not None:
            res["cpu_baseline_decode"] = cpu_baseline_decode(dec_host, args.cpu_decode_steps)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
