#!/usr/bin/env python3
"""Throughput of causal linear attention (phi = ELU + 1) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg2] [--chunk 0] [--cold-only]

A step is one ``linattn_fwd`` call (causal, normaliser on) over the whole
batch of the chosen workload: segment totals, their prefix scan and the
chunked main pass.  Inputs are seeded N(0, 1) tensors already resident in
HBM.  ``value`` and ``ms_per_step`` are cold: the K timed steps each run on
their own copy of the inputs (enough copies that more than twice the 256 MiB
memory-side cache is moved between two uses of one copy), captured as one HIP
graph that is replayed right behind another graph of K steps continuing the
same rotation, after a cache sweep (a 512 MiB read); the device time between
two HIP events around the second graph over K, median of 5 measurements (the
first graph keeps the host's graph submission out of the timed region).
``roofline`` prices the dominant kernel (the chunked main pass) against HBM:
algorithmic bytes (Q, K, V read once, O written once) per launch over its cold
duration per launch, taken as the difference between the rotated cold steps
above and the same steps without their last stage (``linattn_fwd_timed`` with
reps = 0, also one HIP graph after a sweep), so that no event pair sits around
a launch.  ``stage_us`` holds each stage between HIP events (on the call's
stream, created without the system-scope fence, which costs about 1 us per
event here) in K steps that each follow a cache sweep; ``roofline_path``
prices the whole cold step.
``warm`` holds the same step with the caches warm: replayed K times back to
back from one HIP graph on the same inputs (checked bitwise against an eager
call), the eager rate with host launches, and the main pass launched 10 times
back to back.  ``cpu_baseline`` is the fp64 oracle on the same workload timed
on this host.  ``rows`` holds the other workloads (non-causal, bf16 N=16384
and N=65536 with the chunk sweep, the GQA prefill, measured the same way; the
prefill in pieces, decayed sums, packed batches and the backward as warm graph
replays; the 1024-step decode warm, plus single cold steps).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0                               # MI355X HBM3E, GB/s
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}       # dense MFMA, flop/s
ESZ = {"f32": 4, "bf16": 2}


def fwd_bytes(w) -> int:
    """Algorithmic bytes of one forward: q, k, v read once and out written once."""
    e = ESZ[w.dtype]
    return e * w.N * w.d * w.B * (2 * w.H + 2 * w.Hkv)


def fwd_flops(w) -> float:
    """The recurrence only: per kv-head token 2d^2 + 2d, per query-head token 2d^2 + 4d."""
    d = w.d
    return float(w.B * w.N) * (w.Hkv * (2 * d * d + 2 * d) + w.H * (2 * d * d + 4 * d))


def decode_bytes(B, H, Hkv, d, dtype) -> int:
    """State and normaliser read and written once, q/out/k/v once per step."""
    e = ESZ[dtype]
    return B * Hkv * (2 * d * d * 4 + 2 * d * 4) + e * d * (2 * B * H + 2 * B * Hkv)


def roofline(nbytes, flops, seconds, dtype, kernel, traffic=None):
    """traffic: measured HBM bytes per launch (PMC, calibrated) or None."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / MFMA_PEAK[dtype]
    if t_hbm >= t_mfma:
        ach = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel}
    ach = flops / seconds / 1e12
    peak = MFMA_PEAK[dtype] / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4), "traffic": traffic, "kernel": kernel}


class Hip:
    """The few HIP runtime calls the benchmark needs for events (plumbing only)."""

    # Events without the system-scope fence at record time: that fence costs
    # about 1 us per event on this GPU (measured: an empty event pair after a
    # long kernel reads 4.4 us with the default flags, 3.4 us with this one).
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e.value

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0


SOURCES = ["sequence_mixing_amd/csrc/linattn_fmt.hip", "sequence_mixing_amd/csrc/linattn_kern.h",
           "sequence_mixing_amd/csrc/linattn_plan.h", "sequence_mixing_amd/csrc/linattn_plan.cpp"]


def measured_traffic(workload: str, key_prefix: str):
    """HBM bytes per launch of a kernel from the committed PMC summary of this workload.

    The summaries (profiles/traffic_*.txt) record the SHA-256 of the kernel
    sources they were taken on; after any change to those sources the figure is
    stale and None is returned."""
    import glob

    from bench_profsum import sources_sha256

    root = os.path.dirname(os.path.abspath(__file__))
    try:
        sha = sources_sha256([os.path.join(root, f) for f in SOURCES])
    except OSError:
        return None
    for path in glob.glob(os.path.join(root, "profiles", "traffic_*.txt")):
        for line in open(path):
            if not line.startswith("json: "):
                continue
            rec = json.loads(line[6:])
            if rec.get("workload") != workload or rec.get("sources_sha256") != sha:
                continue
            hits = [v for k, v in rec["bytes_per_launch"].items() if k.startswith(key_prefix)]
            if len(hits) == 1:
                return hits[0]
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_name(w, chunk, causal):
    t = {"f32": "float", "bf16": "bf16"}[w.dtype]
    return (f"k_causal_chunks<{t},{w.d},{chunk}>" if causal else f"k_noncausal_apply<{t},{w.d}>")


def fwd_args(la, w, q, k, v, out, ws, ws_bytes, causal, chunk):
    dt = la.LINATTN_BF16 if w.dtype == "bf16" else la.LINATTN_F32
    return (q, k, v, out, w.B, w.H, w.Hkv, w.N, w.d, causal, 1, dt, None, None, chunk, ws, ws_bytes)


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def time_stages(la, hip, torch, args, steps, warmup, stream, flush=None, reps=1):
    """Steps through linattn_fwd_timed: HIP events on the library's stream around each stage.

    The last stage (the chunked pass) runs `reps` times back to back inside its
    event pair and is reported per launch.  With `flush`, the memory-side
    cache is swept before every step (warm-up steps included), outside the
    events.  Returns per-stage medians and means, and the median and minimum
    of the whole step (first event to last, device time)."""
    evs = [[hip.event() for _ in range(4)] for _ in range(steps)]
    warm = [hip.event() for _ in range(4)]

    def call(ev):
        rc = la.linattn_fwd_timed(*args, stream, events=ev, reps=reps)
        if rc != 0:
            raise la.LinattnError(rc, "linattn_fwd_timed")

    for _ in range(warmup):
        if flush is not None:
            flush()
        call(warm)
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush()
        call(evs[i])
    torch.cuda.synchronize()
    st = [[hip.ms(e[0], e[1]), hip.ms(e[1], e[2]), hip.ms(e[2], e[3]) / reps] for e in evs]
    step = [hip.ms(e[0], e[3]) - (reps - 1) * s[2] for e, s in zip(evs, st)]
    return {"stage_ms": [median([s[j] for s in st]) for j in range(3)],
            "stage_mean_ms": [sum(s[j] for s in st) / steps for j in range(3)],
            "step_ms": median(step), "step_min_ms": min(step)}


def time_eager(la, torch, args, steps, warmup, stream):
    """K plain linattn_fwd calls back to back between two synchronisations (host launch cost included)."""
    for _ in range(warmup):
        rc = la.linattn_fwd(*args, stream)
        if rc != 0:
            raise la.LinattnError(rc, "linattn_fwd")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        la.linattn_fwd(*args, stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_graph(la, hip, torch, args, out, steps):
    """The K steps captured once as a HIP graph and replayed: per-step time without host launch cost.

    Also checks that the replay leaves the same output as an eager call (bitwise:
    the kernels are deterministic)."""
    la.linattn_fwd(*args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = out.clone()
    out.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        la.linattn_fwd(*args, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            rc = la.linattn_fwd(*args, cap)
            if rc != 0:
                raise la.LinattnError(rc, "linattn_fwd (graph capture)")
    g.replay()
    torch.cuda.synchronize()
    out.zero_()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(e0, stream)
    g.replay()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    same = bool(torch.equal(out, ref))
    del g
    return {"event_ms": hip.ms(e0, e1) / steps, "ms": wall * 1e3 / steps, "matches_eager": same}


def time_rotated(la, hip, torch, w, causal, chunk, steps, flush, out_check=True):
    """K steps, each on its own copy of the inputs (enough copies that the
    steps between two uses of one copy move more than twice the 256 MiB
    memory-side cache), so every step reads its inputs from HBM.  Two graphs
    of K steps each are captured, the second continuing the rotation of the
    first (its step i takes copy (K + i) mod copies, which the first graph
    last used `copies` steps earlier); per measurement the cache is swept, the
    first graph replayed, then the second, and the second is timed between two
    HIP events: its launch was submitted while the first ran, so the host's
    graph submission is not inside the timed region and no host or event work
    sits between steps.  The same is done for the steps without their last
    stage (linattn_fwd_timed with reps = 0): the difference prices the last
    stage per launch, cold, without an event pair around each launch.
    Returns the medians over 5 measurements (ms per step, with and without the
    last stage), the copies used, and whether copy 0's output from a replay
    equals an eager call's bitwise."""
    from linattn_inputs import workload_qkv
    from sequence_mixing_amd import ops

    q, k, v = (t.cuda() for t in workload_qkv(w))
    step_bytes = fwd_bytes(w)
    ncopy = max(2, 1 + -(-(512 << 20) // step_bytes))
    copies = [(q, k, v, torch.empty_like(q))] + [(q.clone(), k.clone(), v.clone(), torch.empty_like(q))
                                                 for _ in range(ncopy - 1)]
    del q, k, v
    ws = ops.workspace(w.B, w.H, w.Hkv, w.N, w.d, causal, copies[0][0].dtype, chunk)
    ws_bytes = ws.numel() * 4 if ws is not None else 0
    argv = [fwd_args(la, w, *c, ws, ws_bytes, causal, chunk) for c in copies]
    la.linattn_fwd(*argv[0], torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = copies[0][3].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        la.linattn_fwd(*argv[0], side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    evs = [hip.event() for _ in range(4)]

    def capture(step, first):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream().cuda_stream
            for i in range(first, first + steps):
                rc = step(argv[i % ncopy], cap)
                if rc != 0:
                    raise la.LinattnError(rc, "linattn_fwd (graph capture)")
        return g

    full = [capture(lambda a, cap: la.linattn_fwd(*a, cap), f) for f in (0, steps)]
    pre = [capture(lambda a, cap: la.linattn_fwd_timed(*a, cap, events=evs, reps=0), f) for f in (0, steps)]
    copies[0][3].zero_()
    full[0].replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(copies[0][3], ref))
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    per, per_pre = [], []
    for _ in range(5):
        for (ga, gb), acc in ((full, per), (pre, per_pre)):
            flush()
            ga.replay()
            hip.record(e0, stream)
            gb.replay()
            hip.record(e1, stream)
            torch.cuda.synchronize()
            acc.append(hip.ms(e0, e1) / steps)
    del full, pre, copies, argv, ws, ref
    return {"ms": median(per), "pre_ms": median(per_pre), "copies": ncopy, "matches_eager": same}


class Flush:
    """Empties the 256 MiB memory-side cache by reading a 512 MiB buffer (outside
    any timed event pair).  It only reads: a writing sweep would leave dirty lines
    whose write-back would be billed to the next kernel."""

    def __init__(self, torch):
        self.scratch = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")
        self.torch = torch

    def __call__(self):
        self.torch.sum(self.scratch, dim=0, out=self.sink)


def timing_note(steps, copies):
    return (f"cold: {steps} steps each on its own copy of the inputs ({copies} copies, rotated), one HIP graph "
            "replayed behind another of the same rotation after a cache sweep; device time by events / steps, "
            "median of 5 replays")


def fwd_row(la, hip, torch, w, causal, chunk, steps, warmup, stream, flush, tag="", cold_only=False):
    """One workload measured; returns a summary dict.

    Primary figures are cold: the memory-side cache is swept before every step
    and each step is timed by HIP events on the library's stream (device time,
    no host launch cost); the median over the steps is reported.  `warm` holds
    the same step replayed back to back from a HIP graph (caches warm)."""
    from linattn_inputs import workload_qkv
    from sequence_mixing_amd import ops

    q, k, v = (t.cuda() for t in workload_qkv(w))
    out = torch.empty_like(q)
    ws = ops.workspace(w.B, w.H, w.Hkv, w.N, w.d, causal, q.dtype, chunk)
    ws_bytes = ws.numel() * 4 if ws is not None else 0
    dt = la.LINATTN_BF16 if w.dtype == "bf16" else la.LINATTN_F32
    _, c, P = la.linattn_fwd_plan(w.B, w.H, w.Hkv, w.N, w.d, causal, dt, chunk)
    args = fwd_args(la, w, q, k, v, out, ws, ws_bytes, causal, chunk)
    nb, fl = fwd_bytes(w), fwd_flops(w)
    kname = kernel_name(w, c, causal)
    cold = time_stages(la, hip, torch, args, steps, warmup, stream, flush=flush, reps=1)
    rot = time_rotated(la, hip, torch, w, causal, chunk, steps, flush)
    # the last stage per launch, cold: whole steps minus steps without it (rotated graphs)
    main_s = (rot["ms"] - rot["pre_ms"]) / 1e3
    main_label = kname + " (cold, per launch: rotated steps with it minus steps without it)"
    main_rot = {"us": round(main_s * 1e6, 2), "steps_without_it_ms": round(rot["pre_ms"], 5)}
    if cold_only:
        step_s = rot["ms"] / 1e3
        return {"causal": bool(causal), "chunk": c, "segments": P, "ms_per_step": round(rot["ms"], 5),
                "tokens_per_s": round(w.B * w.N / step_s, 1), "graph_matches_eager": rot["matches_eager"],
                "timing": timing_note(steps, rot["copies"]),
                "stage_us": {"seg_totals": round(cold["stage_ms"][0] * 1e3, 2),
                             "seg_scan": round(cold["stage_ms"][1] * 1e3, 2),
                             "main": round(cold["stage_ms"][2] * 1e3, 2)},
                "main_rotated": main_rot,
                "roofline_main": roofline(nb, fl, main_s, w.dtype, main_label, measured_traffic(tag, kname[:-1] + ",")),
                "roofline_path": roofline(nb, fl, step_s, w.dtype, "whole step (cold)")}
    eager_s = time_eager(la, torch, args, steps, warmup, stream)
    gr = time_graph(la, hip, torch, args, out, steps)
    warm = time_stages(la, hip, torch, args, steps, warmup, stream, reps=10)
    step_s = rot["ms"] / 1e3
    row = {
        "causal": bool(causal), "chunk": c, "segments": P,
        "ms_per_step": round(rot["ms"], 5),
        "tokens_per_s": round(w.B * w.N / step_s, 1),
        "timing": timing_note(steps, rot["copies"]),
        "single_step_ms": {"median": round(cold["step_ms"], 5), "min": round(cold["step_min_ms"], 5),
                           "note": "one step after a cache sweep, between two events (includes the events' cost)"},
        "graph_matches_eager": gr["matches_eager"] and rot["matches_eager"],
        "stage_us": {"seg_totals": round(cold["stage_ms"][0] * 1e3, 2),
                     "seg_scan": round(cold["stage_ms"][1] * 1e3, 2),
                     "main": round(cold["stage_ms"][2] * 1e3, 2)},
        "main_rotated": main_rot,
        "roofline_main": roofline(nb, fl, main_s, w.dtype, main_label, measured_traffic(tag, kname[:-1] + ",")),
        "roofline_path": roofline(nb, fl, step_s, w.dtype, "whole step (cold)"),
        "warm": {
            "ms_per_step": round(gr["event_ms"], 5), "tokens_per_s": round(w.B * w.N / (gr["event_ms"] / 1e3), 1),
            "launch": "the steps replayed back to back from one HIP graph, device time by events",
            "eager_ms_per_step": round(eager_s * 1e3, 5),
            "stage_us": {"seg_totals": round(warm["stage_ms"][0] * 1e3, 2),
                         "seg_scan": round(warm["stage_ms"][1] * 1e3, 2),
                         "main": round(warm["stage_ms"][2] * 1e3, 2)},
            "roofline_main": roofline(nb, fl, warm["stage_ms"][2] / 1e3, w.dtype,
                                      kname + " (warm, 10 launches back to back)"),
        },
    }
    if not causal:
        # pass 1, the reduction phi(K)^T V, sum phi(K) over every token: K and V
        # read once (the partial sums it writes are not counted)
        kv = 2 * w.B * w.Hkv * w.N * w.d * (2 if w.dtype == "bf16" else 4)
        # fp32 rows take the pass without staging, k_seg_totals_f32<d, ...>
        kn = f"k_seg_totals_f32<{w.d}" if w.dtype == "f32" else f"k_seg_totals<bf16,{w.d}"
        row["roofline_reduction"] = roofline(kv, 0.0, cold["stage_ms"][0] / 1e3, w.dtype,
                                             f"{kn}> (pass 1, cold)", measured_traffic(tag, kn + ","))
    del q, k, v, out, ws
    return row


def pieces_row(la, hip, torch, w, pieces, steps):
    """The causal prefill of w run as `pieces` equal pieces through linattn_fwd_from_state,
    each piece starting from the sums the previous one ended with (chunked prefill).

    The whole chain (all pieces) is one step; steps are captured as one HIP graph."""
    from linattn_inputs import workload_qkv
    from sequence_mixing_amd import ops

    q, k, v = (t.cuda() for t in workload_qkv(w))
    n = w.N // pieces
    assert n * pieces == w.N
    dt = la.LINATTN_BF16 if w.dtype == "bf16" else la.LINATTN_F32
    sl = [(slice(None), slice(None), slice(i * n, (i + 1) * n)) for i in range(pieces)]
    qs, ks, vs = ([t[s].contiguous() for s in sl] for t in (q, k, v))
    outs = [torch.empty_like(x) for x in qs]
    S = [torch.zeros(w.B, w.Hkv, w.d, w.d, device="cuda") for _ in range(2)]
    z = [torch.zeros(w.B, w.Hkv, w.d, device="cuda") for _ in range(2)]
    S0 = torch.zeros_like(S[0])
    z0 = torch.zeros_like(z[0])
    ws = ops.workspace(w.B, w.H, w.Hkv, n, w.d, 1, q.dtype)
    ws_bytes = ws.numel() * 4 if ws is not None else 0
    _, c, P = la.linattn_fwd_plan(w.B, w.H, w.Hkv, n, w.d, 1, dt, 0)

    def chain(st):
        for i in range(pieces):
            si, zi = (S0, z0) if i == 0 else (S[(i - 1) % 2], z[(i - 1) % 2])
            rc = la.linattn_fwd_from_state(qs[i], ks[i], vs[i], outs[i], w.B, w.H, w.Hkv, n, w.d, 1, 1, dt, si, zi,
                                           S[i % 2], z[i % 2], 0, ws, ws_bytes, st)
            if rc != 0:
                raise la.LinattnError(rc, "linattn_fwd_from_state")

    chain(torch.cuda.current_stream().cuda_stream)
    whole = ops.fwd(q, k, v)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2).float()
    ref = whole.float()
    err = ((got - ref).abs().amax(-1) / ref.abs().amax(-1).clamp_min(1e-30)).max().item()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            chain(cap)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    g.replay()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.ms(e0, e1) / steps
    del g
    nb, fl = fwd_bytes(w), fwd_flops(w)
    return {"pieces": pieces, "piece_tokens": n, "chunk": c, "segments_per_piece": P,
            "ms_per_step": round(ms, 5), "tokens_per_s": round(w.B * w.N / (ms / 1e3), 1),
            "max_row_rel_diff_vs_one_pass": err,
            "roofline_path": roofline(nb, fl, ms / 1e3, w.dtype, "whole chain (graph replay, events)")}


def bwd_bytes(w) -> int:
    """Algorithmic HBM bytes of the backward: q, o, dO read and dq written per query
    head; k, v read and dk, dv written per kv head (each once)."""
    e = 2 if w.dtype == "bf16" else 4
    return w.B * w.N * w.d * e * (4 * w.H + 4 * w.Hkv)


def bwd_row(la, hip, torch, w, causal, steps):
    """linattn_bwd on a workload: all its launches as one step, K steps in one HIP graph."""
    from linattn_inputs import randn, workload_qkv
    from sequence_mixing_amd import ops

    q, k, v = (t.cuda() for t in workload_qkv(w))
    dout = randn((w.B, w.H, w.N, w.d), w.seed + 1).to(q.dtype).cuda()
    out = ops.fwd(q, k, v, causal=causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dt = la.LINATTN_BF16 if w.dtype == "bf16" else la.LINATTN_F32
    nb = la.linattn_bwd_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.d, causal, dt)
    ws = torch.empty(nb // 4 + 1, dtype=torch.float32, device="cuda")

    def call(st):
        rc = la.linattn_bwd(q, k, v, out, dout, dq, dk, dv, w.B, w.H, w.Hkv, w.N, w.d, causal, 1, dt, ws, nb, st)
        if rc != 0:
            raise la.LinattnError(rc, "linattn_bwd")

    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            call(cap)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    g.replay()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.ms(e0, e1) / steps
    same = all(torch.equal(a, b) for a, b in zip(ref, (dq, dk, dv)))
    del g
    nb_alg = bwd_bytes(w)
    return {"causal": bool(causal), "ms_per_step": round(ms, 5), "tokens_per_s": round(w.B * w.N / (ms / 1e3), 1),
            "graph_matches_eager": same,
            "roofline_path": roofline(nb_alg, 0.0, ms / 1e3, w.dtype, "whole backward (graph replay, events)")}


def bwd_oracle(w, causal, seconds, max_tokens=1024):
    """The fp64 oracle's backward on the first `max_tokens` tokens of every sequence."""
    import numpy as np

    import oracle
    from linattn_inputs import randn, workload_qkv

    n = min(w.N, max_tokens)
    q, k, v = (np.ascontiguousarray(t[:, :, :n].double().numpy()) for t in workload_qkv(w))
    dout = np.ascontiguousarray(randn((w.B, w.H, w.N, w.d), w.seed + 1)[:, :, :n].double().numpy())
    threads = oracle.default_threads()
    o = oracle.ref_fwd(q, k, v, causal=bool(causal), nthreads=threads)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ref_bwd(q, k, v, o, dout, causal=bool(causal), nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return {"value": round(w.B * n * reps / el, 1), "unit": "tokens/s", "cores": min(threads, w.B * w.Hkv),
            "kind": "oracle", "sample": f"backward of the first {n} of {w.N} tokens of all {w.B * w.Hkv} sequences, "
                                        f"{reps} reps in {el:.1f} s"}


def packed_row(la, hip, torch, steps):
    """linattn_fwd_packed on the seeded packed batch (sequences of different lengths, no
    padding), K steps in one HIP graph; tokens/s counts real tokens only."""
    from linattn_inputs import PACKED, packed_qkv
    from sequence_mixing_amd import ops

    P = PACKED
    lens, seqs = packed_qkv(P)
    qf, cu = ops.pack([s[0][0] for s in seqs])
    kf, _ = ops.pack([s[1][0] for s in seqs])
    vf, _ = ops.pack([s[2][0] for s in seqs])
    qf, kf, vf, cu = qf.cuda(), kf.cuda(), vf.cuda(), cu.cuda()
    total = sum(lens)
    dt = la.LINATTN_BF16 if P["dtype"] == "bf16" else la.LINATTN_F32
    nb = la.linattn_fwd_packed_workspace_bytes(len(lens), P["H"], P["Hkv"], total, P["d"], 1, dt)
    ws = torch.empty(nb // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty_like(qf)

    def call(st):
        rc = la.linattn_fwd_packed(qf, kf, vf, out, cu, len(lens), total, P["H"], P["Hkv"], P["d"], 1, 1, dt,
                                   None, None, 0, ws, nb, st)
        if rc != 0:
            raise la.LinattnError(rc, "linattn_fwd_packed")

    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            call(cap)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    g.replay()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.ms(e0, e1) / steps
    same = bool(torch.equal(out, ref))
    del g
    e = 2 if P["dtype"] == "bf16" else 4
    nbytes = total * P["d"] * e * (2 * P["H"] + 2 * P["Hkv"])
    return {"workload": P["name"], "sequences": len(lens), "total_tokens": total, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(total / (ms / 1e3), 1), "graph_matches_eager": same,
            "roofline_path": roofline(nbytes, 0.0, ms / 1e3, P["dtype"], "whole packed forward (graph replay, events)")}


def graph_ms(hip, torch, call, out, steps):
    """ms per call of `call(stream)` replayed `steps` times from one HIP graph, and
    whether the replayed output equals the eager call's bitwise."""
    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            call(cap)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    g.replay()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.ms(e0, e1) / steps
    same = bool(torch.equal(out, ref))
    del g
    return ms, same


def decay_row(la, hip, torch, steps):
    """linattn_fwd_decay on the decayed workload (cfg3's shape with a per-token gate), K
    calls in one HIP graph, beside the plain forward pass of the same inputs."""
    from linattn_inputs import DECAY, make_decay, make_qkv

    w = DECAY
    q, k, v = (t.cuda() for t in make_qkv(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.seed))
    g = make_decay(w.B, w.Hkv, w.N, w.seed + 1).cuda()
    dt = la.LINATTN_BF16 if w.dtype == "bf16" else la.LINATTN_F32
    nb = la.linattn_fwd_decay_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.d, dt, 0)
    ws = torch.empty(nb // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)

    def call(st):
        rc = la.linattn_fwd_decay(q, k, v, g, out, w.B, w.H, w.Hkv, w.N, w.d, 1, dt, None, None, None, None, 0, ws,
                                  nb, st)
        if rc != 0:
            raise la.LinattnError(rc, "linattn_fwd_decay")

    def plain(st):
        rc = la.linattn_fwd(q, k, v, out, w.B, w.H, w.Hkv, w.N, w.d, 1, 1, dt, None, None, 0, ws, nb, st)
        if rc != 0:
            raise la.LinattnError(rc, "linattn_fwd")

    ms_plain, _ = graph_ms(hip, torch, plain, out, steps)
    ms, same = graph_ms(hip, torch, call, out, steps)
    nbytes = fwd_bytes(w) + 4 * w.B * w.Hkv * w.N  # + the log-decays
    return {"workload": w.name, "ms_per_step": round(ms, 5), "tokens_per_s": round(w.B * w.N / (ms / 1e3), 1),
            "graph_matches_eager": same, "plain_forward_ms": round(ms_plain, 5),
            "roofline_path": roofline(nbytes, 0.0, ms / 1e3, w.dtype, "whole decayed forward (graph replay, events)")}


def window_row(la, hip, torch, steps, W=256):
    """Sliding-window pass (band of W keys) on the bf16 B2 H8 N16384 d64 shape, replayed
    from one HIP graph (warm), beside the plain causal pass of the same inputs."""
    from linattn_inputs import WORKLOADS, workload_qkv

    w = WORKLOADS["cfg3"]
    q, k, v = (t.cuda() for t in workload_qkv(w))
    out = torch.empty_like(q)
    dt = la.LINATTN_BF16

    def call(st):
        rc = la.linattn_fwd_window(q, k, v, out, w.B, w.H, w.Hkv, w.N, w.d, W, 1, dt, st)
        if rc != 0:
            raise la.LinattnError(rc, "linattn_fwd_window")

    ms, same = graph_ms(hip, torch, call, out, steps)
    nb = fwd_bytes(w)
    # the band's flops: per query-head token and key of its band, 2d for the score, 2d for the value
    # product and 2 for the denominator (the masked half of the diagonal tile is not counted)
    band = sum(min(t + 1, W) for t in range(w.N))
    fl = float(w.B * w.H) * band * (4 * w.d + 2)
    row = {"window": W, "workload": "bf16 B2 H8 N16384 d64", "ms_per_step": round(ms, 5),
           "tokens_per_s": round(w.B * w.N / (ms / 1e3), 1), "graph_matches_eager": same,
           "roofline_path": roofline(nb, fl, ms / 1e3, w.dtype, "k_window<bf16,64> (graph replay, warm)"),
           "band_tflops": round(fl / (ms / 1e3) / 1e12, 2)}
    del q, k, v, out
    return row


def window_oracle(seconds, W=256, max_tokens=2048):
    """The oracle's band sum on the first tokens of every sequence of the window workload."""
    import numpy as np

    import oracle
    from linattn_inputs import WORKLOADS, workload_qkv

    w = WORKLOADS["cfg3"]
    n = min(w.N, max_tokens)
    q, k, v = (np.ascontiguousarray(t[:, :, :n].double().numpy()) for t in workload_qkv(w))
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ref_fwd_window(q, k, v, W, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return {"value": round(w.B * n * reps / el, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {w.N} tokens of all {w.B * w.H} heads, W = {W}, {reps} reps in {el:.1f} s"}


def decay_oracle(seconds, max_tokens=2048):
    """The fp64 oracle's decayed recurrence on the first tokens of every sequence of the
    decayed workload (the cost per token does not depend on the position)."""
    import numpy as np

    import oracle
    from linattn_inputs import DECAY, make_decay, make_qkv

    w = DECAY
    n = min(w.N, max_tokens)
    q, k, v = (np.ascontiguousarray(t[:, :, :n].double().numpy())
               for t in make_qkv(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.seed))
    g = np.ascontiguousarray(make_decay(w.B, w.Hkv, w.N, w.seed + 1)[:, :, :n].double().numpy())
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ref_fwd_decay(q, k, v, g, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return {"value": round(w.B * n * reps / el, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {w.N} tokens of all {w.B * w.Hkv} sequences, {reps} reps in {el:.1f} s"}


def packed_oracle(seconds):
    """The fp64 oracle on the first sequences of the packed batch, one after another."""
    import oracle
    from linattn_inputs import packed_qkv

    lens, seqs = packed_qkv()
    threads = oracle.default_threads()
    done, t0 = 0, time.perf_counter()
    for (q, k, v), n in zip(seqs, lens):
        oracle.ref_fwd(q, k, v, nthreads=threads)
        done += n
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(done / el, 1), "unit": "tokens/s", "cores": min(threads, 8), "kind": "oracle",
            "sample": f"the first {done} tokens of the packed batch, sequence by sequence, in {el:.1f} s"}


def decode_row(la, hip, torch, steps_total, stream, flush=None, cold_steps=20):
    """GQA prefill (N=32768), state replicated into 64 slots, 1024 decode steps.

    The graph-replayed steps keep the 32 MiB state in the 256 MiB memory-side
    cache (warm); with `flush`, `cold_steps` more steps each follow a cache
    sweep, so the state comes from HBM, and are timed one by one by events."""
    from linattn_inputs import DECODE, WORKLOADS, DecodeStream, workload_qkv
    from sequence_mixing_amd import ops

    w, dw = WORKLOADS["cfg5"], DECODE
    q, k, v = (t.cuda() for t in workload_qkv(w))
    _, S1, z1 = ops.fwd(q, k, v, want_state=True)
    del q, k, v
    S = S1.expand(dw.B, -1, -1, -1).contiguous()
    z = z1.expand(dw.B, -1, -1).contiguous()
    gen = DecodeStream(dw.B, dw.H, dw.Hkv, dw.d, dw.dtype, dw.seed)
    qs, ks, vs = [], [], []
    for _ in range(steps_total):
        a, b, c = gen.next()
        qs.append(a)
        ks.append(b)
        vs.append(c)
    qs, ks, vs = torch.stack(qs).cuda(), torch.stack(ks).cuda(), torch.stack(vs).cuda()
    out = torch.empty(steps_total, dw.B, dw.H, dw.d, dtype=qs.dtype, device="cuda")
    dt = la.LINATTN_BF16
    # eager pass (host launch cost included): one event pair around the loop
    S0, z0 = S.clone(), z.clone()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for t in range(steps_total):
        rc = la.linattn_decode_step(S, z, qs[t], ks[t], vs[t], out[t], dw.B, dw.H, dw.Hkv, dw.d, 1, dt, stream)
        assert rc == 0
    hip.record(e1, stream)
    torch.cuda.synchronize()
    eager_us = hip.ms(e0, e1) / steps_total * 1e3
    ref = out.clone()
    # the same 1024 steps captured as one HIP graph and replayed from the same
    # start state: per-step kernel time with no host in the loop
    S.copy_(S0)
    z.copy_(z0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for t in range(steps_total):
            la.linattn_decode_step(S, z, qs[t], ks[t], vs[t], out[t], dw.B, dw.H, dw.Hkv, dw.d, 1, dt, cap)
    S.copy_(S0)
    z.copy_(z0)
    out.zero_()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    hip.record(e0, stream)
    g.replay()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_us = hip.ms(e0, e1) / steps_total * 1e3
    same = bool(torch.equal(out, ref))
    nb = decode_bytes(dw.B, dw.H, dw.Hkv, dw.d, dw.dtype)
    fl = float(dw.B) * (dw.Hkv * (2 * dw.d ** 2 + 2 * dw.d) + dw.H * (2 * dw.d ** 2 + 4 * dw.d))
    res = {
        "batch": dw.B, "steps": steps_total,
        "graph_us_per_step": round(k_us, 2),
        "tokens_per_s": round(dw.B * steps_total / wall, 1),
        "graph_matches_eager": same,
        "eager_us_per_step": round(eager_us, 2),
        "roofline": roofline(nb, fl, k_us / 1e6, "bf16",
                             "k_decode_step<bf16,128> (graph replay, per step; state resident in the memory-side cache)",
                             measured_traffic("decode", "k_decode_step<bf16,128,")),
        "note": "warm: the state (32 MiB fp32) stays in the 256 MiB memory-side cache between replayed steps",
    }
    if flush is not None:
        cold, gap = [], []
        for t in range(cold_steps):
            flush()
            hip.record(e0, stream)
            la.linattn_decode_step(S, z, qs[t], ks[t], vs[t], out[t], dw.B, dw.H, dw.Hkv, dw.d, 1, dt, stream)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            cold.append(hip.ms(e0, e1) * 1e3)
            flush()
            hip.record(e0, stream)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            gap.append(hip.ms(e0, e1) * 1e3)
        c_us = median(cold)
        res["cold_us_per_step"] = round(c_us, 2)
        res["cold_event_gap_us"] = round(median(gap), 2)
        res["roofline_cold"] = roofline(nb, fl, c_us / 1e6, "bf16",
                                        "k_decode_step<bf16,128> (one step after a cache sweep, state from HBM; "
                                        "event pair around one launch)")

    del S, z, qs, ks, vs, out, g
    res["state_beyond_cache"] = decode_hbm(la, hip, torch, S1, z1, dw)
    return res


def decode_hbm(la, hip, torch, S1, z1, dw, batch=1024, steps=32):
    """Decode steps of the cfg5 shape at a batch whose state (512 MiB fp32) is twice the
    256 MiB memory-side cache: replayed back to back from one HIP graph, every step streams
    the state from HBM, so the per-step time prices the kernel against HBM."""
    from linattn_inputs import DecodeStream

    S = S1.expand(batch, -1, -1, -1).contiguous()
    z = z1.expand(batch, -1, -1).contiguous()
    gen = DecodeStream(batch, dw.H, dw.Hkv, dw.d, dw.dtype, dw.seed + 1)
    qs, ks, vs = (torch.stack(x).cuda() for x in zip(*(gen.next() for _ in range(steps))))
    out = torch.empty(steps, batch, dw.H, dw.d, dtype=qs.dtype, device="cuda")
    dt = la.LINATTN_BF16
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream().cuda_stream
        for t in range(steps):
            la.linattn_decode_step(S, z, qs[t], ks[t], vs[t], out[t], batch, dw.H, dw.Hkv, dw.d, 1, dt, cap)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    g.replay()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    us = hip.ms(e0, e1) / steps * 1e3
    nb = decode_bytes(batch, dw.H, dw.Hkv, dw.d, dw.dtype)
    fl = float(batch) * (dw.Hkv * (2 * dw.d ** 2 + 2 * dw.d) + dw.H * (2 * dw.d ** 2 + 4 * dw.d))
    del S, z, qs, ks, vs, out, g
    return {"batch": batch, "steps": steps, "graph_us_per_step": round(us, 2),
            "tokens_per_s": round(batch / (us / 1e6), 1),
            "roofline": roofline(nb, fl, us / 1e6, "bf16",
                                 f"k_decode_step<bf16,128> (graph replay, per step; batch {batch}: the "
                                 f"{batch * dw.Hkv * dw.d * dw.d * 4 >> 20} MiB state is twice the memory-side "
                                 "cache, so it streams from HBM every step)")}


def cpu_baseline(w, seconds):
    """The fp64 oracle on the whole workload, repeated until `seconds` have passed."""
    import numpy as np

    import oracle
    from linattn_inputs import workload_qkv

    q, k, v = (np.ascontiguousarray(t.double().numpy()) for t in workload_qkv(w))
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ref_fwd(q, k, v, causal=True, normalise=True, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return {"value": round(w.B * w.N * reps / el, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole workload ({w.B}x{w.N} tokens, {w.H} heads), {reps} reps in {el:.1f} s, fp64 C, "
                      f"{threads} threads over (batch, kv head, 16-column block)"}


def row_oracle(w, causal, seconds, max_tokens=2048):
    """The fp64 oracle on a bounded sample of a workload: the first `max_tokens`
    tokens of every (batch, kv head) sequence with all their query heads.  The
    recurrence's cost per token does not depend on how many came before, so
    tokens/s of the sample is the whole workload's rate."""
    import numpy as np

    import oracle
    from linattn_inputs import workload_qkv

    n = min(w.N, max_tokens)
    q, k, v = (np.ascontiguousarray(t[:, :, :n].double().numpy()) for t in workload_qkv(w))
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.ref_fwd(q, k, v, causal=bool(causal), normalise=True, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return {"value": round(w.B * n * reps / el, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {w.N} tokens of all {w.B * w.Hkv} sequences ({w.H} query heads), "
                      f"{reps} reps in {el:.1f} s"}


def decode_oracle(seconds):
    """The fp64 oracle's decode step at batch 64 (state from zero: the cost does not depend on it)."""
    import numpy as np

    import oracle
    from linattn_inputs import DECODE, DecodeStream

    dw = DECODE
    S = np.zeros((dw.B, dw.Hkv, dw.d, dw.d))
    z = np.zeros((dw.B, dw.Hkv, dw.d))
    gen = DecodeStream(dw.B, dw.H, dw.Hkv, dw.d, dw.dtype, dw.seed)
    steps, t0 = 0, time.perf_counter()
    while True:
        qs, ks, vs = gen.next()
        oracle.ref_decode_step(S, z, qs, ks, vs, normalise=True)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds or steps >= 1024:
            break
    return {"value": round(dw.B * steps / el, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} decode steps at batch {dw.B} in {el:.1f} s (single thread)"}


def gpu_clocks():
    """Current shader (sclk) and memory (mclk) clocks of the GPU in MHz, read
    after the timed work with rocm-smi in a child process; None if unavailable."""
    import re
    import subprocess

    # Under a profiler that preloads itself into child processes the tool's
    # interpreter would start with the GPU already initialised and could not
    # re-exec itself: the figures are left out there.
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout)
    except Exception:  # no tool, no JSON: the figures are optional
        return None
    dev = os.environ.get("HIP_VISIBLE_DEVICES", "0").split(",")[0] or "0"
    card = data.get(f"card{dev}") or next((v for k, v in data.items() if k.startswith("card")), None)
    if not isinstance(card, dict):
        return None
    out = {}
    for key, val in card.items():
        m = re.search(r"(\d+)\s*Mhz", str(val), re.IGNORECASE)
        for name in ("sclk", "mclk"):
            if name in key.lower() and m and f"{name}_mhz" not in out:
                out[f"{name}_mhz"] = int(m.group(1))
    if not out:
        return None
    out["source"] = "rocm-smi --showclocks, after the timed work"
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="cfg2", choices=["cfg1", "cfg2", "cfg3", "cfg4", "cfg5"])
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--rows", type=int, default=1, help="also measure the other workloads (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--causal", type=int, default=1,
                    help="0: the timed workload runs the non-causal path instead (for profiling it alone)")
    ap.add_argument("--cold-only", action="store_true",
                    help="only the cold steps of the timed workload (no warm replay, no rows): a kernel "
                         "trace of this run holds cold launches only")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the sharded path is not part of this library.", file=sys.stderr)
        sys.exit(2)

    import torch

    import sequence_mixing_amd as la
    from linattn_inputs import WORKLOADS

    la.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    w = WORKLOADS[args.workload]
    log(f"workload {args.workload}: {w.name}; steps {args.steps}, warmup {args.warmup}")

    tag = args.workload if args.causal else args.workload + "_noncausal"
    flush = Flush(torch)
    head = fwd_row(la, hip, torch, w, args.causal, args.chunk, args.steps, args.warmup, stream, flush, tag=tag,
                   cold_only=args.cold_only)
    if args.cold_only:
        args.rows = 0
    log("headline", json.dumps(head))
    rows = {}
    if args.rows:
        if args.workload == "cfg2":
            rows["cfg2_noncausal"] = fwd_row(la, hip, torch, w, 0, args.chunk, 20, 5, stream, flush,
                                             tag="cfg2_noncausal")
            if args.cpu_seconds > 0:
                rows["cfg2_noncausal"]["cpu_oracle"] = row_oracle(w, 0, min(2.0, args.cpu_seconds))
            log("cfg2_noncausal", json.dumps(rows["cfg2_noncausal"]))
        for name, chunk in (("cfg3", 0), ("cfg4_c64", 64), ("cfg4_c128", 128), ("cfg4_c256", 256), ("cfg5_prefill", 0)):
            key = name.split("_")[0] if name != "cfg5_prefill" else "cfg5"
            rows[name] = fwd_row(la, hip, torch, WORKLOADS[key], 1, chunk, 20, 5, stream, flush,
                                 tag=name)
            if args.cpu_seconds > 0 and name != "cfg4_c64" and name != "cfg4_c256":
                rows[name]["cpu_oracle"] = row_oracle(WORKLOADS[key], 1, min(2.0, args.cpu_seconds))
            log(name, json.dumps(rows[name]))
        rows["cfg5_prefill_4_pieces"] = pieces_row(la, hip, torch, WORKLOADS["cfg5"], 4, 20)
        log("cfg5_prefill_4_pieces", json.dumps(rows["cfg5_prefill_4_pieces"]))
        rows["decay"] = decay_row(la, hip, torch, 20)
        if args.cpu_seconds > 0:
            rows["decay"]["cpu_oracle"] = decay_oracle(min(2.0, args.cpu_seconds))
        log("decay", json.dumps(rows["decay"]))
        rows["window"] = window_row(la, hip, torch, 20)
        if args.cpu_seconds > 0:
            rows["window"]["cpu_oracle"] = window_oracle(min(2.0, args.cpu_seconds))
        log("window", json.dumps(rows["window"]))
        rows["packed"] = packed_row(la, hip, torch, 20)
        if args.cpu_seconds > 0:
            rows["packed"]["cpu_oracle"] = packed_oracle(min(2.0, args.cpu_seconds))
        log("packed", json.dumps(rows["packed"]))
        for name, key in (("cfg2_bwd", "cfg2"), ("cfg3_bwd", "cfg3"), ("cfg5_bwd", "cfg5")):
            rows[name] = bwd_row(la, hip, torch, WORKLOADS[key], 1, 10)
            if args.cpu_seconds > 0:
                rows[name]["cpu_oracle"] = bwd_oracle(WORKLOADS[key], 1, min(2.0, args.cpu_seconds))
            log(name, json.dumps(rows[name]))
        rows["cfg5_decode"] = decode_row(la, hip, torch, 1024, stream, flush)
        if args.cpu_seconds > 0:
            rows["cfg5_decode"]["cpu_oracle"] = decode_oracle(min(2.0, args.cpu_seconds))
        log("cfg5_decode", json.dumps(rows["cfg5_decode"]))

    cpu = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    if cpu:
        log("cpu_baseline", json.dumps(cpu))

    tok_s = head["tokens_per_s"]
    if not head.get("graph_matches_eager", True):
        raise SystemExit("graph replay output differs from the eager call")
    res = {
        "metric": "causal linear-attn fwd tokens/s (B2 H8 d64) + % of MFMA/HBM roofline",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) q, k, v (no dataset involved)",
        "config": {"workload": f"{args.workload}: {w.name}, {'causal' if args.causal else 'non-causal'}, "
                               "normaliser on", "B": w.B, "H": w.H,
                   "Hkv": w.Hkv, "N": w.N, "d": w.d, "chunk": head["chunk"], "segments": head["segments"],
                   "timing": head["timing"]},
        "roofline": head["roofline_main"],
        "roofline_path": head["roofline_path"],
        "single_step_ms": head.get("single_step_ms"),
        "stage_us": head["stage_us"],
        "warm": head.get("warm"),
        "cpu_baseline": cpu,
        "gpu_clocks": gpu_clocks(),
        "rows": rows,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
