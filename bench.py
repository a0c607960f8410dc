#!/usr/bin/env python3
"""Decode-step benchmark of libkvq on one MI355X.

A step is one pass of the whole decode hot path for one attention layer over a
batch of sequences: kvq_append (the new token; a residual flush when a window
is full) then kvq_decode_attn (split partials + combine).  Steps rotate over
--layers independent layer caches (by default as many as keep at least 1 GB
of decode bytes in rotation, and at least 4: 4 for the default workload) so the
256 MB Infinity Cache cannot serve a layer's cache from one step to the next:
the bytes come from HBM, as in a real multi-layer model.

Every timed step runs at the workload's context.  A steady step appends at
position context - 1 and attends over the context; a flush step appends into a
full window, flushes it and attends over the next multiple of R plus one.
Both kinds repeat the same work on every pass (an append at a fixed position
rewrites the same slots), so K steps of a kind are captured as one HIP graph
and replayed many times; the median replay gives the time per step.  value
amortizes one flush step per R / T steps (the rate a decode loop at these
contexts flushes at), so it does not depend on --steps or --warmup.

Default workload: the Llama-3-8B-shaped GQA layer (32 query / 8 KV heads,
head_dim 128, batch 32, context 8192, 2-bit keys / 4-bit values, G = 32,
R = 128).  --config 6 runs the KV1-shaped layer in the rotated per-token 2-bit
format (kvq_bq2_append + kvq_bq2_decode_attn, batch 16, context 32768).

Prints one JSON line: effective HBM GB/s of the whole step (algorithmic bytes /
time), tokens/s, the steady and flush steps apart, the roofline of the dominant
kernel (decode partial: HIP events around each launch on the launch stream)
and the CPU oracle timed on a bounded sample of the same workload on the host
cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=128)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--config", type=int, default=3, help="workload 1..6 (default 3)")
    p.add_argument("--layers", type=int, default=0,
                   help="rotating layer caches (0: enough for 1 GB of decode bytes, at "
                        "least 4, at most 16)")
    p.add_argument("--tokens", type=int, default=1,
                   help="query tokens per sequence per step (T > 1: kvq_append_tokens, then "
                        "kvq_decode_attn_multi; KIVI-format workloads)")
    p.add_argument("--page-size", type=int, default=0,
                   help="KIVI workloads: a paged cache with pages of this many positions, "
                        "handed out in shuffled order (0: the dense cache)")
    p.add_argument("--eager", action="store_true",
                   help="time the steps as launched one by one (default: the timed steps "
                        "are also captured as one HIP graph, and value is the median of "
                        "its replays)")
    p.add_argument("--eager-launches", type=int, default=1024,
                   help="at least this many eager steps of each kind carry the per-launch "
                        "kernel events (fewer for a profiled run)")
    p.add_argument("--min-seconds", type=float, default=0.3,
                   help="graph replays continue until they cover this much time (and at "
                        "least 10 replays)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--probe-sweep", action="store_true",
                   help="only sweep the plain stream-read probe over waves per SIMD, loads "
                        "in flight per lane and nontemporal loads; prints one JSON line")
    p.add_argument("--probe-chunks", action="store_true",
                   help="only run the chunk-stream probe: the decode partial kernel's loads for "
                        "the --config workload (its 32-token chunk pieces, one chunk per work "
                        "unit) without the arithmetic, then with 16..192 dependent FMAs per "
                        "chunk; prints one JSON line")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (5 times); used to "
                        "calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return p.parse_args()


# kernel sources whose change invalidates a committed traffic reading
KERNEL_SOURCES = {
    "decode_partial": ("kvq_decode_impl.h", "kvq_decode_inst.hip", "kvq_device.h",
                       "kvq_quant.hip", "kvq_internal.h"),
    "bq2_partial": ("kvq_bq2_decode.hip", "kvq_device.h", "kvq_bq2_quant.hip", "kvq_internal.h"),
}


def source_hash(kernel: str = "decode_partial") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "quantized_decode_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str = "decode_partial"):
    """HBM traffic per partial-kernel launch from committed rocprofv3 --pmc
    summaries, if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash(kernel):
        return None
    return d.get("bytes_per_launch")


def _timed_oracle_steps(run_step, seconds: float, max_steps: int):
    """Runs run_step(i) -> bytes until about `seconds` have passed (at least
    one step); returns (steps, bytes, seconds)."""
    steps, nbytes, t_total = 0, 0.0, 0.0
    while steps < 1 or (t_total < seconds and steps < max_steps):
        t0 = time.perf_counter()
        b = run_step(steps)
        t_total += time.perf_counter() - t0
        nbytes += b
        steps += 1
    return steps, nbytes, t_total


def _baseline_record(w, bs, ctx, steps, nbytes, t_total, threads, one, extra_sample="",
                     T=1):
    """cpu_baseline entry: the all-thread run, the one-thread run beside it, and
    the whole workload's oracle time extrapolated from the all-thread time per
    sequence-step (labelled as such)."""
    per_seq_step = t_total / (bs * steps)
    whole = per_seq_step * w.batch * w.layers * max(w.steps, 1)
    o_steps, o_bytes, o_t = one
    return {
        "value": round(nbytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(bs * T * steps / t_total, 3),
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{bs} of {w.batch} sequences at context {ctx}, {steps} decode steps "
                   f"(append + attention){extra_sample}, {t_total:.1f} s on {threads} threads"),
        "single_thread": {"value": round(o_bytes / o_t / 1e9, 4), "unit": "GB/s",
                          "tokens_per_s": round(bs * T * o_steps / o_t, 3), "cores": 1,
                          "sample": f"the same sequences, {o_steps} steps, {o_t:.1f} s"},
        "whole_workload_s_extrapolated": {
            "value": round(whole, 4),
            "what": (f"{w.batch} sequences x {w.layers} layers x {max(w.steps, 1)} steps at "
                     f"the sample's per-sequence-step time on {threads} threads "
                     "(extrapolated, not run)")},
    }


def cpu_baseline(w, target_seconds: float, T: int = 1):
    """The oracle, as it stands, on a bounded sample of the workload: the first
    few sequences of the batch, decode steps (T appends, then attention) from
    the workload's context, for about target_seconds on all host threads, then
    about a third of that on one thread.  Every R / T steps (one flush) the
    lengths start again from the context."""
    import oracle
    from quantized_decode_attention_amd import metrics, synth

    bs = min(w.batch, 4)
    ctx = int(np.mean(synth.seq_lens(w))) if w.ctx_range else w.context
    n0 = ctx - T
    cap = synth.capacity_for(w, w.residual + T)
    og = oracle.Geom(bs, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                     w.group, w.residual, cap)
    k = synth.keys(w, n0, batch=bs)
    v = synth.values(w, n0, batch=bs)
    oc = oracle.Cache(og)
    oracle.prefill(og, oc, k, v, n0)
    del k, v
    scale = 1.0 / math.sqrt(w.head_dim)
    lens = np.full(bs, n0, np.int32)
    cycle = max(1, w.residual // T)

    def run_step(i):
        if i % cycle == 0:  # one window's worth of steps (one flush), then from n0 again
            lens[:] = n0
        before = lens.copy()
        qs = []
        for j in range(T):
            kn, vn, q = synth.step_token(w, i * T + j, batch=bs)
            oracle.append(og, oc, kn, vn, lens)
            lens[:] += 1
            qs.append(q)
        if T == 1:
            oracle.decode_attn(og, oc, qs[0], lens, scale)
        else:
            oracle.decode_attn_multi(og, oc, np.stack(qs, 1), lens, T, scale)
        b = metrics.decode_step_bytes(lens, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits,
                                      w.v_bits, w.group, w.residual)
        b += (T - 1) * 4 * bs * w.n_q_heads * w.head_dim
        b += T * metrics.append_bytes(bs, w.n_kv_heads, w.head_dim)
        for j in range(T):
            flushing = int(np.sum((before + j > 0) & ((before + j) % w.residual == 0)))
            b += metrics.flush_bytes(flushing * w.n_kv_heads, w.residual, w.head_dim,
                                     w.k_bits, w.v_bits, w.group)
        return b

    threads = oracle.max_threads()
    steps, nbytes, t_total = _timed_oracle_steps(run_step, target_seconds, 100000)
    oracle.set_threads(1)
    try:
        one = _timed_oracle_steps(run_step, target_seconds / 3, 100000)
    finally:
        oracle.set_threads(threads)
    return _baseline_record(w, bs, ctx, steps, nbytes, t_total, threads, one,
                            f", {T} query tokens per step" if T > 1 else "", T)


def cpu_baseline_bq2(w, target_seconds: float):
    """The oracle of the rotated format on a bounded sample: the first few
    sequences, decode steps (append + attention) from the workload's context,
    for about target_seconds on all host threads, then about a third of that
    on one thread.  Every 1024 steps the lengths start again from the
    context."""
    import oracle
    from quantized_decode_attention_amd import metrics, synth

    bs = min(w.batch, 2)
    n0 = w.context - 1
    og = oracle.Bq2Geom(bs, w.n_q_heads, w.n_kv_heads, synth.capacity_for(w, 2048))
    oc = oracle.Bq2Cache(og)
    oracle.bq2_prefill(og, oc, synth.keys(w, n0, batch=bs), synth.values(w, n0, batch=bs), n0)
    scale = 1.0 / math.sqrt(w.head_dim)
    lens = np.full(bs, n0, np.int32)

    def run_step(i):
        if i % 1024 == 0:
            lens[:] = n0
        kn, vn, q = synth.step_token(w, i, batch=bs)
        oracle.bq2_append(og, oc, kn, vn, lens)
        lens[:] += 1
        oracle.bq2_decode_attn(og, oc, q, lens, scale)
        return (metrics.bq2_decode_step_bytes(lens, w.n_q_heads, w.n_kv_heads)
                + metrics.bq2_append_bytes(bs, w.n_kv_heads))

    threads = oracle.max_threads()
    steps, nbytes, t_total = _timed_oracle_steps(run_step, target_seconds, 100000)
    oracle.set_threads(1)
    try:
        one = _timed_oracle_steps(run_step, target_seconds / 3, 100000)
    finally:
        oracle.set_threads(threads)
    return _baseline_record(w, bs, w.context, steps, nbytes, t_total, threads, one)


ROTATION_BYTES = 1e9  # decode bytes kept in rotation: four times the Infinity Cache


def rotating_layers(a, step_bytes: float) -> int:
    """--layers, or enough layer caches that one pass over them reads at least
    ROTATION_BYTES (4 to 16)."""
    if a.layers:
        return a.layers
    return int(min(16, max(4, math.ceil(ROTATION_BYTES / step_bytes))))


def stream_ceiling(kvq) -> dict:
    """The read rate of the stream probe in the shape that reads fastest (one
    wave per SIMD, four nontemporal 16-byte loads per lane in flight, two
    batches deep): the practical ceiling of a read-only stream."""
    r = kvq.stream_read_sweep([(1, 4, 1)], reps=20)[0]
    return {"gbs": r["gbs"], "median_us": r["median_us"], "bytes": 2 << 30,
            "kernel": "kvq_probe_stream_read_sweep (1 wave per SIMD, 4 nontemporal 16-byte "
                      "loads per lane in flight, 2 GiB buffer beyond the Infinity Cache)"}


def steady_and_flush_lengths(base: np.ndarray, T: int, R: int):
    """Lengths before the first append of the two kinds of decode step at the
    workload's contexts `base` (current tokens included).

    A steady step appends its T tokens inside the fp16 window and attends over
    base (moved down by at most T where that append would fill a window); a
    flush step's first token finds its window full, so the step flushes R
    tokens into packed rows, then attends over the next multiple of R plus T.
    A cache prefilled to the flush length holds both states: a sequence of n
    tokens with n mod R in [1, R - T] has the same packed rows as one of the
    next multiple of R."""
    n_s = base.astype(np.int64) - T
    r = n_s % R
    n_s = np.where(r == 0, n_s - T, np.where(r > R - T, n_s - (r - (R - T)), n_s))
    n_s = np.maximum(n_s, 1)
    n_f = -(-n_s // R) * R
    assert np.all((n_s % R >= 1) & (n_s % R <= R - T)) and np.all(n_f - n_s >= T)
    return n_s.astype(np.int32), n_f.astype(np.int32)


def replay_per_step(graph, K: int, torch, min_seconds: float, min_reps: int = 10,
                    max_reps: int = 2000):
    """Seconds per step of a captured K-step graph: one untimed replay, then
    replays each bracketed by torch.cuda.synchronize() and timed on the host
    clock (HIP events on the replay stream beside it), until min_reps and
    min_seconds are reached.  Returns (host, events) arrays, one per replay."""
    stream = torch.cuda.current_stream()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    host, gpu = [], []
    while len(host) < max_reps and (len(host) < min_reps or sum(host) * K < min_seconds):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        host.append((time.perf_counter() - t0) / K)
        gpu.append(e0.elapsed_time(e1) / 1e3 / K)
    return np.array(host), np.array(gpu)


def eager_per_step(step, K: int, passes: int, torch):
    """The K steps launched one by one, `passes` times, with HIP events around
    the dominant kernel of every step (step(i, (ev_a, ev_b)) records them on
    the launch stream).  Returns (seconds per step of each pass, kernel
    milliseconds of every launch)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(passes * K)]
    per_step = []
    for p in range(passes):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(i, evs[p * K + i])
        torch.cuda.synchronize()
        per_step.append((time.perf_counter() - t0) / K)
    return np.array(per_step), np.array([a.elapsed_time(b) for a, b in evs])


def measure(a, step, torch, label: str, kernel=None):
    """Warmup, eager passes with per-launch kernel events, then (unless
    --eager) the K steps captured as one HIP graph and replayed.  Every step
    of a kind does the same work at the same lengths, so passes and replays
    repeat it exactly.  kernel(i), if given, launches only step i's dominant
    kernel: K of them are captured as a graph of their own and replayed, so
    that its average launch is timed as it runs inside the step graph (back to
    back, HIP events around each replay) rather than launched one by one."""
    K = a.steps
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    passes = max(2, -(-a.eager_launches // K))
    eager, kern_ms = eager_per_step(step, K, passes, torch)
    print(f"[bench] {label}: {passes} eager passes of {K} steps, "
          f"{np.median(eager) * 1e6:.2f} us per step", file=sys.stderr, flush=True)
    res = {"eager_s": float(np.median(eager)), "kernel_ms": kern_ms, "passes": passes}
    if a.eager:
        res["step_s"] = res["eager_s"]
        res["replays"] = 0
        return res
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(K):
            step(i)
    host, gpu = replay_per_step(graph, K, torch, a.min_seconds)
    del graph
    res.update(step_s=float(np.median(host)), step_events_s=float(np.median(gpu)),
               replays=len(host), replay_spread=float(np.percentile(host, 90) /
                                                      np.percentile(host, 10)))
    print(f"[bench] {label}: {len(host)} graph replays of {K} steps, "
          f"{res['step_s'] * 1e6:.2f} us per step", file=sys.stderr, flush=True)
    if kernel is not None:
        kg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(kg):
            for i in range(K):
                kernel(i)
        _, kgpu = replay_per_step(kg, K, torch, a.min_seconds)
        del kg
        res.update(kernel_graph_s=float(np.median(kgpu)), kernel_replays=len(kgpu))
        print(f"[bench] {label}: {len(kgpu)} replays of {K} back-to-back kernel launches, "
              f"{res['kernel_graph_s'] * 1e6:.2f} us per launch", file=sys.stderr, flush=True)
    return res


def kernel_roofline(kernel: str, m: dict, dec_bytes: float, traffic, ceiling: dict):
    """The dominant kernel against the HBM roofline: its algorithmic bytes per
    launch over its average launch as timed in a graph of back-to-back launches
    (or, with --eager, over the per-launch events of the eager passes)."""
    kern_ms = m["kernel_ms"]
    eager_avg_s = float(np.mean(kern_ms)) / 1e3
    avg_s = m.get("kernel_graph_s", eager_avg_s)
    achieved = dec_bytes / avg_s / 1e9
    return {
        "kernel": kernel,
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": traffic,
        "avg_launch_us": round(avg_s * 1e6, 3),
        "launch_timing": ("HIP events around replays of a graph of back-to-back launches "
                          "(median replay / launches)" if "kernel_graph_s" in m else
                          "HIP events around each eager launch"),
        "eager_launches": {
            "avg_us": round(eager_avg_s * 1e6, 3), "launches": int(len(kern_ms)),
            **{f"p{q}_us": round(float(np.percentile(kern_ms, q)) * 1e3, 3)
               for q in (10, 50, 90)}},
        "algorithmic_bytes_per_launch": round(dec_bytes),
        "frac_of_stream_read": round(achieved / ceiling["gbs"], 4),
    }


DTYPE = "f16 mfma, f32 accumulate"
DTYPE_NOTE = ("codes enter v_mfma_f32_16x16x32_f16 as exact fp16 operands against fp16 "
              "hi + lo splits of the fp32 factors (q times the key scale, the softmax "
              "weight times the value scale; about 2^-21 relative); products, sums, "
              "softmax and the split combine in fp32; fp16 out")


def run_bq2(a, w, torch, kvq, metrics, synth):
    """The rotated per-token 2-bit format: kvq_bq2_append then
    kvq_bq2_decode_partial (timed per launch) and kvq_bq2_decode_combine, every
    step appending at position context - 1 and attending over the context
    (the format has no window to flush)."""
    dev = torch.device("cuda:0")
    L = rotating_layers(a, metrics.bq2_decode_step_bytes(np.full(w.batch, w.context),
                                                         w.n_q_heads, w.n_kv_heads))
    cap = synth.capacity_for(w, 1)
    g = kvq.Bq2Geom(w.batch, w.n_q_heads, w.n_kv_heads, cap)
    n0 = w.context - 1
    print(f"[bench] workload {w.name}: {L} layer caches, capacity {cap}, steps append at "
          f"{n0} and attend over {w.context}", file=sys.stderr, flush=True)
    caches = [kvq.Bq2Cache(g, dev) for _ in range(L)]
    kd = torch.from_numpy(synth.keys(w, n0)).to(dev)
    vd = torch.from_numpy(synth.values(w, n0)).to(dev)
    for c in caches:
        kvq.kvq_bq2_prefill(g, kd, vd, n0, c)
    del kd, vd
    torch.cuda.synchronize()
    pool = [tuple(torch.from_numpy(x).to(dev) for x in synth.step_token(w, s)) for s in range(8)]
    before = torch.full((w.batch,), n0, dtype=torch.int32, device=dev)
    after = before + 1
    max_len = w.context
    ws = kvq.alloc_bq2_workspace(g, max_len, dev)
    out = torch.empty((w.batch, w.n_q_heads, 64), dtype=torch.float16, device=dev)
    scale = 1.0 / math.sqrt(w.head_dim)
    n_workers = kvq.kvq_bq2_decode_workers(g)
    dec_bytes = metrics.bq2_decode_step_bytes(np.full(w.batch, w.context), w.n_q_heads,
                                              w.n_kv_heads)
    step_bytes = dec_bytes + metrics.bq2_append_bytes(w.batch, w.n_kv_heads)

    def step(i, ev=None):
        stream = torch.cuda.current_stream()  # the capture stream inside a graph capture
        kn, vn, q = pool[i % len(pool)]
        c = caches[i % L]
        kvq.kvq_bq2_append(g, kn, vn, before, c, stream)
        if ev is not None:
            ev[0].record(stream)
        kvq.kvq_bq2_decode_partial(g, q, c, after, max_len, scale, ws, out, stream)
        if ev is not None:
            ev[1].record(stream)
        kvq.kvq_bq2_decode_combine(g, q, c, after, max_len, scale, ws, out, stream)

    def kernel(i):
        kvq.kvq_bq2_decode_partial(g, pool[i % len(pool)][2], caches[i % L], after, max_len,
                                   scale, ws, out, torch.cuda.current_stream())

    m = measure(a, step, torch, "steady steps", kernel)
    ceiling = stream_ceiling(kvq)
    t = m["step_s"]
    gbs = step_bytes / t / 1e9
    return {
        "metric": "quantized-KV decode attention: effective HBM GB/s (% of peak) + tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(t * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "dtype_note": DTYPE_NOTE,
        "data": "synthetic (seeded; keys with per-channel lognormal scales and outlier "
                "channels before rotation, values and queries N(0,1), fp16)",
        "config": {
            "workload": w.name,
            "format": "rotated per-token 2-bit (KV1 BQ2_0), 4 fp16 sinks",
            "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "context": w.context,
            "rotating_layer_caches": L, "decode_worker_waves": n_workers,
            "step": "kvq_bq2_append + kvq_bq2_decode_attn, one layer",
            "launch": ("kernels launched one by one" if a.eager else
                       "the K timed steps captured as one HIP graph; value from the median "
                       "of its replays"),
            "graph_replays": m["replays"],
        },
        "eager": {"value": round(step_bytes / m["eager_s"] / 1e9, 2), "unit": "GB/s",
                  "ms_per_step": round(m["eager_s"] * 1e3, 5)},
        **({"events_ms_per_step": round(m["step_events_s"] * 1e3, 5),
            "replay_p90_over_p10": round(m["replay_spread"], 4)} if not a.eager else {}),
        "bytes_per_step": round(step_bytes),
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(w.batch / t, 1),
        "tokens_per_s_unit": "decoded tokens per second through one layer",
        "roofline": kernel_roofline("bq2_partial", m, dec_bytes,
                                    load_traffic(w.name, "bq2_partial"), ceiling),
        "stream_read": ceiling,
        "gpu": torch.cuda.get_device_name(0),
    }


def run_kivi(a, w, torch, kvq, metrics, synth):
    """The KIVI format: steady steps and flush steps (see
    steady_and_flush_lengths) timed apart, the flush amortized at one step in
    R / T per layer cache, as a decode loop at these contexts sees it."""
    dev = torch.device("cuda:0")
    T, R = a.tokens, w.residual
    L = w.layers if w.layers > 1 else rotating_layers(
        a, metrics.decode_step_bytes(synth.seq_lens(w), w.n_q_heads, w.n_kv_heads, w.head_dim,
                                     w.k_bits, w.v_bits, w.group, R))
    if T >= R:
        raise SystemExit(f"--tokens must be below the window ({R})")
    base = synth.seq_lens(w)
    n_s, n_f = steady_and_flush_lengths(base, T, R)
    cap = synth.capacity_for(w, R + T)
    g = kvq.Geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                 w.group, R, cap)
    print(f"[bench] workload {w.name}: {L} layer caches, capacity {cap}, steady steps "
          f"attend over {int((n_s + T).min())}..{int((n_s + T).max())}, flush steps over "
          f"{int((n_f + T).min())}..{int((n_f + T).max())}", file=sys.stderr, flush=True)
    P = a.page_size
    if P:
        # every layer's pool: B * ceil(cap / P) pages, each sequence's pages
        # drawn in shuffled order
        maxp = -(-cap // P)
        prng = np.random.default_rng(7)
        caches = []
        for _ in range(L):
            table = prng.permutation(w.batch * maxp).astype(np.int32).reshape(w.batch, maxp)
            caches.append(kvq.PagedCache(g, P, w.batch * maxp, torch.from_numpy(table).to(dev),
                                         dev))
        prefill, append = kvq.kvq_paged_prefill, kvq.kvq_paged_append
        append_tokens = kvq.kvq_paged_append_tokens
        partial, combine = kvq.kvq_paged_decode_partial, kvq.kvq_paged_decode_combine
        multi = kvq.kvq_paged_decode_attn_multi
    else:
        caches = [kvq.Cache(g, dev) for _ in range(L)]
        prefill, append = kvq.kvq_prefill, kvq.kvq_append
        append_tokens = kvq.kvq_append_tokens
        partial, combine = kvq.kvq_decode_partial, kvq.kvq_decode_combine
        multi = kvq.kvq_decode_attn_multi
    # prefill every layer to the flush lengths from the same seeded tensors
    nmax = int(n_f.max())
    kd = torch.from_numpy(synth.keys(w, nmax)).to(dev)
    vd = torch.from_numpy(synth.values(w, nmax)).to(dev)
    for c in caches:
        if np.all(n_f == n_f[0]):
            n = int(n_f[0])
            prefill(g, kd[:, :, :n].contiguous(), vd[:, :, :n].contiguous(), n, c)
        else:
            for b in range(w.batch):
                n = int(n_f[b])
                sub = c.view(b, b + 1)
                prefill(sub.g, kd[b:b + 1, :, :n].contiguous(),
                        vd[b:b + 1, :, :n].contiguous(), n, sub)
    del kd, vd
    torch.cuda.synchronize()

    # per-step inputs (a pool of seeded tokens) and lengths, all on device
    pool = [tuple(torch.from_numpy(x).to(dev) for x in synth.step_token(w, s)) for s in range(8)]
    if T > 1:  # the T new tokens (and queries) of pool slot s: entries s .. s + T - 1
        tpool = [(torch.stack([pool[(s + j) % len(pool)][0] for j in range(T)], 1).contiguous(),
                  torch.stack([pool[(s + j) % len(pool)][1] for j in range(T)], 1).contiguous(),
                  torch.stack([pool[(s + j) % len(pool)][2] for j in range(T)], 1).contiguous())
                 for s in range(len(pool))]
    lens = {kind: (torch.from_numpy(n).to(dev), torch.from_numpy(n + T).to(dev),
                   int((n + T).max()))
            for kind, n in (("steady", n_s), ("flush", n_f))}
    max_len = lens["flush"][2]
    if P:
        ws = kvq.alloc_paged_workspace(g, T, max_len, dev)
    elif T == 1:
        ws = kvq.alloc_workspace(g, max_len, dev)
    else:
        ws = kvq.alloc_multi_workspace(g, T, max_len, dev)
    oshape = (w.batch, w.n_q_heads, w.head_dim) if T == 1 else \
        (w.batch, T, w.n_q_heads, w.head_dim)
    out = torch.empty(oshape, dtype=torch.float16, device=dev)
    scale = 1.0 / math.sqrt(w.head_dim)
    n_workers = (ws.numel() * 4 // (T * (w.n_q_heads // w.n_kv_heads) * (w.head_dim + 4) * 4)
                 - w.batch * w.n_kv_heads)

    def make_step(kind):
        before, after, msl = lens[kind]

        def step(i, ev=None):
            stream = torch.cuda.current_stream()  # the capture stream inside a graph capture
            c = caches[i % L]
            if T == 1:
                kn, vn, q = pool[i % len(pool)]
                append(g, kn, vn, before, c, stream)
            else:  # the T new tokens in one launch
                kn, vn, q = tpool[i % len(tpool)]
                append_tokens(g, T, kn, vn, before, c, stream)
            if ev is not None:
                ev[0].record(stream)
            if T == 1:
                partial(g, q, c, after, msl, scale, ws, out, stream)
                if ev is not None:
                    ev[1].record(stream)
                combine(g, q, c, after, msl, scale, ws, out, stream)
            else:  # partial + combine in one call: the events bracket both
                multi(g, q, c, after, T, msl, scale, ws, out, stream)
                if ev is not None:
                    ev[1].record(stream)
        return step

    def kernel(i):  # the steady step's dominant kernel alone
        before, after, msl = lens["steady"]
        stream = torch.cuda.current_stream()
        c = caches[i % L]
        if T == 1:
            partial(g, pool[i % len(pool)][2], c, after, msl, scale, ws, out, stream)
        else:
            multi(g, tpool[i % len(tpool)][2], c, after, T, msl, scale, ws, out, stream)

    def step_bytes(n_before, flushing):
        after = n_before + T
        db = metrics.decode_step_bytes(after, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                       w.k_bits, w.v_bits, w.group, R)
        db += (T - 1) * 4 * w.batch * w.n_q_heads * w.head_dim  # the other tokens' q and out
        sb = db + T * metrics.append_bytes(w.batch, w.n_kv_heads, w.head_dim)
        if flushing:
            sb += metrics.flush_bytes(w.batch * w.n_kv_heads, R, w.head_dim, w.k_bits,
                                      w.v_bits, w.group)
        return db, sb

    dec_s, b_s = step_bytes(n_s, False)
    dec_f, b_f = step_bytes(n_f, True)
    ms = measure(a, make_step("steady"), torch, "steady steps", kernel)
    mf = measure(a, make_step("flush"), torch, "flush steps")
    F = R / T  # steps per layer cache between its flushes
    t = ((F - 1) * ms["step_s"] + mf["step_s"]) / F
    nbytes = ((F - 1) * b_s + b_f) / F
    t_eager = ((F - 1) * ms["eager_s"] + mf["eager_s"]) / F
    gbs = nbytes / t / 1e9
    ceiling = stream_ceiling(kvq)
    traffic = load_traffic(w.name) if T == 1 and not P else None

    def kind_entry(m, b, n_before, flushes):
        e = {"ms_per_step": round(m["step_s"] * 1e3, 5),
             "value": round(b / m["step_s"] / 1e9, 2), "unit": "GB/s",
             "bytes_per_step": round(b),
             "context": [int((n_before + T).min()), int((n_before + T).max())],
             "flushes_per_step": flushes,
             "eager_ms_per_step": round(m["eager_s"] * 1e3, 5)}
        if not a.eager:
            e.update(graph_replays=m["replays"],
                     events_ms_per_step=round(m["step_events_s"] * 1e3, 5),
                     replay_p90_over_p10=round(m["replay_spread"], 4))
        return e

    rec = {
        "metric": "quantized-KV decode attention: effective HBM GB/s (% of peak) + tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(t * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "dtype_note": DTYPE_NOTE,
        "data": "synthetic (seeded; keys with per-channel lognormal scales and outlier "
                "channels, values and queries N(0,1), fp16)",
        "config": {
            "workload": w.name,
            "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "k_bits": w.k_bits, "v_bits": w.v_bits,
            "group": w.group, "residual": R,
            "context": ([int(base.min()), int(base.max())] if w.ctx_range else int(w.context)),
            "rotating_layer_caches": L, "decode_worker_waves": n_workers,
            "step": ("kvq_append (+flush when a window fills) + kvq_decode_attn, one layer"
                     if T == 1 else
                     f"kvq_append_tokens (T={T}) + kvq_decode_attn_multi, one layer"),
            "query_tokens": T,
            "flush_every_steps": F,
            "cache": f"paged, {P}-position pages in shuffled order" if P else "dense",
            "launch": ("kernels launched one by one" if a.eager else
                       "the K timed steps captured as one HIP graph; value from the median "
                       "of its replays"),
            "amortized": (f"value = bytes / time of {F - 1:g} steady steps and 1 flush step, "
                          f"each timed apart"),
        },
        "steady_step": kind_entry(ms, b_s, n_s, 0),
        "flush_step": kind_entry(mf, b_f, n_f, w.batch * w.n_kv_heads),
        "eager": {"value": round(nbytes / t_eager / 1e9, 2), "unit": "GB/s",
                  "ms_per_step": round(t_eager * 1e3, 5)},
        "bytes_per_step": round(nbytes),
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(w.batch * T / t, 1),
        "tokens_per_s_unit": "decoded tokens per second through one layer",
        **({"stack_tokens_per_s": round(w.batch * T / L / t, 1),
            "stack_tokens_per_s_unit": f"decoded tokens per second through all {L} layers"}
           if w.layers > 1 else {}),
        "roofline": kernel_roofline(
            ("decode_partial" if T == 1 else "decode_partial+decode_combine (multi)")
            + (" (paged)" if P else ""), ms, dec_s, traffic, ceiling),
        "stream_read": ceiling,
        "gpu": torch.cuda.get_device_name(0),
    }
    return rec


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the decode "
                          "path has no multi-GPU part (--gpus must be 1)"}))
        sys.exit(2)
    import torch

    import quantized_decode_attention_amd as kvq
    from quantized_decode_attention_amd import metrics, synth

    if a.calib_copy_mib:
        n = a.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4}))
        return

    if a.probe_sweep:
        shapes = [(wps, loads, nt) for nt in (0, 1, 2, 3) for wps in (1, 2, 3, 4, 8)
                  for loads in (1, 2, 4, 8, 16) if not (loads == 16 and wps > 3)]
        res = kvq.stream_read_sweep(shapes)
        best = max(res, key=lambda r: r["gbs"])
        print(json.dumps({"probe": "kvq_probe_stream_read_sweep, 2 GiB buffer",
                          "best": best, "default_probe": kvq.stream_read_gbs(),
                          "sweep": res}), flush=True)
        return

    w = synth.WORKLOADS[a.config]
    torch.cuda.set_device(torch.device("cuda:0"))
    if a.probe_chunks:
        if w.fmt != "kivi":
            print(json.dumps({"error": "--probe-chunks takes a KIVI-format workload"}))
            sys.exit(2)
        # a packed 32-token chunk's pieces, as the partial kernel loads them: key
        # codes, value codes, value meta, and the key group's meta (a chunk's share)
        D, ng = w.head_dim, w.head_dim // w.group
        pieces = [32 * D * w.k_bits // 8, 32 * D * w.v_bits // 8, 32 * ng * 4,
                  D * 4 * 32 // w.group]
        pieces = [max(512, (b + 511) // 512 * 512) for b in pieces]
        n_chunks = w.batch * w.n_kv_heads * w.context // 32
        res = kvq.chunk_stream(pieces, n_chunks, [0, 16, 32, 64, 96, 128, 192])
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        for r in res:
            r["us_per_chunk_and_wave"] = round(r["median_us"] * 2 * 4 * cus / n_chunks, 3)
        print(json.dumps({"probe": "kvq_probe_chunk_stream", "workload": w.name,
                          "piece_bytes": pieces, "n_chunks": n_chunks,
                          "waves": 2 * 4 * cus, "rows": res}), flush=True)
        return
    if w.fmt == "bq2":
        rec = run_bq2(a, w, torch, kvq, metrics, synth)
    else:
        rec = run_kivi(a, w, torch, kvq, metrics, synth)
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        if w.fmt == "bq2":
            rec["cpu_baseline"] = cpu_baseline_bq2(w, a.cpu_seconds)
        else:
            rec["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds, a.tokens)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
