#!/usr/bin/env python3
"""Decode-step benchmark of libkvq on one MI355X.

A step is one pass of the whole decode hot path for one attention layer over a
batch of sequences: kvq_append (the new token; a residual flush when a window
is full) then kvq_decode_attn (split partials + combine).  Steps rotate over
--layers independent layer caches (default 4, about 1.1 GB for the default
workload) so the 256 MB Infinity Cache cannot serve a layer's packed cache from
one step to the next: the bytes come from HBM, as in a real multi-layer model.

Default workload: the Llama-3-8B-shaped GQA layer (32 query / 8 KV heads,
head_dim 128, batch 32, context 8192, 2-bit keys / 4-bit values, G = 32,
R = 128).  512 steps = 128 tokens per layer, so every layer does exactly one
residual flush inside the timed region.  --config 6 runs the KV1-shaped layer
in the rotated per-token 2-bit format (kvq_bq2_append + kvq_bq2_decode_attn,
batch 16, context 32768).

Prints one JSON line: effective HBM GB/s of the whole step (algorithmic bytes /
time), tokens/s, the roofline of the dominant kernel (decode partial: HIP
events around each launch on the launch stream) and the CPU oracle timed on a
bounded sample of the same workload on the host cores.
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
    p.add_argument("--steps", type=int, default=512)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--config", type=int, default=3, help="workload 1..6 (default 3)")
    p.add_argument("--layers", type=int, default=4, help="rotating layer caches")
    p.add_argument("--tokens", type=int, default=1,
                   help="query tokens per sequence per step (T > 1: kvq_append_tokens, then "
                        "kvq_decode_attn_multi; KIVI-format workloads)")
    p.add_argument("--page-size", type=int, default=0,
                   help="KIVI workloads: a paged cache with pages of this many positions, "
                        "handed out in shuffled order (0: the dense cache)")
    p.add_argument("--eager", action="store_true",
                   help="time the steps as launched one by one (default: the timed steps "
                        "are also captured as one HIP graph, and value is its replay)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
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


def cpu_baseline(w, target_seconds: float):
    """The oracle, as it stands, on a bounded sample of the workload: the first
    few sequences of the batch, one decode step (append + attention) repeated
    until about target_seconds have passed."""
    import oracle
    from quantized_decode_attention_amd import metrics, synth

    bs = min(w.batch, 4)
    n0 = w.context - 1
    cap = synth.capacity_for(w, 64)
    og = oracle.Geom(bs, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                     w.group, w.residual, cap)
    k = synth.keys(w, n0, batch=bs)
    v = synth.values(w, n0, batch=bs)
    oc = oracle.Cache(og)
    oracle.prefill(og, oc, k, v, n0)
    del k, v
    scale = 1.0 / math.sqrt(w.head_dim)
    steps, nbytes, t_total = 0, 0.0, 0.0
    lens = np.full(bs, n0, np.int32)
    while t_total < target_seconds and steps < 256:
        kn, vn, q = synth.step_token(w, steps, batch=bs)
        t0 = time.perf_counter()
        oracle.append(og, oc, kn, vn, lens)
        _ = oracle.decode_attn(og, oc, q, lens + 1, scale)
        t_total += time.perf_counter() - t0
        nbytes += metrics.decode_step_bytes(lens + 1, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                            w.k_bits, w.v_bits, w.group, w.residual)
        nbytes += metrics.append_bytes(bs, w.n_kv_heads, w.head_dim)
        lens += 1
        steps += 1
    return {
        "value": round(nbytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(bs * steps / t_total, 3),
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": (f"{bs} of {w.batch} sequences at context {w.context}, {steps} decode "
                   f"steps (append + attention), {t_total:.1f} s"),
    }


def cpu_baseline_bq2(w, target_seconds: float):
    """The oracle of the rotated format on a bounded sample: the first few
    sequences, one decode step (append + attention) repeated until about
    target_seconds have passed."""
    import oracle
    from quantized_decode_attention_amd import metrics, synth

    bs = min(w.batch, 2)
    n0 = w.context - 1
    og = oracle.Bq2Geom(bs, w.n_q_heads, w.n_kv_heads, synth.capacity_for(w, 64))
    oc = oracle.Bq2Cache(og)
    oracle.bq2_prefill(og, oc, synth.keys(w, n0, batch=bs), synth.values(w, n0, batch=bs), n0)
    scale = 1.0 / math.sqrt(w.head_dim)
    steps, nbytes, t_total = 0, 0.0, 0.0
    lens = np.full(bs, n0, np.int32)
    while t_total < target_seconds and steps < 1024:
        kn, vn, q = synth.step_token(w, steps, batch=bs)
        t0 = time.perf_counter()
        oracle.bq2_append(og, oc, kn, vn, lens)
        _ = oracle.bq2_decode_attn(og, oc, q, lens + 1, scale)
        t_total += time.perf_counter() - t0
        nbytes += metrics.bq2_decode_step_bytes(lens + 1, w.n_q_heads, w.n_kv_heads)
        nbytes += metrics.bq2_append_bytes(bs, w.n_kv_heads)
        lens += 1
        steps += 1
    return {
        "value": round(nbytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(bs * steps / t_total, 3),
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": (f"{bs} of {w.batch} sequences at context {w.context}, {steps} decode "
                   f"steps (append + attention), {t_total:.1f} s"),
    }


def time_steps(a, step, torch):
    """Times the K steps after the warmup: first launched one by one with the
    decode-partial events (step(s, i) records them), then, unless --eager, the
    same K steps captured as one HIP graph (a serving loop's launch form) and
    replayed: one untimed replay, then the timed one.  Each pass appends the
    same tokens at the same positions: the same work on the same sizes.
    Returns (eager seconds, seconds of the run that gives value)."""
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(a.warmup + i, i)
    torch.cuda.synchronize()
    eager = time.perf_counter() - t0
    if a.eager:
        return eager, eager
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(a.steps):
            step(a.warmup + i)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    return eager, time.perf_counter() - t0


def run_bq2(a, w, torch, kvq, metrics, synth):
    """The rotated per-token 2-bit format: kvq_bq2_append then
    kvq_bq2_decode_partial (timed per launch) and kvq_bq2_decode_combine."""
    dev = torch.device("cuda:0")
    L = a.layers
    total_steps = a.warmup + a.steps
    per_layer_tokens = -(-total_steps // L)
    cap = synth.capacity_for(w, per_layer_tokens + 1)
    g = kvq.Bq2Geom(w.batch, w.n_q_heads, w.n_kv_heads, cap)
    start = np.full(w.batch, w.context - 1 - (a.warmup + L - 1) // L, np.int32)
    n0 = int(start[0])
    print(f"[bench] workload {w.name}: {L} layer caches, capacity {cap}, start len {n0}",
          file=sys.stderr, flush=True)
    caches = [kvq.Bq2Cache(g, dev) for _ in range(L)]
    kd = torch.from_numpy(synth.keys(w, n0)).to(dev)
    vd = torch.from_numpy(synth.values(w, n0)).to(dev)
    for c in caches:
        kvq.kvq_bq2_prefill(g, kd, vd, n0, c)
    del kd, vd
    torch.cuda.synchronize()
    pool = [tuple(torch.from_numpy(x).to(dev) for x in synth.step_token(w, s)) for s in range(8)]
    lens_host = np.zeros((total_steps, 2, w.batch), np.int32)
    cur = [start.copy() for _ in range(L)]
    for s in range(total_steps):
        l = s % L
        lens_host[s, 0] = cur[l]
        lens_host[s, 1] = cur[l] + 1
        cur[l] = cur[l] + 1
    lens_dev = torch.from_numpy(lens_host).to(dev)
    max_len = int(lens_host[:, 1].max())
    ws = kvq.alloc_bq2_workspace(g, max_len, dev)
    out = torch.empty((w.batch, w.n_q_heads, 64), dtype=torch.float16, device=dev)
    scale = 1.0 / math.sqrt(w.head_dim)
    n_workers = kvq.kvq_bq2_decode_workers(g)
    dec_bytes = [metrics.bq2_decode_step_bytes(lens_host[s, 1], w.n_q_heads, w.n_kv_heads)
                 for s in range(total_steps)]
    step_bytes = [d + metrics.bq2_append_bytes(w.batch, w.n_kv_heads) for d in dec_bytes]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]

    def step(s, timed_idx=None):
        stream = torch.cuda.current_stream()  # the capture stream inside a graph capture
        kn, vn, q = pool[s % len(pool)]
        c = caches[s % L]
        kvq.kvq_bq2_append(g, kn, vn, lens_dev[s, 0], c, stream)
        if timed_idx is not None:
            ev_a[timed_idx].record(stream)
        kvq.kvq_bq2_decode_partial(g, q, c, lens_dev[s, 1], max_len, scale, ws, out, stream)
        if timed_idx is not None:
            ev_b[timed_idx].record(stream)
        kvq.kvq_bq2_decode_combine(g, q, c, lens_dev[s, 1], max_len, scale, ws, out, stream)

    for s in range(a.warmup):
        step(s)
    torch.cuda.synchronize()
    elapsed_eager, elapsed = time_steps(a, step, torch)
    timed = slice(a.warmup, a.warmup + a.steps)
    gbs = float(np.sum(step_bytes[timed])) / elapsed / 1e9
    gbs_eager = float(np.sum(step_bytes[timed])) / elapsed_eager / 1e9
    part_ms = np.array([ev_a[i].elapsed_time(ev_b[i]) for i in range(a.steps)])
    part_avg_s = float(np.mean(part_ms)) / 1e3
    part_pct = {f"p{q}_us": round(float(np.percentile(part_ms, q)) * 1e3, 3) for q in (10, 50, 90)}
    dec_avg_bytes = float(np.mean(dec_bytes[timed]))
    achieved = dec_avg_bytes / part_avg_s / 1e9
    ceiling = kvq.stream_read_gbs()
    return {
        "metric": "quantized-KV decode attention: effective HBM GB/s (% of peak) + tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(elapsed / a.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; keys with per-channel lognormal scales and outlier "
                "channels before rotation, values and queries N(0,1), fp16)",
        "config": {
            "workload": w.name,
            "format": "rotated per-token 2-bit (KV1 BQ2_0), 4 fp16 sinks",
            "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim,
            "context_first_step": int(lens_host[a.warmup, 1].max()),
            "context_last_step": int(lens_host[-1, 1].max()),
            "rotating_layer_caches": L, "decode_worker_waves": n_workers,
            "step": "kvq_bq2_append + kvq_bq2_decode_attn, one layer",
            "launch": ("kernels launched one by one" if a.eager else
                       "the timed steps replayed as one HIP graph"),
        },
        "eager": {"value": round(gbs_eager, 2), "unit": "GB/s",
                  "ms_per_step": round(elapsed_eager / a.steps * 1e3, 5),
                  "tokens_per_s": round(w.batch * a.steps / elapsed_eager, 1)},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(w.batch * a.steps / elapsed, 1),
        "tokens_per_s_unit": "decoded tokens per second through one layer",
        "roofline": {
            "kernel": "bq2_partial",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(w.name, "bq2_partial"),
            "avg_launch_us": round(part_avg_s * 1e6, 3),
            **part_pct,
            "algorithmic_bytes_per_launch": round(dec_avg_bytes),
            "frac_of_stream_read": round(achieved / ceiling["gbs"], 4),
        },
        "stream_read": {**ceiling, "kernel": "kvq_probe_stream_read (plain 16-byte loads, "
                                              "2 GiB buffer beyond the Infinity Cache)"},
        "gpu": torch.cuda.get_device_name(0),
    }


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

    w = synth.WORKLOADS[a.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.fmt == "bq2":
        rec = run_bq2(a, w, torch, kvq, metrics, synth)
        if not a.no_cpu_baseline:
            print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
            rec["cpu_baseline"] = cpu_baseline_bq2(w, a.cpu_seconds)
        print(json.dumps(rec), flush=True)
        return
    L = a.layers if w.layers == 1 else w.layers
    T = a.tokens
    total_steps = a.warmup + a.steps
    per_layer_tokens = -(-total_steps // L) * T
    cap = synth.capacity_for(w, per_layer_tokens + T)
    g = kvq.Geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                 w.group, w.residual, cap)

    # sequence lengths before the first warmup step: the first timed step of
    # each layer attends over the workload's context
    base = synth.seq_lens(w)
    if w.ctx_range is None:
        start = base - T - T * ((a.warmup + L - 1) // L)
        if w.cfg == 5:
            start = np.full(w.batch, w.context, np.int32)
    else:
        start = base - T
    start = np.maximum(start, 1).astype(np.int32)
    nmax0 = int(start.max())

    print(f"[bench] workload {w.name}: {L} layer caches, capacity {cap}, "
          f"start len {int(start.min())}..{nmax0}", file=sys.stderr, flush=True)
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
    # prefill every layer from the same seeded tensors (layer 0's draw)
    k = synth.keys(w, nmax0)
    v = synth.values(w, nmax0)
    kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    del k, v
    for c in caches:
        if np.all(start == start[0]):
            n = int(start[0])
            prefill(g, kd[:, :, :n].contiguous(), vd[:, :, :n].contiguous(), n, c)
        else:
            for b in range(w.batch):
                n = int(start[b])
                sub = c.view(b, b + 1)
                prefill(sub.g, kd[b:b + 1, :, :n].contiguous(),
                        vd[b:b + 1, :, :n].contiguous(), n, sub)
    del kd, vd
    torch.cuda.synchronize()

    # per-step inputs (a pool of seeded tokens) and lengths, all on device
    pool = [tuple(torch.from_numpy(x).to(dev) for x in synth.step_token(w, s)) for s in range(8)]
    # T > 1: the T new tokens of step s as [B][T][Hkv][D] (pool entries s .. s + T - 1)
    tpool = [(torch.stack([pool[(s + j) % len(pool)][0] for j in range(T)], 1).contiguous(),
              torch.stack([pool[(s + j) % len(pool)][1] for j in range(T)], 1).contiguous())
             for s in range(len(pool))] if T > 1 else None
    # lens_host[s, j]: length before append j of step s (j < T); [s, T]: after
    lens_host = np.zeros((total_steps, T + 1, w.batch), np.int32)
    cur = [start.copy() for _ in range(L)]
    for s in range(total_steps):
        l = s % L
        for j in range(T + 1):
            lens_host[s, j] = cur[l] + j
        cur[l] = cur[l] + T
    lens_dev = torch.from_numpy(lens_host).to(dev)
    max_len = int(lens_host[:, T].max())
    if P:
        ws = kvq.alloc_paged_workspace(g, T, max_len, dev)
    elif T == 1:
        ws = kvq.alloc_workspace(g, max_len, dev)
    else:
        ws = kvq.alloc_multi_workspace(g, T, max_len, dev)
    if T == 1:
        out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float16, device=dev)
    else:
        out = torch.empty((w.batch, T, w.n_q_heads, w.head_dim), dtype=torch.float16,
                          device=dev)
        qpool = [torch.stack([pool[(s + j) % len(pool)][2] for j in range(T)], 1).contiguous()
                 for s in range(len(pool))]
    scale = 1.0 / math.sqrt(w.head_dim)
    n_workers = (ws.numel() * 4 // (T * (w.n_q_heads // w.n_kv_heads) * (w.head_dim + 4) * 4)
                 - w.batch * w.n_kv_heads)

    # algorithmic bytes of every step
    step_bytes, dec_bytes = [], []
    for s in range(total_steps):
        after = lens_host[s, T]
        db = metrics.decode_step_bytes(after, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                       w.k_bits, w.v_bits, w.group, w.residual)
        db += (T - 1) * 4 * w.batch * w.n_q_heads * w.head_dim  # the other tokens' q and out
        sb = db
        for j in range(T):
            before = lens_host[s, j]
            flushing = int(np.sum((before > 0) & (before % w.residual == 0)))
            sb += metrics.append_bytes(w.batch, w.n_kv_heads, w.head_dim)
            sb += metrics.flush_bytes(flushing * w.n_kv_heads, w.residual, w.head_dim,
                                      w.k_bits, w.v_bits, w.group)
        step_bytes.append(sb)
        dec_bytes.append(db)

    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]

    def step(s, timed_idx=None):
        stream = torch.cuda.current_stream()  # the capture stream inside a graph capture
        l = s % L
        c = caches[l]
        if T == 1:
            kn, vn, _ = pool[s % len(pool)]
            append(g, kn, vn, lens_dev[s, 0], c, stream)
        else:  # the T new tokens in one launch
            kt, vt = tpool[s % len(tpool)]
            append_tokens(g, T, kt, vt, lens_dev[s, 0], c, stream)
        if timed_idx is not None:
            ev_a[timed_idx].record(stream)
        if T == 1:
            q = pool[s % len(pool)][2]
            partial(g, q, c, lens_dev[s, 1], max_len, scale, ws, out, stream)
            if timed_idx is not None:
                ev_b[timed_idx].record(stream)
            combine(g, q, c, lens_dev[s, 1], max_len, scale, ws, out, stream)
        else:  # partial + combine in one call: the events bracket both
            multi(g, qpool[s % len(qpool)], c, lens_dev[s, T], T, max_len, scale, ws, out,
                  stream)
            if timed_idx is not None:
                ev_b[timed_idx].record(stream)

    for s in range(a.warmup):
        step(s)
    torch.cuda.synchronize()
    elapsed_eager, elapsed = time_steps(a, step, torch)

    timed = slice(a.warmup, a.warmup + a.steps)
    total_bytes = float(np.sum(step_bytes[timed]))
    part_ms = np.array([ev_a[i].elapsed_time(ev_b[i]) for i in range(a.steps)])
    part_avg_s = float(np.mean(part_ms)) / 1e3
    part_pct = {f"p{q}_us": round(float(np.percentile(part_ms, q)) * 1e3, 3) for q in (10, 50, 90)}
    ceiling = kvq.stream_read_gbs()
    dec_avg_bytes = float(np.mean(dec_bytes[timed]))
    achieved = dec_avg_bytes / part_avg_s / 1e9
    gbs = total_bytes / elapsed / 1e9
    gbs_eager = total_bytes / elapsed_eager / 1e9
    traffic = load_traffic(w.name) if T == 1 and not P else None

    rec = {
        "metric": "quantized-KV decode attention: effective HBM GB/s (% of peak) + tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(elapsed / a.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; keys with per-channel lognormal scales and outlier "
                "channels, values and queries N(0,1), fp16)",
        "config": {
            "workload": w.name,
            "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "k_bits": w.k_bits, "v_bits": w.v_bits,
            "group": w.group, "residual": w.residual,
            "context_first_step": int(lens_host[a.warmup, T].max()),
            "context_last_step": int(lens_host[-1, T].max()),
            "rotating_layer_caches": L, "decode_worker_waves": n_workers,
            "step": ("kvq_append (+flush when a window fills) + kvq_decode_attn, one layer"
                     if T == 1 else
                     f"kvq_append_tokens (T={T}) + kvq_decode_attn_multi, one layer"),
            "query_tokens": T,
            "cache": f"paged, {P}-position pages in shuffled order" if P else "dense",
            "launch": ("kernels launched one by one" if a.eager else
                       "the timed steps replayed as one HIP graph"),
        },
        "eager": {"value": round(gbs_eager, 2), "unit": "GB/s",
                  "ms_per_step": round(elapsed_eager / a.steps * 1e3, 5),
                  "tokens_per_s": round(w.batch * T * a.steps / elapsed_eager, 1)},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(w.batch * T * a.steps / elapsed, 1),
        "tokens_per_s_unit": "decoded tokens per second through one layer",
        **({"stack_tokens_per_s": round(w.batch * T * a.steps / L / elapsed, 1),
            "stack_tokens_per_s_unit": f"decoded tokens per second through all {L} layers"}
           if w.layers > 1 else {}),
        "roofline": {
            "kernel": ("decode_partial" if T == 1 else
                       "decode_partial+decode_combine (multi)") + (" (paged)" if P else ""),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(part_avg_s * 1e6, 3),
            **part_pct,
            "algorithmic_bytes_per_launch": round(dec_avg_bytes),
            "frac_of_stream_read": round(achieved / ceiling["gbs"], 4),
        },
        "stream_read": {**ceiling, "kernel": "kvq_probe_stream_read (plain 16-byte loads, "
                                              "2 GiB buffer beyond the Infinity Cache)"},
        "gpu": torch.cuda.get_device_name(0),
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
