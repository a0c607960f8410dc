"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay, with eager work and synchronizations in between, must give the
eager run's bits.  libkvq's calls enqueue kernels only (no allocation, no
memset, no synchronization), so a step of append + decode can be captured as
serving loops do."""
import sys

import numpy as np
import pytest
import torch

import quantized_decode_attention_amd as kvq

from kvq_testutil import dev, geoms

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("paged", [False, True])
def test_graph_replays_equal_eager(paged):
    B, Hq, Hkv, D, bK, bV, G, R, C = 4, 32, 8, 128, 2, 4, 32, 128, 2048
    g, _ = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(41)
    n0 = np.array([1000, 1023, 1024, 1500], np.int32)   # flushes inside the steps
    steps = 6
    k = rng.standard_normal((B, Hkv, int(n0.max()) + steps, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, int(n0.max()) + steps, D)).astype(np.float16)
    qs = [dev(rng.standard_normal((B, Hq, D)).astype(np.float16)) for _ in range(steps)]
    kn = [dev(np.ascontiguousarray(k[np.arange(B), :, n0 + s])) for s in range(steps)]
    vn = [dev(np.ascontiguousarray(v[np.arange(B), :, n0 + s])) for s in range(steps)]
    before = [dev(n0 + s) for s in range(steps)]
    after = [dev(n0 + s + 1) for s in range(steps)]
    msl = int(n0.max()) + steps
    _say(f"graph replay paged={paged}")

    def fresh():
        if paged:
            P = 128
            table = np.arange(B * (C // P), dtype=np.int32).reshape(B, C // P)[:, ::-1].copy()
            c = kvq.PagedCache(g, P, B * (C // P), dev(table))
            pre, app, dec = kvq.kvq_paged_prefill, kvq.kvq_paged_append, kvq.kvq_paged_decode_attn
            ws = kvq.alloc_paged_workspace(g, 1, msl)
        else:
            c = kvq.Cache(g)
            pre, app, dec = kvq.kvq_prefill, kvq.kvq_append, kvq.kvq_decode_attn
            ws = kvq.alloc_workspace(g, msl)
        for b in range(B):
            sub = c.view(b, b + 1)
            n = int(n0[b])
            pre(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        outs = [torch.empty((B, Hq, D), dtype=torch.float16, device="cuda") for _ in range(steps)]
        return c, app, dec, ws, outs

    def run_steps(c, app, dec, ws, outs):
        st = torch.cuda.current_stream()
        for s in range(steps):
            app(g, kn[s], vn[s], before[s], c, st)
            dec(g, qs[s], c, after[s], msl, 0.125, ws, outs[s], st)

    # eager reference
    c, app, dec, ws, outs = fresh()
    run_steps(c, app, dec, ws, outs)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    # capture on a fresh cache, replay from the same starting state each time
    c, app, dec, ws, outs = fresh()
    snapshot = [t.clone() for t in c.tensors()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps(c, app, dec, ws, outs)
    for rep in range(4):
        for t, s0 in zip(c.tensors(), snapshot):   # eager work between replays
            t.copy_(s0)
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs[s].view(torch.int16), ref[s].view(torch.int16)), (rep, s)


@pytest.mark.parametrize("paged", [False, True])
def test_graph_replays_equal_eager_multi_token(paged):
    """Steps of kvq_append_tokens (T = 4, flushes part-way) + multi-token decode."""
    B, Hq, Hkv, D, bK, bV, G, R, C, T = 4, 32, 8, 128, 2, 4, 32, 128, 2048, 4
    g, _ = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(43)
    n0 = np.array([1000, 1022, 1024, 1500], np.int32)
    steps = 3
    k = rng.standard_normal((B, Hkv, int(n0.max()) + steps * T, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, int(n0.max()) + steps * T, D)).astype(np.float16)
    qs = [dev(rng.standard_normal((B, T, Hq, D)).astype(np.float16)) for _ in range(steps)]
    kt = [dev(np.ascontiguousarray(np.stack([k[np.arange(B), :, n0 + s * T + t] for t in range(T)], 1)))
          for s in range(steps)]
    vt = [dev(np.ascontiguousarray(np.stack([v[np.arange(B), :, n0 + s * T + t] for t in range(T)], 1)))
          for s in range(steps)]
    before = [dev(n0 + s * T) for s in range(steps)]
    after = [dev(n0 + (s + 1) * T) for s in range(steps)]
    msl = int(n0.max()) + steps * T
    _say(f"graph replay multi-token paged={paged}")

    def fresh():
        if paged:
            P = 128
            table = np.arange(B * (C // P), dtype=np.int32).reshape(B, C // P)[:, ::-1].copy()
            c = kvq.PagedCache(g, P, B * (C // P), dev(table))
            pre, app, dec = (kvq.kvq_paged_prefill, kvq.kvq_paged_append_tokens,
                             kvq.kvq_paged_decode_attn_multi)
            ws = kvq.alloc_paged_workspace(g, T, msl)
        else:
            c = kvq.Cache(g)
            pre, app, dec = kvq.kvq_prefill, kvq.kvq_append_tokens, kvq.kvq_decode_attn_multi
            ws = kvq.alloc_multi_workspace(g, T, msl)
        for b in range(B):
            sub = c.view(b, b + 1)
            n = int(n0[b])
            pre(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        outs = [torch.empty((B, T, Hq, D), dtype=torch.float16, device="cuda")
                for _ in range(steps)]
        return c, app, dec, ws, outs

    def run_steps(c, app, dec, ws, outs):
        st = torch.cuda.current_stream()
        for s in range(steps):
            app(g, T, kt[s], vt[s], before[s], c, st)
            dec(g, qs[s], c, after[s], T, msl, 0.125, ws, outs[s], st)

    c, app, dec, ws, outs = fresh()
    run_steps(c, app, dec, ws, outs)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    c, app, dec, ws, outs = fresh()
    snapshot = [t.clone() for t in c.tensors()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps(c, app, dec, ws, outs)
    for rep in range(4):
        for t, s0 in zip(c.tensors(), snapshot):   # eager work between replays
            t.copy_(s0)
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs[s].view(torch.int16), ref[s].view(torch.int16)), (rep, s)


def test_graph_replays_equal_eager_bq2():
    """The rotated 2-bit format's append + decode, captured and replayed."""
    B, Hq, Hkv, C = 4, 32, 8, 4096
    g = kvq.Bq2Geom(B, Hq, Hkv, C)
    rng = np.random.default_rng(42)
    n0 = np.array([1000, 3, 2047, 3000], np.int32)
    steps = 5
    k = rng.standard_normal((B, Hkv, int(n0.max()) + steps, 64)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, int(n0.max()) + steps, 64)).astype(np.float16)
    qs = [dev(rng.standard_normal((B, Hq, 64)).astype(np.float16)) for _ in range(steps)]
    kn = [dev(np.ascontiguousarray(k[np.arange(B), :, n0 + s])) for s in range(steps)]
    vn = [dev(np.ascontiguousarray(v[np.arange(B), :, n0 + s])) for s in range(steps)]
    before = [dev(n0 + s) for s in range(steps)]
    after = [dev(n0 + s + 1) for s in range(steps)]
    msl = int(n0.max()) + steps
    _say("graph replay bq2")

    def fresh():
        c = kvq.Bq2Cache(g)
        for b in range(B):
            n = int(n0[b])
            gb = kvq.Bq2Geom(1, Hq, Hkv, C)
            sub = kvq.Bq2Cache.__new__(kvq.Bq2Cache)
            for name, t in zip(("k_codes", "v_codes", "k_meta", "v_meta", "k_sink", "v_sink"),
                               c.tensors()):
                setattr(sub, name, t[b:b + 1])
            kvq.kvq_bq2_prefill(gb, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        ws = kvq.alloc_bq2_workspace(g, msl)
        outs = [torch.empty((B, Hq, 64), dtype=torch.float16, device="cuda") for _ in range(steps)]
        return c, ws, outs

    def run_steps(c, ws, outs):
        st = torch.cuda.current_stream()
        for s in range(steps):
            kvq.kvq_bq2_append(g, kn[s], vn[s], before[s], c, st)
            kvq.kvq_bq2_decode_attn(g, qs[s], c, after[s], msl, 0.125, ws, outs[s], st)

    c, ws, outs = fresh()
    run_steps(c, ws, outs)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    c, ws, outs = fresh()
    snapshot = [t.clone() for t in c.tensors()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps(c, ws, outs)
    for rep in range(3):
        for t, s0 in zip(c.tensors(), snapshot):
            t.copy_(s0)
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs[s].view(torch.int16), ref[s].view(torch.int16)), (rep, s)
