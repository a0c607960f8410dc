"""GPU parity at the benchmark workloads' full sizes.

The GPU runs the whole configuration exactly as bench.py launches it: every
sequence of the batch, the workload's lengths, prefill of the packed prefix,
then decode steps (kvq_append + kvq_decode_attn) with the worker grid the
library picks for the geometry.  The oracle then recomputes sampled sequences
one by one: their packed codes, scales, mins and live residual slots must match
bit for bit, and all their query heads' outputs must be within
|gpu - oracle| <= 1e-3 * (1 + |oracle|).  Because the work decomposition spans
all (sequence, KV head) units of the batch, a sampled sequence's units sit
wherever the full launch puts them, worker boundaries included.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq
from quantized_decode_attention_amd import synth

from kvq_testutil import assert_close, cache_np, dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu_prefill(g, cache, kd, vd, start):
    if np.all(start == start[0]):
        n = int(start[0])
        kvq.kvq_prefill(g, kd[:, :, :n].contiguous(), vd[:, :, :n].contiguous(), n, cache)
        return
    for b, n in enumerate(start.tolist()):
        sub = cache.view(b, b + 1)
        kvq.kvq_prefill(sub.g, kd[b:b + 1, :, :n].contiguous(),
                        vd[b:b + 1, :, :n].contiguous(), n, sub)


def _oracle_seq(w, cap, k, v, b, n):
    """Oracle cache of sequence b alone, prefilled to n tokens."""
    og = oracle.Geom(1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                     w.group, w.residual, cap)
    oc = oracle.Cache(og)
    oracle.prefill(og, oc, k[b:b + 1, :, :n], v[b:b + 1, :, :n], n)
    return og, oc


def _check_seq_cache(got, oc, w, b, n, what):
    """Sequence b of the GPU cache (host copy) against the oracle's one-sequence
    cache: packed prefix and live residual slots bit-exact."""
    lq = oracle.packed_len(n, w.residual)
    for name, blocks in (("k_codes", lq // 32), ("v_codes", lq // 32),
                         ("k_meta", lq // w.group), ("v_meta", lq // 32)):
        gg = got[name][b, :, :blocks]
        oo = getattr(oc, name)[0, :, :blocks]
        bad = np.argwhere(gg != oo)
        assert bad.size == 0, f"{what} seq {b} {name}: {len(bad)} mismatches, first {bad[0]}"
    og = oc.g
    vg = oracle.value_res_rows(og, got["v_res"][b:b + 1])
    vo = oracle.value_res_rows(og, oc.v_res)
    for t in range(lq, n):
        s = t % w.residual
        assert np.array_equal(got["k_res"][b, :, s], oc.k_res[0, :, s]), \
            f"{what} seq {b} k_res slot {s}"
        assert np.array_equal(vg[0, :, s], vo[0, :, s]), f"{what} seq {b} v_res slot {s}"


@pytest.mark.parametrize("cfg,samples", [(2, (0, 5)), (3, (0, 13, 31)), (4, (0, 1, 2, 3))])
def test_one_step_full_size(cfg, samples):
    """One decode step (append of the token at n - 1, attention over n) at the
    workload's full batch and lengths."""
    w = synth.WORKLOADS[cfg]
    lens = synth.seq_lens(w)                 # n at attention time
    start = (lens - 1).astype(np.int32)      # tokens before the step's append
    cap = synth.capacity_for(w, 2)
    g = kvq.Geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                 w.group, w.residual, cap)
    _say(f"full-size cfg {cfg} ({w.name}): lengths {int(lens.min())}..{int(lens.max())}, "
         f"workers {kvq.kvq_decode_workers(g)}")
    nmax = int(start.max())
    k = synth.keys(w, nmax)
    v = synth.values(w, nmax)
    kn, vn, q = synth.step_token(w, 0)
    cache = kvq.Cache(g)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    _gpu_prefill(g, cache, kd, vd, start)
    del kd, vd
    kvq.kvq_append(g, dev(kn), dev(vn), dev(start), cache)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float16, device="cuda")
    msl = int(lens.max())
    ws = kvq.alloc_workspace(g, msl)
    scale = 1.0 / math.sqrt(w.head_dim)
    kvq.kvq_decode_attn(g, dev(q), cache, dev(lens), msl, scale, ws, out)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    og_full = oracle.Geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits,
                          w.v_bits, w.group, w.residual, cap)
    got = cache_np(cache, oracle.Cache(og_full))
    del cache
    for b in samples:
        _say(f"  oracle sequence {b} (n = {int(lens[b])})")
        og, oc = _oracle_seq(w, cap, k, v, b, int(start[b]))
        oracle.append(og, oc, kn[b:b + 1], vn[b:b + 1], start[b:b + 1])
        _check_seq_cache(got, oc, w, b, int(lens[b]), f"cfg{cfg}")
        ref = oracle.decode_attn(og, oc, q[b:b + 1], lens[b:b + 1], float(np.float32(scale)))
        err = assert_close(o[b:b + 1], ref, what=f"cfg{cfg} seq {b}")
        _say(f"    max err {err:.2e}")


@pytest.mark.parametrize("layer", [0, 15, 31])
def test_full_stack_layer_through_flushes(layer):
    """The full-stack workload (32 layers, 256 decode steps from a 4096-token
    prefix, K4/V2, G = R = 64) at its full batch, layers 0, 15 and 31 (each
    layer its own seeded keys, values and tokens): all 256 steps, so the
    flushes at n = 4096 (step 1), 4160, 4224 and 4288 all happen; sampled
    outputs on both sides of every flush and at the last step, for sequences
    0, 37 and 63, and their packed state after the last step."""
    w = synth.WORKLOADS[5]
    steps = w.steps
    start = np.full(w.batch, w.context, np.int32)
    cap = synth.capacity_for(w, steps + 1)
    g = kvq.Geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                 w.group, w.residual, cap)
    _say(f"full-stack layer {layer} ({w.name}): {steps} steps, workers "
         f"{kvq.kvq_decode_workers(g)}")
    k = synth.keys(w, w.context, layer=layer)
    v = synth.values(w, w.context, layer=layer)
    cache = kvq.Cache(g)
    _gpu_prefill(g, cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), start)
    toks = [synth.step_token(w, s, layer=layer) for s in range(steps)]
    msl = w.context + steps
    ws = kvq.alloc_workspace(g, msl)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float16, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    check_at = (1, 2, 64, 65, 128, 129, 192, 193, 256)
    outs = {}
    lens = start.copy()
    for s in range(steps):
        kn, vn, q = toks[s]
        kvq.kvq_append(g, dev(kn), dev(vn), dev(lens), cache)
        kvq.kvq_decode_attn(g, dev(q), cache, dev(lens + 1), msl, scale, ws, out)
        lens += 1
        if s + 1 in check_at:
            outs[s + 1] = out.float().cpu().numpy()
    torch.cuda.synchronize()
    og_full = oracle.Geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits,
                          w.v_bits, w.group, w.residual, cap)
    got = cache_np(cache, oracle.Cache(og_full))
    for b in (0, 37, 63):
        _say(f"  layer {layer}: oracle sequence {b}")
        og, oc = _oracle_seq(w, cap, k, v, b, w.context)
        n = w.context
        for s in range(steps):
            kn, vn, q = toks[s]
            oracle.append(og, oc, kn[b:b + 1], vn[b:b + 1], np.array([n], np.int32))
            n += 1
            if s + 1 in check_at:
                ref = oracle.decode_attn(og, oc, q[b:b + 1], np.array([n], np.int32),
                                         float(np.float32(scale)))
                assert_close(outs[s + 1][b:b + 1], ref,
                             what=f"cfg5 layer {layer} seq {b} step {s + 1}")
        _check_seq_cache(got, oc, w, b, n, f"cfg5 layer {layer}")
