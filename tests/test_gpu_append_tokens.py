"""kvq_append_tokens / kvq_paged_append_tokens: T new tokens per sequence in
one call.  The cache must end bit-identical to T kvq_append calls (token t
with lengths + t) on the full buffers, and to the oracle's T appends on every
sequence's live state; multi-token decode over it matches the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq

from kvq_testutil import assert_cache_equal, assert_close, dev, geoms, prefill_both

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[append_tokens] {msg}", flush=True)
    sys.stdout.flush()


def _tokens(k, v, lens, T):
    """[B][T][Hkv][D] of positions lens[b] + t, and the [B][Hkv][D] slices."""
    B = k.shape[0]
    kt = np.stack([np.stack([k[b, :, lens[b] + t] for t in range(T)]) for b in range(B)])
    vt = np.stack([np.stack([v[b, :, lens[b] + t] for t in range(T)]) for b in range(B)])
    return np.ascontiguousarray(kt), np.ascontiguousarray(vt)


@pytest.mark.parametrize("bK,bV,G,R,Rv,T", [
    (2, 4, 32, 128, 0, 4),     # the Llama-3-8B budget
    (2, 2, 32, 32, 0, 16),     # several tokens past a flush
    (4, 2, 64, 64, 0, 2),
    (8, 8, 32, 64, 0, 3),
    (2, 4, 32, 64, 128, 4),    # separate key and value windows
    (4, 4, 64, 128, 64, 5),
])
def test_append_tokens_equals_single_appends(bK, bV, G, R, Rv, T):
    B, Hq, Hkv, D = 4, 4, 2, 128
    Rmax = max(R, Rv or R)
    calls = 2 * Rmax // T + 2           # crosses at least two flushes per window
    start = np.array([R - 2, 0, 2 * Rmax, 3 * Rmax - 1], np.int32)
    C = (int(start.max()) + calls * T) // Rmax * Rmax + 2 * Rmax
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C, Rv)
    _say(f"bK={bK} bV={bV} G={G} R={R} Rv={Rv} T={T} start {start.tolist()}")
    rng = np.random.default_rng(100 + 10 * bK + bV + T)
    total = int(start.max()) + calls * T
    k = rng.standard_normal((B, Hkv, total, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, total, D)).astype(np.float16)
    multi, oc = prefill_both(g, og, k, v, start)
    single, _ = prefill_both(g, og, k, v, start)
    lens = start.copy()
    scale = 1.0 / math.sqrt(D)
    for call in range(calls):
        kt, vt = _tokens(k, v, lens, T)
        kvq.kvq_append_tokens(g, T, dev(kt), dev(vt), dev(lens), multi)
        for t in range(T):
            kn, vn = kt[:, t], vt[:, t]
            kvq.kvq_append(g, dev(np.ascontiguousarray(kn)), dev(np.ascontiguousarray(vn)),
                           dev(lens + t), single)
            oracle.append(og, oc, np.ascontiguousarray(kn), np.ascontiguousarray(vn), lens + t)
        lens = lens + T
        torch.cuda.synchronize()
        for name, a, b in zip(("k_codes", "v_codes", "k_meta", "v_meta", "k_res", "v_res"),
                              multi.tensors(), single.tensors()):
            assert torch.equal(a, b), f"call {call} {name}: T-token append != {T} appends"
        if call in (0, calls // 2, calls - 1):
            assert_cache_equal(multi, oc, lens=lens, what=f"call {call}")
            if T * Hq // Hkv not in (1, 2, 4, 8, 16):  # rows the multi-token decode tiles
                continue
            q = rng.standard_normal((B, T, Hq, D)).astype(np.float16)
            out = torch.empty((B, T, Hq, D), dtype=torch.float16, device="cuda")
            msl = int(lens.max())
            ws = kvq.alloc_multi_workspace(g, T, msl)
            kvq.kvq_decode_attn_multi(g, dev(q), multi, dev(lens), T, msl, scale, ws, out)
            torch.cuda.synchronize()
            ref = oracle.decode_attn_multi(og, oc, q, lens, T, float(np.float32(scale)))
            assert_close(out, ref, what=f"multi decode after call {call}")


def test_append_tokens_out_of_range_is_noop():
    """A sequence whose T tokens would not all fit (or with a negative length)
    is left untouched; the others are appended."""
    B, Hq, Hkv, D, T = 3, 4, 2, 64, 4
    g, og = geoms(B, Hq, Hkv, D, 2, 2, 32, 32, 128)
    rng = np.random.default_rng(7)
    k = rng.standard_normal((B, Hkv, 128, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, 128, D)).astype(np.float16)
    start = np.array([125, 40, 64], np.int32)
    multi, _ = prefill_both(g, og, k, v, start)
    single, _ = prefill_both(g, og, k, v, start)
    kt = rng.standard_normal((B, T, Hkv, D)).astype(np.float16)
    vt = rng.standard_normal((B, T, Hkv, D)).astype(np.float16)
    lens = np.array([125, -1, 64], np.int32)  # 125 + 4 > 128: untouched
    kvq.kvq_append_tokens(g, T, dev(kt), dev(vt), dev(lens), multi)
    for t in range(T):  # only sequence 2 takes them
        keep = np.array([-1, -1, 64 + t], np.int32)
        kvq.kvq_append(g, dev(np.ascontiguousarray(kt[:, t])), dev(np.ascontiguousarray(vt[:, t])),
                       dev(keep), single)
    torch.cuda.synchronize()
    for a, b in zip(multi.tensors(), single.tensors()):
        assert torch.equal(a, b)


def test_paged_append_tokens_equals_single_appends():
    B, Hq, Hkv, D, bK, bV, G, R, C, P, T = 3, 8, 2, 128, 2, 4, 32, 64, 512, 64, 4
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(31)
    start = np.array([62, 128, 1], np.int32)
    calls = 40
    total = int(start.max()) + calls * T
    k = rng.standard_normal((B, Hkv, total, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, total, D)).astype(np.float16)
    maxp = C // P
    perm = rng.permutation(B * maxp).astype(np.int32)  # every page of every row, shuffled
    table = perm.reshape(B, maxp)
    _say(f"paged T={T} start {start.tolist()} calls {calls}")
    multi = kvq.PagedCache(g, P, B * maxp, dev(table))
    single = kvq.PagedCache(g, P, B * maxp, dev(table))
    # the same start on both, by single appends from empty (a sequence that
    # has reached its start gets length -1: untouched)
    lens = np.zeros(B, np.int32)
    while np.any(lens < start):
        step = (lens < start).astype(np.int32)
        kn = np.ascontiguousarray(k[np.arange(B), :, lens])
        vn = np.ascontiguousarray(v[np.arange(B), :, lens])
        ln = np.where(step > 0, lens, -1).astype(np.int32)
        kvq.kvq_paged_append(g, dev(kn), dev(vn), dev(ln), multi)
        kvq.kvq_paged_append(g, dev(kn), dev(vn), dev(ln), single)
        lens = lens + step
    _, oc = prefill_both(g, og, k, v, start)
    scale = 1.0 / math.sqrt(D)
    for call in range(calls):
        kt, vt = _tokens(k, v, lens, T)
        kvq.kvq_paged_append_tokens(g, T, dev(kt), dev(vt), dev(lens), multi)
        for t in range(T):
            kvq.kvq_paged_append(g, dev(np.ascontiguousarray(kt[:, t])),
                                 dev(np.ascontiguousarray(vt[:, t])), dev(lens + t), single)
        lens = lens + T
        torch.cuda.synchronize()
        for a, b in zip(multi.tensors(), single.tensors()):
            assert torch.equal(a, b), f"paged call {call}"
    q = rng.standard_normal((B, T, Hq, D)).astype(np.float16)
    # the oracle's cache of the same positions (prefill of the start, then
    # single appends of every later token)
    ol = start.copy()
    while np.any(ol < lens):
        kn = np.ascontiguousarray(k[np.arange(B), :, ol])
        vn = np.ascontiguousarray(v[np.arange(B), :, ol])
        oracle.append(og, oc, kn, vn, ol)
        ol = ol + 1
    out = torch.empty((B, T, Hq, D), dtype=torch.float16, device="cuda")
    msl = int(lens.max())
    ws = kvq.alloc_paged_workspace(g, T, msl)
    kvq.kvq_paged_decode_attn_multi(g, dev(q), multi, dev(lens), T, msl, scale, ws, out)
    torch.cuda.synchronize()
    ref = oracle.decode_attn_multi(og, oc, q, lens, T, float(np.float32(scale)))
    assert_close(out, ref, what="paged multi decode after T-token appends")
