"""GPU parity with separate key and value windows (Rk = residual, Rv =
residual_v), through the C ABI.

Keys flush every Rk positions and values every Rv, so between the two packed
lengths lie chunks packed for one tensor and in the window for the other.
Packed state and both windows must equal the oracle's bit for bit and outputs
be within |gpu - oracle| <= 1e-3 * (1 + |oracle|), for both orders of the two
lengths, lengths that do not divide each other, single- and multi-token
attention, and the paged cache.  Rv = Rk set explicitly equals Rv = 0 bit for
bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq

from kvq_testutil import assert_cache_equal, assert_close, decode_both, dev, geoms, prefill_both

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(rng, B, Hkv, D, n, Hq, T=None):
    k = (rng.standard_normal((B, Hkv, n, D)) *
         rng.lognormal(0, 0.5, (1, Hkv, 1, D))).astype(np.float16)
    v = rng.standard_normal((B, Hkv, n, D)).astype(np.float16)
    qs = (B, Hq, D) if T is None else (B, T, Hq, D)
    q = rng.standard_normal(qs).astype(np.float16)
    return k, v, q


CASES = [
    # (B, Hq, Hkv, D, bK, bV, G, Rk, Rv, C, lens)
    (3, 8, 2, 128, 2, 4, 32, 32, 128, 1024, [200, 129, 1000]),    # keys packed further
    (3, 8, 2, 128, 2, 4, 32, 128, 32, 1024, [200, 129, 1000]),    # values packed further
    (2, 16, 2, 64, 4, 2, 32, 64, 96, 1152, [300, 1100]),          # lengths not dividing
    (4, 4, 4, 64, 2, 2, 64, 64, 128, 512, [64, 65, 128, 511]),    # window edges
    (2, 32, 8, 128, 8, 4, 32, 32, 256, 1024, [1000, 289]),        # 8-bit keys, GQA 4
    (2, 4, 1, 128, 4, 8, 128, 256, 128, 1024, [700, 257]),        # G128
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"D{c[3]}K{c[4]}V{c[5]}G{c[6]}Rk{c[7]}Rv{c[8]}")
def test_windows_prefill_and_decode(case):
    B, Hq, Hkv, D, bK, bV, G, Rk, Rv, C, lens = case
    _say(f"windows prefill+decode {case}")
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, Rk, C, Rv)
    rng = np.random.default_rng(Rk + 7 * Rv + sum(lens))
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq)
    cache, oc = prefill_both(g, og, k, v, lens)
    assert_cache_equal(cache, oc, lens, what="windows prefill")
    out, ref = decode_both(g, og, cache, oc, q, lens)
    assert_close(out, ref, what=f"windows {case}")


@pytest.mark.parametrize("Rk,Rv", [(32, 64), (64, 32), (32, 96)])
def test_windows_append_steps(Rk, Rv):
    """Decode steps over flushes of both windows at their own times; packed
    state and windows bit-exact at the end, outputs checked along the way."""
    B, Hq, Hkv, D, bK, bV, G, C = 3, 8, 2, 128, 2, 4, 32, 768
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, Rk, C, Rv)
    rng = np.random.default_rng(Rk * Rv)
    lens0 = np.array([1, 60, 200], np.int32)
    steps = 200
    k, v, _ = _inputs(rng, B, Hkv, D, int(lens0.max()) + steps, Hq)
    _say(f"windows append Rk={Rk} Rv={Rv}")
    cache, oc = prefill_both(g, og, k, v, lens0)
    lens = lens0.copy()
    for s in range(steps):
        kn = np.ascontiguousarray(k[np.arange(B), :, lens])
        vn = np.ascontiguousarray(v[np.arange(B), :, lens])
        kvq.kvq_append(g, dev(kn), dev(vn), dev(lens), cache)
        oracle.append(og, oc, kn, vn, lens)
        lens = lens + 1
        if s % 40 == 39:
            q = rng.standard_normal((B, Hq, D)).astype(np.float16)
            out, ref = decode_both(g, og, cache, oc, q, lens)
            assert_close(out, ref, what=f"windows step {s}")
    assert_cache_equal(cache, oc, lens, what="windows append")


@pytest.mark.parametrize("Rk,Rv,lens", [(32, 128, [131, 190, 4, 97]), (128, 32, [131, 190, 4, 97])])
def test_windows_multi_token(Rk, Rv, lens):
    """T = 4 over mixed chunks: the causal mask reaches into them."""
    B, Hq, Hkv, D, bK, bV, G, C, T = 4, 8, 2, 128, 2, 4, 32, 512, 4
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, Rk, C, Rv)
    rng = np.random.default_rng(Rk + Rv + 5)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq, T)
    _say(f"windows multi Rk={Rk} Rv={Rv} lens {lens}")
    cache, oc = prefill_both(g, og, k, v, lens)
    out = torch.empty((B, T, Hq, D), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_multi_workspace(g, T, max(lens))
    kvq.kvq_decode_attn_multi(g, dev(q), cache, dev(np.asarray(lens, np.int32)), T, max(lens),
                              0.125, ws, out)
    torch.cuda.synchronize()
    ref = oracle.decode_attn_multi(og, oc, q, np.asarray(lens, np.int32), T, 0.125)
    assert_close(out, ref, what="windows T=4")


def test_windows_paged():
    """The paged cache with separate windows: pages must cover the longer of
    the two packed lengths."""
    B, Hq, Hkv, D, bK, bV, G, Rk, Rv, C, P = 3, 8, 2, 128, 2, 4, 32, 32, 128, 1024, 64
    lens = [1000, 200, 129]
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, Rk, C, Rv)
    rng = np.random.default_rng(31)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq)
    need = [-(-max(oracle.packed_len(n, Rk), oracle.packed_len(n, Rv)) // P) for n in lens]
    npages = sum(need) + 2
    perm = rng.permutation(npages).astype(np.int32)
    table = np.full((B, C // P), -1, np.int32)
    o = 0
    for b in range(B):
        table[b, :need[b]] = perm[o:o + need[b]]
        o += need[b]
    _say(f"windows paged {need}")
    pc = kvq.PagedCache(g, P, npages, dev(table))
    for b, n in enumerate(lens):
        sub = pc.view(b, b + 1)
        kvq.kvq_paged_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
    _, oc = prefill_both(g, og, k, v, lens)
    out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_paged_workspace(g, 1, max(lens))
    kvq.kvq_paged_decode_attn(g, dev(q), pc, dev(np.asarray(lens, np.int32)), max(lens), 0.125,
                              ws, out)
    torch.cuda.synchronize()
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), 0.125)
    assert_close(out, ref, what="windows paged")


def test_equal_windows_set_explicitly_are_the_single_window():
    B, Hq, Hkv, D, bK, bV, G, R, C = 2, 8, 2, 128, 2, 4, 32, 128, 1024
    lens = [1000, 300]
    rng = np.random.default_rng(32)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq)
    outs = []
    for rv in (0, R):
        g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C, rv)
        cache, oc = prefill_both(g, og, k, v, lens)
        out, _ = decode_both(g, og, cache, oc, q, lens)
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("Rk,Rv", [(32, 128), (128, 32)])
def test_windows_paged_multi_token_8bit(Rk, Rv):
    """The new parts together: 8-bit keys, separate windows, the paged cache in
    shuffled 32-position pages and T = 4 (causal mask across packed, mixed and
    window chunks)."""
    B, Hq, Hkv, D, bK, bV, G, C, P, T = 3, 8, 2, 128, 8, 4, 32, 1024, 32, 4
    lens = [700, 131, 290]
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, Rk, C, Rv)
    rng = np.random.default_rng(Rk + 3 * Rv + 1)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq, T)
    need = [-(-max(oracle.packed_len(n, Rk), oracle.packed_len(n, Rv)) // P) for n in lens]
    npages = sum(need) + 4
    perm = rng.permutation(npages).astype(np.int32)
    table = np.full((B, C // P), -1, np.int32)
    o = 0
    for b in range(B):
        table[b, :need[b]] = perm[o:o + need[b]]
        o += need[b]
    _say(f"windows paged multi 8-bit Rk={Rk} Rv={Rv} pages {need}")
    pc = kvq.PagedCache(g, P, npages, dev(table))
    for b, n in enumerate(lens):
        sub = pc.view(b, b + 1)
        kvq.kvq_paged_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
    _, oc = prefill_both(g, og, k, v, lens)
    out = torch.empty((B, T, Hq, D), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_paged_workspace(g, T, max(lens))
    kvq.kvq_paged_decode_attn_multi(g, dev(q), pc, dev(np.asarray(lens, np.int32)), T,
                                    max(lens), 0.125, ws, out)
    torch.cuda.synchronize()
    ref = oracle.decode_attn_multi(og, oc, q, np.asarray(lens, np.int32), T, 0.125)
    assert_close(out, ref, what="paged multi 8-bit windows")
