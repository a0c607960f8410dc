"""GPU parity of decode in one kernel (kvq_decode_attn_fused and its paged
form), through the C ABI: the wave that completes a unit's partials merges
them.  Outputs within |gpu - oracle| <= 1e-3 * (1 + |oracle|) of the oracle
and of the two-kernel decode; degenerate lengths as kvq_decode_attn; the
workspace is zeroed once and reused across calls (its counters return to
zero after every call)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq
from quantized_decode_attention_amd import synth

from kvq_testutil import assert_close, dev, geoms, prefill_both

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # B, Hq, Hkv, D, bK, bV, G, R, lens
    (1, 2, 2, 64, 2, 2, 32, 32, [256]),
    (2, 32, 8, 128, 2, 4, 32, 128, [3000, 2177]),
    (3, 32, 8, 128, 2, 2, 64, 128, [5000, 129, 4097]),
    (2, 16, 2, 64, 4, 4, 64, 64, [777, 64]),
    (1, 16, 1, 128, 8, 4, 128, 128, [1500]),
    (4, 4, 2, 64, 2, 2, 32, 32, [33, 64, 65, 31]),
    (70, 4, 2, 64, 2, 4, 32, 32, list(range(1, 141, 2))),   # more sequences than a wave
]


def _inputs(rng, B, Hkv, D, n, Hq, T=None):
    k = (rng.standard_normal((B, Hkv, n, D)) *
         rng.lognormal(0, 0.5, (1, Hkv, 1, D))).astype(np.float16)
    v = rng.standard_normal((B, Hkv, n, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D) if T is None else (B, T, Hq, D)).astype(np.float16)
    return k, v, q


def _fused(g, cache, q, lens, T, msl, scale, ws=None, paged=False):
    out = torch.full(tuple(q.shape), 7.0, dtype=torch.float16, device="cuda")
    if ws is None:
        ws = kvq.alloc_fused_workspace(g, T, msl, paged)
    kvq.kvq_decode_attn_fused(g, dev(q), cache, dev(np.asarray(lens, np.int32)), T, msl, scale,
                              ws, out)
    torch.cuda.synchronize()
    return out, ws


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_fused_parity(case):
    B, Hq, Hkv, D, bK, bV, G, R, lens = case
    _say(f"fused {case[:8]} {len(lens)} seqs")
    nmax = max(lens)
    C = (nmax // R + 2) * R
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(nmax + B + 3)
    k, v, q = _inputs(rng, B, Hkv, D, nmax, Hq)
    cache, oc = prefill_both(g, og, k, v, lens)
    scale = 1.0 / math.sqrt(D)
    out, ws = _fused(g, cache, q, lens, 1, nmax, scale)
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), float(np.float32(scale)))
    assert_close(out, ref, what="fused")
    # the two-kernel path on the same inputs
    two = torch.empty_like(out)
    kvq.kvq_decode_attn(g, dev(q), cache, dev(np.asarray(lens, np.int32)), nmax, scale,
                        kvq.alloc_workspace(g, nmax), two)
    torch.cuda.synchronize()
    assert_close(out, two.float().cpu().numpy().astype(np.float64), what="fused vs two-kernel")
    # the counters are back to zero: the same workspace serves the next call
    counters = ws.view(torch.int32)[-((B * Hkv + 3) // 4 * 4):][:B * Hkv]
    assert int(counters.abs().sum()) == 0
    q2 = rng.standard_normal(q.shape).astype(np.float16)
    out2, _ = _fused(g, cache, q2, lens, 1, nmax, scale, ws)
    ref2 = oracle.decode_attn(og, oc, q2, np.asarray(lens, np.int32), float(np.float32(scale)))
    assert_close(out2, ref2, what="fused, reused workspace")


def test_fused_degenerate_lengths():
    """Length 0 gives zeros and an out-of-range length NaN, as kvq_decode_attn."""
    B, Hq, Hkv, D, bK, bV, G, R, C = 4, 8, 2, 64, 2, 2, 32, 32, 256
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(51)
    k, v, q = _inputs(rng, B, Hkv, D, 200, Hq)
    lens = [200, 0, 150, 100]
    cache, oc = prefill_both(g, og, k, v, lens)
    lens_bad = [200, 0, 150, 230]                  # 230 > max_seq_len = 200
    out, _ = _fused(g, cache, q, lens_bad, 1, 200, 0.125)
    o = out.float().cpu().numpy()
    assert np.all(o[1] == 0)
    assert np.all(np.isnan(o[3]))
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), 0.125)
    assert_close(o[[0, 2]], ref[[0, 2]], what="fused, other sequences")


def test_fused_multi_token():
    B, Hq, Hkv, D, bK, bV, G, R, C, T = 3, 8, 2, 128, 2, 4, 32, 128, 1024, 4
    lens = [131, 900, 4]
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(52)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq, T)
    cache, oc = prefill_both(g, og, k, v, lens)
    out, _ = _fused(g, cache, q, lens, T, max(lens), 0.125)
    ref = oracle.decode_attn_multi(og, oc, q, np.asarray(lens, np.int32), T, 0.125)
    assert_close(out, ref, what="fused T=4")


def test_fused_paged():
    B, Hq, Hkv, D, bK, bV, G, R, C, P = 3, 8, 2, 128, 2, 4, 32, 128, 1024, 128
    lens = [1000, 129, 640]
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(53)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq)
    npages = B * (C // P)
    table = rng.permutation(npages).astype(np.int32).reshape(B, C // P)
    pc = kvq.PagedCache(g, P, npages, dev(table))
    for b, n in enumerate(lens):
        sub = pc.view(b, b + 1)
        kvq.kvq_paged_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
    _, oc = prefill_both(g, og, k, v, lens)
    out, _ = _fused(g, pc, q, lens, 1, max(lens), 0.125, paged=True)
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), 0.125)
    assert_close(out, ref, what="fused paged")


def test_fused_full_size_matches_two_kernel():
    """The Llama-3-8B-shaped layer at 32 x 8192: fused decode within the
    tolerance of the two-kernel decode (itself checked against the oracle at
    this size)."""
    w = synth.WORKLOADS[3]
    lens = synth.seq_lens(w)
    n = int(lens.max())
    C = synth.capacity_for(w, 256)
    g = kvq.Geom(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits, w.group,
                 w.residual, C)
    _say("fused full size")
    cache = kvq.Cache(g)
    kvq.kvq_prefill(g, torch.from_numpy(synth.keys(w, n)).cuda(),
                    torch.from_numpy(synth.values(w, n)).cuda(), n, cache)
    q = synth.queries(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    out, ws = _fused(g, cache, q, lens, 1, n, scale)
    two = torch.empty_like(out)
    kvq.kvq_decode_attn(g, dev(q), cache, dev(lens), n, scale, kvq.alloc_workspace(g, n), two)
    torch.cuda.synchronize()
    assert_close(out, two.float().cpu().numpy().astype(np.float64), what="fused full size")
