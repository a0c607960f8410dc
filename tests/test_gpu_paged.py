"""GPU parity of the paged (block-table) cache, through the C ABI.

The pools are filled by kvq_paged_prefill / kvq_paged_append with pages handed
out in a shuffled order (pool pages left unused in between, unread table
entries set to -1).  Gathering every sequence's pages back through its table
row must give the oracle's packed cache bit for bit, and decode over the pages
must be within |gpu - oracle| <= 1e-3 * (1 + |oracle|) of the oracle's
attention.  When the paged and dense kernels run with the same worker count,
decode over the pages must also equal decode over a dense cache holding the
same positions bit for bit (the page indirection changes addresses only).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq
from quantized_decode_attention_amd import synth

from kvq_testutil import assert_cache_equal, assert_close, dev, geoms, prefill_both

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _table(rng, B, maxp, needed, spare=3, shared=None):
    """Shuffled pool pages for logical pages [0, needed[b]) of every sequence
    (the rest of a row -1: never read).  shared = (b_from, b_to, pages): the
    first `pages` entries of row b_to repeat those of row b_from."""
    num_pages = int(sum(needed)) + spare
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((B, maxp), -1, np.int32)
    k = 0
    for b in range(B):
        table[b, :needed[b]] = perm[k:k + needed[b]]
        k += needed[b]
    if shared is not None:
        bf, bt, pages = shared
        table[bt, :pages] = table[bf, :pages]
    return table, num_pages


def _gather(pc: kvq.PagedCache, table: np.ndarray, g):
    """The pools read back through the table into the dense layout of kvq.h
    (chunks of unset entries left zero); returns an object with tensors()."""
    P, G = pc.page_size, g.group
    cpp, gpp = P // 32, P // G
    nchunk, ngroup = g.capacity // 32, g.capacity // G
    t = torch.from_numpy(table).long()
    ok = t >= 0
    k = torch.arange(nchunk)
    pg_c = t[:, k // cpp].clamp(min=0)              # [B][C/32]
    ok_c = ok[:, k // cpp]
    j = torch.arange(ngroup)
    pg_g = t[:, (j * G) // P].clamp(min=0)          # [B][C/G]
    ok_g = ok[:, (j * G) // P]

    def take(pool, pg, inpage, okm):
        x = pool.cpu()[pg, :, inpage]                 # [B][n][H][...]
        x = x * okm.view(*okm.shape, *([1] * (x.dim() - 2))).to(x.dtype)
        return x.transpose(1, 2).contiguous()         # [B][H][n][...]

    class Dense:
        pass

    d = Dense()
    d.k_codes = take(pc.k_codes, pg_c, k % cpp, ok_c)
    d.v_codes = take(pc.v_codes, pg_c, k % cpp, ok_c)
    d.k_meta = take(pc.k_meta, pg_g, j % gpp, ok_g)
    d.v_meta = take(pc.v_meta, pg_c, k % cpp, ok_c)
    d.k_res, d.v_res = pc.k_res.cpu(), pc.v_res.cpu()
    d.tensors = lambda: (d.k_codes, d.v_codes, d.k_meta, d.v_meta, d.k_res, d.v_res)
    return d


def _paged_prefill(pc, k, v, lens):
    for b, n in enumerate(np.asarray(lens).tolist()):
        sub = pc.view(b, b + 1)
        kvq.kvq_paged_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)


def _pages_needed(lens, R, P):
    return [max(1, -(-oracle.packed_len(int(n), R) // P)) for n in lens]


def _decode_paged(g, pc, q, lens, scale):
    msl = int(np.max(lens))
    out = torch.empty((g.batch, g.n_q_heads, g.head_dim), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_paged_workspace(g, 1, msl)
    kvq.kvq_paged_decode_attn(g, dev(q), pc, dev(np.asarray(lens, np.int32)), msl, scale, ws, out)
    torch.cuda.synchronize()
    return out


def _decode_dense(g, cache, q, lens, scale):
    msl = int(np.max(lens))
    out = torch.empty((g.batch, g.n_q_heads, g.head_dim), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_workspace(g, msl)
    kvq.kvq_decode_attn(g, dev(q), cache, dev(np.asarray(lens, np.int32)), msl, scale, ws, out)
    torch.cuda.synchronize()
    return out


def _same_workers(g, msl):
    return kvq.kvq_paged_decode_workspace_bytes(g, 1, msl) == \
        kvq.kvq_decode_workspace_bytes(g, msl)


CASES = [
    # (B, Hq, Hkv, D, bK, bV, G, R, C, P, lens)
    (3, 8, 2, 128, 2, 4, 32, 128, 1024, 128, [1000, 129, 640]),
    (4, 4, 1, 64, 4, 2, 64, 64, 512, 64, [512, 65, 300, 128]),
    (2, 16, 2, 128, 4, 4, 128, 128, 2048, 256, [2048, 1500]),
    (3, 2, 2, 64, 2, 2, 32, 32, 256, 32, [256, 33, 100]),
    (2, 32, 8, 128, 2, 4, 32, 128, 1024, 1024, [1024, 700]),
    (2, 8, 2, 128, 8, 8, 32, 64, 512, 64, [500, 200]),
    (3, 4, 2, 64, 8, 2, 64, 64, 256, 64, [256, 100, 65]),
]


def _inputs(rng, B, Hkv, D, n, Hq):
    k = (rng.standard_normal((B, Hkv, n, D)) *
         rng.lognormal(0, 0.5, (1, Hkv, 1, D))).astype(np.float16)
    v = rng.standard_normal((B, Hkv, n, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    return k, v, q


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"D{c[3]}K{c[4]}V{c[5]}G{c[6]}R{c[7]}P{c[9]}")
def test_paged_prefill_and_decode(case):
    B, Hq, Hkv, D, bK, bV, G, R, C, P, lens = case
    _say(f"paged prefill+decode {case}")
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(sum(lens) + P)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq)
    maxp = -(-C // P)
    table, npages = _table(rng, B, maxp, _pages_needed(lens, R, P))
    pc = kvq.PagedCache(g, P, npages, dev(table))
    _paged_prefill(pc, k, v, lens)
    cache, oc = prefill_both(g, og, k, v, lens)
    assert_cache_equal(_gather(pc, table, g), oc, lens, what="paged prefill")
    scale = 1.0 / math.sqrt(D)
    out = _decode_paged(g, pc, q, lens, scale)
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), float(np.float32(scale)))
    assert_close(out, ref, what="paged decode")
    # the two phases called apart give the same bits
    out2 = torch.empty_like(out)
    ws = kvq.alloc_paged_workspace(g, 1, max(lens))
    ld = dev(np.asarray(lens, np.int32))
    kvq.kvq_paged_decode_partial(g, dev(q), pc, ld, max(lens), scale, ws, out2)
    kvq.kvq_paged_decode_combine(g, dev(q), pc, ld, max(lens), scale, ws, out2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    if _same_workers(g, max(lens)):
        dense = _decode_dense(g, cache, q, lens, scale)
        assert torch.equal(out.view(torch.int16), dense.view(torch.int16))


def test_paged_append_across_flushes_and_pages():
    """Decode steps of ragged sequences over several flushes (R = 64) and page
    boundaries (P = 64): every step's append, then attention; the final packed
    state bit-exact."""
    B, Hq, Hkv, D, bK, bV, G, R, C, P = 3, 8, 2, 128, 2, 4, 32, 64, 512, 64
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(21)
    lens0 = np.array([60, 128, 1], np.int32)
    steps = 140
    final = lens0 + steps
    k, v, _ = _inputs(rng, B, Hkv, D, int(final.max()), Hq)
    table, npages = _table(rng, B, C // P, _pages_needed(final, R, P), spare=5)
    _say(f"paged append lens0 {lens0.tolist()} steps {steps}")
    pc = kvq.PagedCache(g, P, npages, dev(table))
    _paged_prefill(pc, k, v, lens0)
    _, oc = prefill_both(g, og, k, v, lens0)
    lens = lens0.copy()
    scale = 1.0 / math.sqrt(D)
    for s in range(steps):
        kn = np.ascontiguousarray(k[np.arange(B), :, lens])   # [B][Hkv][D]
        vn = np.ascontiguousarray(v[np.arange(B), :, lens])
        kvq.kvq_paged_append(g, dev(kn), dev(vn), dev(lens), pc)
        oracle.append(og, oc, kn, vn, lens)
        lens = lens + 1
        if s % 35 == 34 or s == steps - 1:
            q = rng.standard_normal((B, Hq, D)).astype(np.float16)
            out = _decode_paged(g, pc, q, lens, scale)
            ref = oracle.decode_attn(og, oc, q, lens, float(np.float32(scale)))
            assert_close(out, ref, what=f"paged step {s}")
    assert_cache_equal(_gather(pc, table, g), oc, lens, what="paged append")


def test_paged_multi_token():
    B, Hq, Hkv, D, bK, bV, G, R, C, P, T = 3, 8, 2, 128, 2, 4, 32, 128, 1024, 128, 4
    lens = [131, 900, 4]
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(22)
    k, v, _ = _inputs(rng, B, Hkv, D, max(lens), Hq)
    q = rng.standard_normal((B, T, Hq, D)).astype(np.float16)
    table, npages = _table(rng, B, C // P, _pages_needed(lens, R, P))
    _say(f"paged multi T={T} lens {lens}")
    pc = kvq.PagedCache(g, P, npages, dev(table))
    _paged_prefill(pc, k, v, lens)
    _, oc = prefill_both(g, og, k, v, lens)
    out = torch.empty((B, T, Hq, D), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_paged_workspace(g, T, max(lens))
    kvq.kvq_paged_decode_attn_multi(g, dev(q), pc, dev(np.asarray(lens, np.int32)), T, max(lens),
                                    0.125, ws, out)
    torch.cuda.synchronize()
    ref = oracle.decode_attn_multi(og, oc, q, np.asarray(lens, np.int32), T, 0.125)
    assert_close(out, ref, what="paged T=4")


def test_paged_shared_prefix_pages():
    """Two sequences whose first 512 positions are the same tokens read the
    same pool pages for them (the second's table row repeats the first's)."""
    B, Hq, Hkv, D, bK, bV, G, R, C, P = 2, 8, 2, 128, 2, 4, 32, 128, 1024, 128
    lens = [900, 700]
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(23)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq)
    k[1, :, :512], v[1, :, :512] = k[0, :, :512], v[0, :, :512]
    table, npages = _table(rng, B, C // P, _pages_needed(lens, R, P), shared=(0, 1, 512 // P))
    _say(f"paged shared prefix {table.tolist()}")
    pc = kvq.PagedCache(g, P, npages, dev(table))
    _paged_prefill(pc, k, v, lens)  # sequence 1 rewrites the shared pages with the same bits
    _, oc = prefill_both(g, og, k, v, lens)
    assert_cache_equal(_gather(pc, table, g), oc, lens, what="shared prefix")
    out = _decode_paged(g, pc, q, lens, 0.125)
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), 0.125)
    assert_close(out, ref, what="shared prefix decode")


def test_paged_table_entry_outside_pool():
    """A read table entry outside [0, num_pages) gives NaN for its sequence
    only (page 0 is read in its place, nothing outside the pools); the writers
    skip that page."""
    B, Hq, Hkv, D, bK, bV, G, R, C, P = 3, 4, 2, 64, 2, 2, 32, 32, 256, 32
    lens = [200, 200, 200]
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(24)
    k, v, q = _inputs(rng, B, Hkv, D, max(lens), Hq)
    table, npages = _table(rng, B, C // P, _pages_needed(lens, R, P))
    table[1, 2] = npages + 7
    _say(f"paged bad entry {table[1].tolist()} of {npages}")
    pc = kvq.PagedCache(g, P, npages, dev(table))
    _paged_prefill(pc, k, v, lens)
    _, oc = prefill_both(g, og, k, v, lens)
    out = _decode_paged(g, pc, q, lens, 0.125).float().cpu().numpy()
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), 0.125)
    assert np.all(np.isnan(out[1]))
    assert_close(out[[0, 2]], ref[[0, 2]], what="other sequences")


def test_paged_equals_dense_full_size():
    """The Llama-3-8B-shaped layer at 32 x 8192 (K2/V4, G32, R128) in pages of
    128 positions handed out in shuffled order: one decode step over the pages
    equals the dense cache's bit for bit (same worker grid), or is within the
    tolerance of it otherwise."""
    w = synth.WORKLOADS[3]
    lens = synth.seq_lens(w)
    B, n = w.batch, int(lens.max())
    C = synth.capacity_for(w, int(lens.max()))
    P = 128
    g = kvq.Geom(B, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits, w.group,
                 w.residual, C)
    rng = np.random.default_rng(25)
    table, npages = _table(rng, B, C // P, _pages_needed(lens, w.residual, P), spare=11)
    _say(f"paged full size B={B} n={n} pages={npages}")
    kd = torch.from_numpy(synth.keys(w, n, batch=B)).cuda()
    vd = torch.from_numpy(synth.values(w, n, batch=B)).cuda()
    q = rng.standard_normal((B, w.n_q_heads, w.head_dim)).astype(np.float16)
    pc = kvq.PagedCache(g, P, npages, dev(table))
    cache = kvq.Cache(g)
    assert np.all(lens == n)
    kvq.kvq_paged_prefill(g, kd, vd, n, pc)
    kvq.kvq_prefill(g, kd, vd, n, cache)
    del kd, vd
    scale = 1.0 / math.sqrt(w.head_dim)
    out = _decode_paged(g, pc, q, lens, scale)
    dense = _decode_dense(g, cache, q, lens, scale)
    if _same_workers(g, n):
        assert torch.equal(out.view(torch.int16), dense.view(torch.int16))
    else:
        assert_close(out, dense.float().cpu().numpy().astype(np.float64), what="paged vs dense")


def test_paged_table_window_moves():
    """Pages of 32 positions and shares of more than 64 chunks per worker wave:
    the wave's 64-entry window of its table row must move on inside a share.
    4 sequences x 2 KV heads x 2^21 positions (inputs drawn on the device with
    a seeded generator); decode over the pages equals decode over the dense
    cache."""
    B, Hq, Hkv, D, bK, bV, G, R, P = 4, 16, 2, 64, 2, 2, 32, 128, 32
    n = 1 << 21
    g = kvq.Geom(B, Hq, Hkv, D, bK, bV, G, R, n)
    gq = Hq // Hkv
    workers = kvq.kvq_paged_decode_workspace_bytes(g, 1, n) // (gq * (D + 4) * 4) - B * Hkv
    per_wave = B * Hkv * (oracle.packed_len(n, R) // 32) / workers
    assert per_wave > 80, f"{per_wave} chunks per wave: the window would not move"
    rng = np.random.default_rng(26)
    table, npages = _table(rng, B, n // P, _pages_needed([n] * B, R, P), spare=9)
    _say(f"paged window: {workers} workers, {per_wave:.0f} chunks each, {npages} pages")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(26)
    kd = torch.randn((B, Hkv, n, D), generator=gen, device="cuda", dtype=torch.float16)
    vd = torch.randn((B, Hkv, n, D), generator=gen, device="cuda", dtype=torch.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    pc = kvq.PagedCache(g, P, npages, dev(table))
    cache = kvq.Cache(g)
    kvq.kvq_paged_prefill(g, kd, vd, n, pc)
    kvq.kvq_prefill(g, kd, vd, n, cache)
    del kd, vd
    lens = np.full(B, n, np.int32)
    out = _decode_paged(g, pc, q, lens, 0.125)
    dense = _decode_dense(g, cache, q, lens, 0.125)
    assert torch.isfinite(out.float()).all()
    if _same_workers(g, n):
        assert torch.equal(out.view(torch.int16), dense.view(torch.int16))
    else:
        assert_close(out, dense.float().cpu().numpy().astype(np.float64), what="paged vs dense")
