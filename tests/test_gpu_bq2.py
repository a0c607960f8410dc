"""GPU parity of the rotated per-token 2-bit format (KV1's BQ2_0) against the
CPU oracle, through the C ABI.

Stored state (codes of every quantized position, their (d, m), the fp16
sinks) must match the oracle bit for bit; outputs must satisfy
|gpu - oracle| <= 1e-3 * (1 + |oracle|) elementwise.  Sizes span several
32-position chunks with ragged tails, the sink boundary (n = 1..5), more than
64 sequences, and the KV1-shaped workload at full size on sampled sequences.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq
from quantized_decode_attention_amd import synth

from kvq_testutil import assert_close, dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _geoms(B, Hq, Hkv, C):
    return kvq.Bq2Geom(B, Hq, Hkv, C), oracle.Bq2Geom(B, Hq, Hkv, C)


def _host(cache: kvq.Bq2Cache, like: oracle.Bq2Cache):
    torch.cuda.synchronize()
    return [t.cpu().numpy().view(o.dtype).reshape(o.shape)
            for t, o in zip(cache.tensors(), like.arrays())]


def _assert_state(g, og, cache, oc, lens, what=""):
    """Positions [4, n) (codes, meta) and sinks [0, min(n, 4)) bit-exact."""
    got = oracle.Bq2Cache(og)
    for dst, src in zip(got.arrays(), _host(cache, oc)):
        dst[...] = src
    gk, gv = oracle.bq2_unpack(og, got)
    ok, ov = oracle.bq2_unpack(og, oc)
    for b, n in enumerate(np.asarray(lens).tolist()):
        s = min(n, 4)
        for name, x, y in (("k_code", gk, ok), ("v_code", gv, ov),
                           ("k_meta", got.k_meta, oc.k_meta), ("v_meta", got.v_meta, oc.v_meta)):
            bad = np.argwhere(x[b, :, 4:n] != y[b, :, 4:n])
            assert bad.size == 0, f"{what} seq {b} {name}: {len(bad)} mismatches, first {bad[0]}"
        assert np.array_equal(got.k_sink[b, :, :s], oc.k_sink[b, :, :s]), f"{what} seq {b} k_sink"
        assert np.array_equal(got.v_sink[b, :, :, :s], oc.v_sink[b, :, :, :s]), \
            f"{what} seq {b} v_sink"


def _prefill_both(g, og, k, v, lens):
    cache = kvq.Bq2Cache(g)
    oc = oracle.Bq2Cache(og)
    lens = np.asarray(lens).tolist()
    for b, n in enumerate(lens):
        if n == 0:
            continue
        g1 = kvq.Bq2Geom(1, g.n_q_heads, g.n_kv_heads, g.capacity)
        sub = kvq.Bq2Cache.__new__(kvq.Bq2Cache)
        sub.g = g1
        for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_sink", "v_sink"):
            setattr(sub, name, getattr(cache, name)[b:b + 1])
        kvq.kvq_bq2_prefill(g1, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        og1 = oracle.Bq2Geom(1, og.n_q_heads, og.n_kv_heads, og.capacity)
        c1 = oracle.Bq2Cache(og1)
        oracle.bq2_prefill(og1, c1, k[b:b + 1], v[b:b + 1], n)
        for dst, src in zip(oc.arrays(), c1.arrays()):
            dst[b] = src[0]
    return cache, oc


def _decode_both(g, og, cache, oc, q, lens, max_seq_len=None, scale=0.125):
    lens = np.asarray(lens, np.int32)
    msl = int(lens.max()) if max_seq_len is None else max_seq_len
    out = torch.empty((g.batch, g.n_q_heads, 64), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_bq2_workspace(g, msl)
    kvq.kvq_bq2_decode_attn(g, dev(q), cache, dev(lens), msl, scale, ws, out)
    torch.cuda.synchronize()
    ref = oracle.bq2_decode_attn(og, oc, q, lens, float(np.float32(scale)))
    return out, ref


def _inputs(B, Hkv, Hq, n, seed, kscale=2.0):
    gen = np.random.default_rng(seed)
    k = (gen.standard_normal((B, Hkv, n, 64)) * kscale).astype(np.float16)
    v = gen.standard_normal((B, Hkv, n, 64)).astype(np.float16)
    q = gen.standard_normal((B, Hq, 64)).astype(np.float16)
    return k, v, q


@pytest.mark.parametrize("lens", [[1, 3], [4, 5], [31, 32], [33, 100], [257, 64]])
def test_prefill_state(lens):
    C = 288
    g, og = _geoms(2, 8, 2, C)
    k, v, _ = _inputs(2, 2, 8, max(lens), 1)
    _say(f"bq2 prefill lens {lens}")
    cache, oc = _prefill_both(g, og, k, v, lens)
    _assert_state(g, og, cache, oc, lens, "prefill")


def test_appends_through_chunks_and_sinks():
    """Appends from empty through the sinks and two chunk boundaries, state
    and outputs checked along the way (decode after each append)."""
    C = 96
    g, og = _geoms(3, 8, 2, C)
    gen = np.random.default_rng(2)
    cache = kvq.Bq2Cache(g)
    oc = oracle.Bq2Cache(og)
    start = np.array([0, 2, 27], np.int32)
    n_steps = 40
    kk = (gen.standard_normal((3, 2, C, 64)) * 3).astype(np.float16)
    vv = gen.standard_normal((3, 2, C, 64)).astype(np.float16)
    for b, n in enumerate(start.tolist()):
        if n:
            g1, og1 = _geoms(1, 8, 2, C)
            c1 = oracle.Bq2Cache(og1)
            oracle.bq2_prefill(og1, c1, kk[b:b + 1], vv[b:b + 1], n)
            for dst, src in zip(oc.arrays(), c1.arrays()):
                dst[b] = src[0]
            sub = kvq.Bq2Cache.__new__(kvq.Bq2Cache)
            sub.g = g1
            for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_sink", "v_sink"):
                setattr(sub, name, getattr(cache, name)[b:b + 1])
            kvq.kvq_bq2_prefill(g1, dev(kk[b:b + 1, :, :n]), dev(vv[b:b + 1, :, :n]), n, sub)
    lens = start.copy()
    for step in range(n_steps):
        kn = np.stack([kk[b, :, lens[b]] for b in range(3)])
        vn = np.stack([vv[b, :, lens[b]] for b in range(3)])
        kvq.kvq_bq2_append(g, dev(kn), dev(vn), dev(lens), cache)
        oracle.bq2_append(og, oc, kn, vn, lens)
        lens = lens + 1
        if step % 7 == 0 or step == n_steps - 1:
            q = gen.standard_normal((3, 8, 64)).astype(np.float16)
            out, ref = _decode_both(g, og, cache, oc, q, lens)
            assert_close(out, ref, what=f"append step {step} lens {lens.tolist()}")
    _assert_state(g, og, cache, oc, lens, "append")


@pytest.mark.parametrize("gq", [1, 2, 4])
def test_decode_ragged_lengths(gq):
    lens = [1, 2, 3, 4, 5, 31, 32, 33, 64, 65, 100, 191, 200, 257]
    B, Hkv = len(lens), 2
    Hq = gq * Hkv
    C = 288
    g, og = _geoms(B, Hq, Hkv, C)
    k, v, q = _inputs(B, Hkv, Hq, max(lens), 10 + gq)
    _say(f"bq2 decode gq {gq} lens {lens}")
    cache, oc = _prefill_both(g, og, k, v, lens)
    out, ref = _decode_both(g, og, cache, oc, q, lens, scale=1 / 8)
    assert_close(out, ref, what=f"gq {gq}")


def test_decode_batch_beyond_one_wave_and_max_len():
    """70 sequences (the work scan spans two 64-lane passes), max_seq_len
    above every length, a large softmax scale."""
    B, Hkv, Hq = 70, 1, 4
    gen = np.random.default_rng(20)
    lens = gen.integers(1, 150, size=B).astype(np.int32)
    g, og = _geoms(B, Hq, Hkv, 192)
    k, v, q = _inputs(B, Hkv, Hq, int(lens.max()), 21)
    cache, oc = _prefill_both(g, og, k, v, lens)
    out, ref = _decode_both(g, og, cache, oc, q, lens, max_seq_len=190, scale=0.5)
    assert_close(out, ref, what="B=70")


def test_zero_and_invalid_lengths():
    g, og = _geoms(4, 4, 1, 64)
    k, v, q = _inputs(4, 1, 4, 40, 30)
    lens = np.array([40, 0, 7, -3], np.int32)
    cache, oc = _prefill_both(g, og, k, v, np.maximum(lens, 0))
    out = torch.empty((4, 4, 64), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_bq2_workspace(g, 40)
    kvq.kvq_bq2_decode_attn(g, dev(q), cache, dev(lens), 40, 0.125, ws, out)
    o = out.float().cpu().numpy()
    ref = oracle.bq2_decode_attn(og, oc, q, np.maximum(lens, 0), float(np.float32(0.125)))
    assert_close(o[[0, 2]], ref[[0, 2]], what="valid rows")
    assert np.all(o[1] == 0)
    assert np.all(np.isnan(o[3]))


def test_deterministic():
    g, og = _geoms(2, 8, 2, 160)
    k, v, q = _inputs(2, 2, 8, 150, 40)
    cache, oc = _prefill_both(g, og, k, v, [150, 77])
    ws = kvq.alloc_bq2_workspace(g, 150)
    outs = []
    for _ in range(2):
        out = torch.empty((2, 8, 64), dtype=torch.float16, device="cuda")
        kvq.kvq_bq2_decode_attn(g, dev(q), cache, dev(np.array([150, 77], np.int32)), 150,
                                0.125, ws, out)
        outs.append(out.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_full_size_kv1_workload():
    """The KV1-shaped layer at its full batch and 32K context, as bench.py
    runs it: prefill of n - 1 positions, one append, one decode; sampled
    sequences recomputed by the oracle."""
    w = synth.WORKLOADS[6]
    n = w.context
    C = synth.capacity_for(w)
    g = kvq.Bq2Geom(w.batch, w.n_q_heads, w.n_kv_heads, C)
    _say(f"bq2 full size: B {w.batch}, n {n}, workers {kvq.kvq_bq2_decode_workers(g)}")
    k = synth.keys(w, n - 1)
    v = synth.values(w, n - 1)
    kn, vn, q = synth.step_token(w, 0)
    cache = kvq.Bq2Cache(g)
    kvq.kvq_bq2_prefill(g, dev(k), dev(v), n - 1, cache)
    kvq.kvq_bq2_append(g, dev(kn), dev(vn), dev(np.full(w.batch, n - 1, np.int32)), cache)
    out = torch.empty((w.batch, w.n_q_heads, 64), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_bq2_workspace(g, n)
    scale = 1.0 / math.sqrt(64)
    kvq.kvq_bq2_decode_attn(g, dev(q), cache, dev(np.full(w.batch, n, np.int32)), n, scale,
                            ws, out)
    o = out.float().cpu().numpy()
    og_full = oracle.Bq2Geom(w.batch, w.n_q_heads, w.n_kv_heads, C)
    host = _host(cache, oracle.Bq2Cache(og_full))
    for b in (0, 7, 15):
        _say(f"  oracle sequence {b}")
        og = oracle.Bq2Geom(1, w.n_q_heads, w.n_kv_heads, C)
        oc = oracle.Bq2Cache(og)
        oracle.bq2_prefill(og, oc, k[b:b + 1], v[b:b + 1], n - 1)
        oracle.bq2_append(og, oc, kn[b:b + 1], vn[b:b + 1], np.array([n - 1], np.int32))
        got = oracle.Bq2Cache(og)
        for dst, src in zip(got.arrays(), host):
            dst[...] = src[b:b + 1]
        _assert_state(og, og, _HostCache(got), oc, [n], f"full seq {b}")
        ref = oracle.bq2_decode_attn(og, oc, q[b:b + 1], np.array([n], np.int32),
                                     float(np.float32(scale)))
        err = assert_close(o[b:b + 1], ref, what=f"full seq {b}")
        _say(f"    max err {err:.2e}")


class _HostCache:
    """A host copy shaped like a device cache for _assert_state."""

    def __init__(self, c):
        self._c = c

    def tensors(self):
        return [torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32))
                for a in self._c.arrays()]
