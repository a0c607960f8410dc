"""GPU parity: libkvq (through its C ABI) against the CPU oracle.

Packed codes, scales and mins must match bit for bit; attention outputs within
|gpu - oracle| <= 1e-3 * (1 + |oracle|) elementwise.  Inputs are the seeded
synthetic workloads (quantized_decode_attention_amd.synth) plus hand-made edge
cases.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq
from quantized_decode_attention_amd import synth

from kvq_testutil import (assert_cache_equal, assert_close, decode_both, dev, geoms,
                          prefill_both)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# -------------------------------------------------------------- quantize ----
QUANT_CASES = [
    # D, bK, bV, G
    (64, 2, 2, 32), (64, 4, 4, 64), (128, 2, 4, 32), (128, 4, 2, 64),
    (128, 4, 4, 128), (128, 2, 2, 64), (64, 2, 4, 64), (128, 2, 2, 128),
    (64, 8, 8, 32), (128, 8, 4, 64), (128, 2, 8, 128), (128, 8, 2, 32),
]


def _edge_tensor(rng, B, H, n, D):
    """fp16 inputs with constant, all-zero (with -0), subnormal-range, huge and
    tie-prone groups mixed into normal data."""
    x = (rng.standard_normal((B, H, n, D)) * 2).astype(np.float16)
    x[0, 0, :32, 0:4] = np.float16(1.5)                      # constant key groups
    x[0, 0, 0:2, :] = np.float16(3.25)                       # constant value rows
    x[0, 0, 32:64, 4] = np.float16(-0.0)
    x[0, 0, 40:50, 4] = np.float16(0.0)                      # zero group with -0
    x[0, 0, 2, :] = np.float16(-0.0)
    sub = (rng.integers(0, 9, size=(32,)) * 2.0 ** -24).astype(np.float16)
    x[0, 0, 64:96, 5] = sub                                   # subnormal range
    x[0, 0, 3, :32] = (rng.integers(0, 5, size=32) * 2.0 ** -24).astype(np.float16)
    x[0, 0, 96:128, 6] = np.float16(60000.0)
    x[0, 0, 96, 6] = np.float16(-60000.0)                    # huge range
    x[0, 0, 4, :] = (np.arange(D) % 7 * 0.5).astype(np.float16)  # ties
    x[0, 0, 128:160, 7] = (np.arange(32) % 4 * 0.5 + 0.25).astype(np.float16)
    return x


@pytest.mark.parametrize("D,bK,bV,G", QUANT_CASES)
def test_quantize_bitexact(D, bK, bV, G):
    _say(f"quantize D={D} bK={bK} bV={bV} G={G}")
    B, H, n = 2, 2, 256
    C = 512
    g, og = geoms(B, 4, H, D, bK, bV, G, G, C)
    rng = np.random.default_rng(D * 100 + bK * 10 + bV + G)
    k = _edge_tensor(rng, B, H, n, D)
    v = _edge_tensor(rng, B, H, n, D)
    cache = kvq.Cache(g)
    oc = oracle.Cache(og)
    pos0 = 2 * G if 2 * G + n <= C else 0
    kvq.kvq_quantize_keys_perchannel(g, dev(k), pos0, cache.k_codes, cache.k_meta)
    kvq.kvq_quantize_values_pertoken(g, dev(v), pos0, cache.v_codes, cache.v_meta)
    oracle.quantize_keys(og, oc, k, pos0)
    oracle.quantize_values(og, oc, v, pos0)
    assert_cache_equal(cache, oc, what="quantize")


def test_quantize_synthetic_configs_bitexact():
    for cfg in (1, 2, 3, 4, 5):
        w = synth.WORKLOADS[cfg]
        B = min(w.batch, 2)
        n = 512
        _say(f"quantize synthetic cfg {cfg}")
        g, og = geoms(B, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                      w.group, w.residual, 512)
        k = synth.keys(w, n, batch=B)
        v = synth.values(w, n, batch=B)
        cache = kvq.Cache(g)
        oc = oracle.Cache(og)
        kvq.kvq_quantize_keys_perchannel(g, dev(k), 0, cache.k_codes, cache.k_meta)
        kvq.kvq_quantize_values_pertoken(g, dev(v), 0, cache.v_codes, cache.v_meta)
        oracle.quantize_keys(og, oc, k, 0)
        oracle.quantize_values(og, oc, v, 0)
        assert_cache_equal(cache, oc, what=f"cfg{cfg}")


# ---------------------------------------------------------------- decode ----
DECODE_CASES = [
    # B, Hq, Hkv, D, bK, bV, G, R, lens
    (1, 2, 2, 64, 2, 2, 32, 32, [256]),                   # tiny: B1, 2 heads, D64
    (2, 8, 8, 128, 2, 2, 32, 128, [1000, 700]),           # MHA
    (2, 32, 8, 128, 2, 4, 32, 128, [3000, 2177]),         # GQA 4, K2V4
    (2, 16, 8, 128, 2, 4, 32, 128, [2600, 1111]),         # GQA 2, D128 (8 columns per head)
    (3, 32, 8, 128, 2, 2, 64, 128, [5000, 129, 4097]),    # varlen, G64
    (2, 16, 8, 128, 4, 2, 64, 64, [4100, 4160]),          # K4V2 G64 R64
    (2, 16, 2, 64, 4, 4, 64, 64, [777, 64]),              # GQA 8, D64
    (1, 16, 1, 128, 2, 4, 128, 128, [1500]),              # GQA 16, G128
    (2, 4, 2, 64, 2, 2, 32, 32, [1, 32]),                 # all residual
    (4, 4, 2, 64, 2, 2, 32, 32, [33, 64, 65, 31]),        # R, R+1, 2R, 2R+1
    (2, 32, 8, 128, 8, 8, 32, 128, [3000, 2177]),         # 8-bit keys and values
    (2, 16, 2, 64, 8, 4, 64, 64, [777, 64]),              # K8V4, D64, GQA 8
    (3, 8, 2, 128, 4, 8, 128, 128, [1500, 129, 900]),     # K4V8, G128
    (1, 16, 1, 128, 8, 2, 32, 128, [2000]),               # K8V2, GQA 16
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_decode_parity(case):
    B, Hq, Hkv, D, bK, bV, G, R, lens = case
    _say(f"decode {case}")
    nmax = max(lens)
    C = (nmax // R + 2) * R
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(nmax + B)
    scl = rng.lognormal(0, 0.5, size=(1, Hkv, 1, D)).astype(np.float32)
    scl[..., :2] *= 12
    k = (rng.standard_normal((B, Hkv, nmax, D)).astype(np.float32) * scl).astype(np.float16)
    v = rng.standard_normal((B, Hkv, nmax, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    cache, oc = prefill_both(g, og, k, v, lens)
    assert_cache_equal(cache, oc, lens=lens, what="prefill")
    out, ref = decode_both(g, og, cache, oc, q, lens)
    err = assert_close(out, ref, what=f"decode {case}")
    _say(f"  max err {err:.2e}")


def test_decode_worker_boundaries():
    """Many short sequences (one wave's share spans several units) mixed with
    long ones (one unit spans many waves), lengths around chunk, group and
    window edges."""
    B, Hq, Hkv, D = 24, 8, 2, 128
    g0 = kvq.Geom(B, Hq, Hkv, D, 2, 4, 32, 128, 8192)
    nw = kvq.kvq_decode_workers(g0)
    _say(f"worker waves: {nw}")
    lens = [1, 31, 32, 33, 127, 128, 129, 160, 161, 255, 256, 257, 383, 384, 385,
            1000, 4095, 4096, 4097, 5000, 8000, 8191, 129, 300]
    g, og = geoms(B, Hq, Hkv, D, 2, 4, 32, 128, 8192)
    rng = np.random.default_rng(1)
    k = rng.standard_normal((B, Hkv, 8191, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, 8191, D)).astype(np.float16)
    q = (rng.standard_normal((B, Hq, D)) * 3).astype(np.float16)
    cache, oc = prefill_both(g, og, k, v, lens)
    out, ref = decode_both(g, og, cache, oc, q, lens, max_seq_len=8191)
    assert_close(out, ref, what="worker boundaries")


def test_decode_batch_beyond_one_wave():
    """More sequences than lanes in a wave (the work layout then spans
    several 64-sequence blocks), lengths mixed from 1 to a few windows."""
    B, Hq, Hkv, D = 70, 4, 2, 64
    rng = np.random.default_rng(70)
    lens = rng.integers(1, 300, size=B).astype(np.int32)
    lens[::9] = 1
    lens[5::11] = 64
    g, og = geoms(B, Hq, Hkv, D, 2, 2, 32, 32, 320)
    k = rng.standard_normal((B, Hkv, int(lens.max()), D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, int(lens.max()), D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    _say(f"batch {B}: lengths {int(lens.min())}..{int(lens.max())}")
    cache, oc = prefill_both(g, og, k, v, lens)
    out, ref = decode_both(g, og, cache, oc, q, lens)
    assert_close(out, ref, what="batch beyond one wave")


def test_decode_degenerate_lengths():
    """n = 0 -> zeros; n above max_seq_len -> NaN (no out-of-bounds reads)."""
    g, og = geoms(3, 4, 2, 64, 2, 2, 32, 32, 1024)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((3, 2, 600, 64)).astype(np.float16)
    v = rng.standard_normal((3, 2, 600, 64)).astype(np.float16)
    q = rng.standard_normal((3, 4, 64)).astype(np.float16)
    cache, oc = prefill_both(g, og, k, v, [600, 600, 600])
    for msl in (600, 1000):  # one split and several splits
        out = torch.empty((3, 4, 64), dtype=torch.float16, device="cuda")
        ws = kvq.alloc_workspace(g, msl)
        lens = np.array([0, 600, msl + 5], np.int32)
        kvq.kvq_decode_attn(g, dev(q), cache, dev(lens), msl, 0.125, ws, out)
        o = out.float().cpu().numpy()
        assert np.all(o[0] == 0)
        assert np.all(np.isnan(o[2]))
        ref = oracle.decode_attn(og, oc, q, np.array([0, 600, 0], np.int32), 0.125)
        assert_close(o[1], ref[1], what=f"degenerate msl={msl}")


def test_decode_deterministic():
    w = synth.WORKLOADS[3]
    B = 4
    g, og = geoms(B, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits, w.group,
                  w.residual, 2048)
    k = synth.keys(w, 2000, batch=B)
    v = synth.values(w, 2000, batch=B)
    q = dev(synth.queries(w, batch=B))
    cache = kvq.Cache(g)
    kvq.kvq_prefill(g, dev(k), dev(v), 2000, cache)
    lens = dev(np.full(B, 2000, np.int32))
    ws = kvq.alloc_workspace(g, 2000)
    outs = []
    for _ in range(2):
        out = torch.empty((B, w.n_q_heads, w.head_dim), dtype=torch.float16, device="cuda")
        kvq.kvq_decode_attn(g, q, cache, lens, 2000, 1 / math.sqrt(128), ws, out)
        outs.append(out.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


# ---------------------------------------------------------- append/flush ----
@pytest.mark.parametrize("bK,bV,G,R", [(2, 2, 32, 32), (2, 4, 32, 128), (4, 2, 64, 64),
                                      (8, 8, 32, 64), (8, 2, 64, 64)])
def test_append_flush_steps(bK, bV, G, R):
    """Several decode steps with appends crossing flushes at different steps per
    sequence: cache bit-exact and outputs within tolerance after every step."""
    B, Hq, Hkv, D = 3, 8, 2, 128
    _say(f"append bK={bK} bV={bV} G={G} R={R}")
    start = np.array([R - 2, 2 * R, 3 * R - 1], np.int32)
    steps = R + 4
    C = (int(start.max()) + steps) // R * R + 2 * R
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(R + bK)
    total = int(start.max()) + steps
    k = rng.standard_normal((B, Hkv, total, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, total, D)).astype(np.float16)
    cache, oc = prefill_both(g, og, k, v, start)
    lens = start.copy()
    ws = kvq.alloc_workspace(g, total)
    check_at = {0, 1, 2, R - 2, R - 1, R, R + 1, steps - 1}
    for step in range(steps):
        kn = np.ascontiguousarray(np.stack([k[b, :, lens[b]] for b in range(B)]))
        vn = np.ascontiguousarray(np.stack([v[b, :, lens[b]] for b in range(B)]))
        q = rng.standard_normal((B, Hq, D)).astype(np.float16)
        kvq.kvq_append(g, dev(kn), dev(vn), dev(lens), cache)
        oracle.append(og, oc, kn, vn, lens)
        lens = lens + 1
        out = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
        kvq.kvq_decode_attn(g, dev(q), cache, dev(lens), total, 1 / math.sqrt(D), ws, out)
        if step in check_at:
            assert_cache_equal(cache, oc, lens=lens, what=f"step {step}")
            ref = oracle.decode_attn(og, oc, q, lens, float(np.float32(1 / math.sqrt(D))))
            assert_close(out, ref, what=f"step {step}")


def test_append_out_of_range_is_noop():
    g, og = geoms(2, 2, 2, 64, 2, 2, 32, 32, 64)
    cache = kvq.Cache(g)
    before = [t.clone() for t in cache.tensors()]
    kn = dev(np.ones((2, 2, 64), np.float16))
    kvq.kvq_append(g, kn, kn, dev(np.array([64, -1], np.int32)), cache)
    torch.cuda.synchronize()
    for a, b in zip(before, cache.tensors()):
        assert torch.equal(a, b)


# ------------------------------------------------------------ error paths ---
def test_workspace_errors():
    g = kvq.Geom(4, 32, 8, 128, 2, 4, 32, 128, 65536)
    nw = kvq.kvq_decode_workers(g)
    assert nw >= 256
    need = kvq.kvq_decode_workspace_bytes(g, 65536)
    assert need == (nw + 4 * 8) * 4 * 132 * 4  # (workers + units) x GQ x (D + 4) floats
    cache = kvq.Cache(kvq.Geom(4, 32, 8, 128, 2, 4, 32, 128, 65536))
    q = torch.zeros((4, 32, 128), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    lens = torch.ones(4, dtype=torch.int32, device="cuda")
    small = torch.empty(need // 4 - 4, dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn(g, q, cache, lens, 65536, 0.1, small, out)
    assert e.value.status == -5
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn(g, q, cache, lens, 65537, 0.1, small, out)
    assert e.value.status == -6
