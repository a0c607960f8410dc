"""Pins of the oracle for the rotated per-token 2-bit format (KV1's BQ2_0).

Each test ties the oracle to something other than itself: scipy's Hadamard
matrix, exact rational sums, a numpy transcription of the quantize formula
printed in the KV1 model card ("Quantization Format: KV1.cpp BQ2_0"), worked
examples derived by hand (tests/golden/bq2_worked_examples.txt), the card's
"Memory" table, and attention written independently in numpy and torch with
the rotation undone.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from quantized_decode_attention_amd import metrics, synth

HERE = os.path.dirname(os.path.abspath(__file__))
H_REF = scipy.linalg.hadamard(64).astype(np.float64) / 8.0


def _f16(gen, shape, scale=1.0):
    return (gen.standard_normal(size=shape) * scale).astype(np.float16)


# ---------------------------------------------------------------- rotation --
def test_hadamard_is_scipy_sylvester_normalized():
    H = oracle.bq2_hadamard()
    assert np.array_equal(H, H_REF)
    assert np.array_equal(H @ H, np.eye(64))  # H H = I (exact in fp64)


def test_rotation_is_exact_product_rounded_once():
    gen = np.random.default_rng(1)
    # mixed magnitudes so that the sum spans many binades
    x = _f16(gen, (40, 64))
    x[:10] *= np.float16(300.0)
    x[10:20, ::3] = np.float16(1e-5)
    x[20, :] = np.float16(65504.0 / 16)
    got = oracle.bq2_rotate(x)
    ref = (H_REF @ x.astype(np.float64).T).T.astype(np.float32)
    assert np.array_equal(got, ref)
    # the fp64 sum is exact: compare two rows with rational arithmetic
    for r in (0, 21):
        for c in (0, 17, 63):
            exact = sum(Fraction(float(H_REF[c, j])) * Fraction(float(x[r, j])) for j in range(64))
            assert got[r, c] == np.float32(float(exact))


def test_rotation_preserves_dot_products():
    gen = np.random.default_rng(2)
    q = _f16(gen, (64,))
    k = _f16(gen, (64,))
    qr = H_REF @ q.astype(np.float64)
    kr = H_REF @ k.astype(np.float64)
    assert math.isclose(qr @ kr, q.astype(np.float64) @ k.astype(np.float64), rel_tol=1e-12,
                        abs_tol=1e-12)


# --------------------------------------------------------------- quantizer --
def _page_formula(x):
    """Literal numpy transcription of the card's quantize step (fp32), with
    the reading that a zero min is stored as +0."""
    x = np.asarray(x, np.float32)
    mn, mx = x.min(), x.max()
    if mn == 0:
        mn = np.float32(0.0)
    d = np.float16(max(np.float32((mx - mn) / np.float32(3.0)), np.float32(1e-6)))
    m = np.float16(mn)
    q = np.clip(np.rint((x - np.float32(m)) / np.float32(d)), 0, 3).astype(np.uint8)
    return int(d.view(np.uint16)), int(m.view(np.uint16)), q


def test_quantizer_matches_page_formula_on_rotated_synthetic_blocks():
    w = synth.WORKLOADS[6]
    k = synth.keys(w, 64, batch=2)
    v = synth.values(w, 64, batch=2)
    blocks = np.concatenate([oracle.bq2_rotate(k).reshape(-1, 64),
                             oracle.bq2_rotate(v).reshape(-1, 64)])
    gen = np.random.default_rng(3)
    extra = [np.full(64, 0.25, np.float32), np.full(64, -0.0, np.float32),
             np.linspace(-1e-7, 1e-7, 64, dtype=np.float32),          # below the floor
             (gen.standard_normal(64) * 1e-3).astype(np.float32),
             (gen.standard_normal(64) * 500).astype(np.float32)]
    for x in list(blocks) + extra:
        assert oracle.bq2_quantize(x)[:2] == _page_formula(x)[:2]
        assert np.array_equal(oracle.bq2_quantize(x)[2], _page_formula(x)[2])


def test_quantizer_picks_nearest_grid_point():
    """Brute force in exact rationals: each code is the nearest grid point
    (ties to even) of the fp32 quotient, clamped."""
    gen = np.random.default_rng(4)
    for _ in range(20):
        x = (gen.standard_normal(64) * gen.uniform(0.01, 10)).astype(np.float32)
        d, m, codes = oracle.bq2_quantize(x)
        df = float(np.uint16(d).view(np.float16))
        mf = float(np.uint16(m).view(np.float16))
        for c in range(64):
            y = np.float32(np.float32(x[c] - np.float32(mf)) / np.float32(df))
            fy = Fraction(float(y))
            if fy <= 0:
                best = 0
            elif fy >= 3:
                best = 3
            else:
                lo = math.floor(fy)
                frac = fy - lo
                if frac == Fraction(1, 2):
                    best = lo if lo % 2 == 0 else lo + 1
                else:
                    best = lo if frac < Fraction(1, 2) else lo + 1
            assert codes[c] == best


def test_reconstruction_bound():
    gen = np.random.default_rng(5)
    for _ in range(50):
        x = (gen.standard_normal(64) * gen.uniform(0.1, 20)).astype(np.float32)
        d, m, codes = oracle.bq2_quantize(x)
        df = float(np.uint16(d).view(np.float16))
        mf = float(np.uint16(m).view(np.float16))
        mn, mx = float(x.min()), float(x.max())
        d32 = max((mx - mn) / 3, 1e-6)
        xh = codes * df + mf
        # half a step, plus the clamp slack of an fp16-rounded d and min
        bound = df / 2 + 3 * abs(d32 - df) + abs(mn - mf) + 4 * np.spacing(np.abs(x))
        assert np.all(np.abs(x - xh) <= bound)


def _golden():
    rows = []
    with open(os.path.join(HERE, "golden", "bq2_worked_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, pattern, d, m, block = [s.strip() for s in line.split("|")]
            pat = np.array([float(t) for t in pattern.split()], np.float32)
            rows.append((name, np.tile(pat, 64 // pat.size), int(d, 16), int(m, 16),
                         bytes.fromhex(block)))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: r[0])
def test_worked_examples(row):
    _, x, d, m, block = row
    gd, gm, codes = oracle.bq2_quantize(x)
    assert (gd, gm) == (d, m)
    assert oracle.bq2_block(gd, gm, codes) == block


# ------------------------------------------------------------------ layout --
def test_cache_layout_holds_the_page_block_words():
    """A packed key word of lane group g is word g (little-endian) of the
    token's code bytes; values and meta as the layout states."""
    g = oracle.Bq2Geom(1, 4, 1, 64)
    gen = np.random.default_rng(6)
    k = _f16(gen, (1, 1, 64, 64))
    v = _f16(gen, (1, 1, 64, 64))
    c = oracle.Bq2Cache(g)
    oracle.bq2_prefill(g, c, k, v, 64)
    kr, vr = oracle.bq2_rotate(k), oracle.bq2_rotate(v)
    for t in range(4, 64):
        kd, km, kc = oracle.bq2_quantize(kr[0, 0, t])
        vd, vm, vc = oracle.bq2_quantize(vr[0, 0, t])
        assert tuple(c.k_meta[0, 0, t]) == (kd, km)
        assert tuple(c.v_meta[0, 0, t]) == (vd, vm)
        words = np.frombuffer(oracle.bq2_block(kd, km, kc)[4:], "<u4")
        tau = t % 32
        i, u = 4 * (tau // 8) + tau % 4, (tau // 4) % 2
        for gg in range(4):
            assert c.k_codes[0, 0, t // 32, 16 * gg + i, u] == words[gg]
        gv, j = tau // 8, tau % 8
        for ch in range(64):
            n, ii = ch // 16, ch % 16
            word = c.v_codes[0, 0, t // 32, 16 * gv + ii, n // 2]
            bit = 8 * (n % 2) + 2 * (j // 2) + 16 * (j % 2)
            assert (word >> bit) & 3 == vc[ch]
    for t in range(4):
        assert np.array_equal(c.k_sink[0, 0, t], kr[0, 0, t].astype(np.float16).view(np.uint16))
        assert np.array_equal(c.v_sink[0, 0, :, t], vr[0, 0, t].astype(np.float16).view(np.uint16))


def test_appends_equal_prefill():
    g = oracle.Bq2Geom(2, 8, 2, 96)
    gen = np.random.default_rng(7)
    n = 70
    k = _f16(gen, (2, 2, n, 64))
    v = _f16(gen, (2, 2, n, 64))
    a = oracle.Bq2Cache(g)
    oracle.bq2_prefill(g, a, k, v, n)
    b = oracle.Bq2Cache(g)
    for t in range(n):
        oracle.bq2_append(g, b, k[:, :, t], v[:, :, t], np.full(2, t, np.int32))
    for x, y in zip(a.arrays(), b.arrays()):
        assert np.array_equal(x, y)


# ------------------------------------------------------------------ memory --
def test_memory_table():
    """KV1 card, "Memory": 6 attention blocks x 8 KV heads, BQ2_0 1.9 KiB per
    token (2.5 bits/value), 15 MiB at 8K, 60 MiB at 32K; fp16 12 KiB, 96 and
    384 MiB."""
    per_tok = 6 * 8 * metrics.bq2_bytes_per_token()
    assert metrics.BQ2_BLOCK_BYTES * 8 / 64 == 2.5
    assert round(per_tok / 1024, 1) == 1.9
    assert per_tok * 8192 == 15 * 2**20
    assert per_tok * 32768 == 60 * 2**20
    fp16 = 6 * 8 * metrics.fp16_bytes_per_token(64)
    assert fp16 == 12 * 1024 and fp16 * 32768 == 384 * 2**20


# --------------------------------------------------------------- attention --
def _setup(B=2, Hq=8, Hkv=2, n=100, C=128, seed=8):
    g = oracle.Bq2Geom(B, Hq, Hkv, C)
    gen = np.random.default_rng(seed)
    k = _f16(gen, (B, Hkv, n, 64), 2.0)
    v = _f16(gen, (B, Hkv, n, 64))
    q = _f16(gen, (B, Hq, 64))
    c = oracle.Bq2Cache(g)
    oracle.bq2_prefill(g, c, k, v, n)
    return g, c, k, v, q


def test_attention_equals_unrotated_attention_numpy():
    """out = softmax(s q . K~) V~ with K~, V~ the cached rotated rows rotated
    back (H is its own inverse), on the unrotated query."""
    g, c, _, _, q = _setup()
    lens = np.array([100, 37], np.int32)
    scale = 0.125
    out = oracle.bq2_decode_attn(g, c, q, lens, scale)
    kr, vr = oracle.bq2_cache_kv(g, c, 100)
    kk = kr @ H_REF.T
    vv = vr @ H_REF.T
    G = g.n_q_heads // g.n_kv_heads
    for b in range(2):
        n = lens[b]
        for h in range(g.n_q_heads):
            qq = q[b, h].astype(np.float64)
            s = scale * kk[b, h // G, :n] @ qq
            p = np.exp(s - s.max())
            p /= p.sum()
            np.testing.assert_allclose(out[b, h], p @ vv[b, h // G, :n], rtol=0, atol=1e-12)


def test_attention_matches_torch_sdpa_in_rotated_domain():
    g, c, _, _, q = _setup(seed=9)
    lens = np.array([100, 100], np.int32)
    out = oracle.bq2_decode_attn(g, c, q, lens, 1 / 8)
    kr, vr = oracle.bq2_cache_kv(g, c, 100)
    G = g.n_q_heads // g.n_kv_heads
    qr = torch.from_numpy(q.astype(np.float64) @ H_REF.T)          # [B][Hq][64]
    K = torch.from_numpy(kr).repeat_interleave(G, dim=1)
    V = torch.from_numpy(vr).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qr[:, :, None], K, V, scale=1 / 8)
    ref = o[:, :, 0].numpy() @ H_REF.T
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_sinks_only_and_closed_forms():
    g, c, k, v, q = _setup(seed=10)
    # n = 1: the output is the first value (fp16 of its rotation, rotated back)
    o1 = oracle.bq2_decode_attn(g, c, q, np.array([1, 1], np.int32), 0.125)
    G = g.n_q_heads // g.n_kv_heads
    for b in range(2):
        for h in range(g.n_q_heads):
            np.testing.assert_allclose(o1[b, h], v[b, h // G, 0].astype(np.float64),
                                       rtol=2e-3, atol=2e-3)
    # n <= 4 is unquantized attention up to the fp16 rounding of the rotation
    o4 = oracle.bq2_decode_attn(g, c, q, np.array([4, 3], np.int32), 0.125)
    for b, n in enumerate((4, 3)):
        for h in range(g.n_q_heads):
            kk = k[b, h // G, :n].astype(np.float64)
            s = 0.125 * kk @ q[b, h].astype(np.float64)
            p = np.exp(s - s.max())
            p /= p.sum()
            np.testing.assert_allclose(o4[b, h], p @ v[b, h // G, :n].astype(np.float64),
                                       rtol=0, atol=5e-3)
    # q = 0: uniform weights, the output is the mean of the cached values
    o0 = oracle.bq2_decode_attn(g, c, np.zeros_like(q), np.array([100, 50], np.int32), 0.125)
    kr, vr = oracle.bq2_cache_kv(g, c, 100)
    for b, n in enumerate((100, 50)):
        ref = vr[b, :, :n].mean(axis=1) @ H_REF.T
        for h in range(g.n_q_heads):
            np.testing.assert_allclose(o0[b, h], ref[h // G], rtol=0, atol=1e-12)


def test_dequantized_cache_is_close_to_the_rotated_inputs():
    g, c, k, v, _ = _setup(seed=11)
    kr, vr = oracle.bq2_cache_kv(g, c, 100)
    for cached, meta, src in ((kr, c.k_meta, k), (vr, c.v_meta, v)):
        rot = oracle.bq2_rotate(src).astype(np.float64)
        for b in range(2):
            for h in range(2):
                for t in range(4, 100):
                    x = rot[b, h, t]
                    d16 = float(meta[b, h, t, 0:1].view(np.float16)[0])
                    m16 = float(meta[b, h, t, 1:2].view(np.float16)[0])
                    d32 = max((x.max() - x.min()) / 3, 1e-6)
                    bound = d16 / 2 + 3 * abs(d32 - d16) + abs(x.min() - m16) + 1e-6
                    assert np.all(np.abs(cached[b, h, t] - x) <= bound)
