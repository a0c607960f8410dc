"""GPU parity on edge-valued caches, through the C ABI, against the CPU oracle.

The caches are built from inputs that reach the quantizer's degenerate and
extreme groups ([KV1] "Quantization Format: KV1.cpp BQ2_0": the scale is the
group's range over 2^b - 1 with fp16 scale and min; a zero scale gives code 0),
and the queries reach the decode kernel's per-head prescale from both ends.
Every batch holds one sequence per regime:

  0  degenerate groups: constant key channel groups (scale 0, the min carries
     the value; zero and -0 included), a whole constant key group, key groups
     whose range gives a subnormal fp16 scale (integers times 2^-24, values near
     1e-5, a normal min with a subnormal step); constant, zero, subnormal and
     partly constant value rows; queries N(0, 1).
  1  huge keys: key channel groups spanning [-60000, 60000] (scale 40000 at
     2 bits), others almost all 60000; query heads scaled by 1e-3, 0, 2^-20
     (fp16 subnormal) and 1e-3.
  2  huge values: on one token in 23, a value channel group spanning
     [-60000, 60000] (scale 40000 at 2 bits); queries N(0, 1).
  3  large and small queries: keys with lognormal channel scales and outlier
     channels (x12), query heads scaled by 100, 1e-3, 100 and 1.

Codes, scales, mins and window slots must match the oracle bit for bit, over
the whole of every cache buffer: the buffers start filled with a canary word
(an fp16 NaN pattern) on both sides, so a write outside what the oracle writes
shows up as a mismatch, and a stale window slot or unwritten group read by the
decode would turn the output into NaN.  Every buffer also sits between guard
bands that must keep the canary.  Outputs: |gpu - oracle| <= 1e-3 (1 + |oracle|)
elementwise.

Conditioning.  The tolerance presumes fp32 accumulation, so the inputs must
be ones on which fp32 accumulation can meet it.  Every test also runs a plain
fp32 implementation on the oracle's dequantized cache (sequential fp32 dot
products, fp32 exponentials, sequential fp32 weighted sum, fp16 output) and
requires it to pass too, which guards the inputs: with huge value groups on
a third of the tokens, say, an output is a sum of terms of 10^4 that cancels
to about 1, and that plain implementation itself misses the tolerance.  The
huge keys are paired with small queries and the x100 queries with ordinary
keys for the same reason: scores of 10^5 log2 units would leave no fp32
implementation within the tolerance.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq

from kvq_testutil import NAMES, assert_close, dev, geoms
from test_gpu_paged import _gather, _pages_needed, _table

pytestmark = pytest.mark.gpu

CANARY16 = 0x7E5A          # fp16 NaN with a payload
PAD = 256                  # guard elements on each side of every buffer


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------ edge inputs ----
def edge_kv(rng, B, Hkv, n, D, G, huge=60000.0):
    """fp16 keys and values [B][Hkv][n][D]; sequence b follows regime b % 4."""
    k = rng.standard_normal((B, Hkv, n, D)) * rng.lognormal(0, 0.5, (1, Hkv, 1, D))
    k[..., :2] *= 12.0
    v = rng.standard_normal((B, Hkv, n, D))
    for b in range(B):
        r = b % 4
        if r == 0:
            for j in range(n // G):            # key group j: tokens [jG, jG + G)
                t0, t1 = j * G, (j + 1) * G
                c = 2 + (5 * j) % (D - 8)
                k[b, :, t0:t1, c] = 1.5 * ((j % 3) - 1)               # constant, 0 included
                k[b, :, t0:t1, c + 1] = 0.0
                k[b, :, t0:t0 + G // 2, c + 1] = -0.0                # zero with -0
                k[b, :, t0:t1, c + 2] = rng.integers(0, 7, (Hkv, G)) * 2.0 ** -24
                k[b, :, t0:t1, c + 3] = 1e-5 * rng.standard_normal((Hkv, G))
                k[b, :, t0:t1, c + 4] = 2.0 ** -14 + rng.integers(0, 3, (Hkv, G)) * 2.0 ** -24
            if n >= 2 * G:
                k[b, :, G:2 * G, :] = 0.75                            # a whole constant group
            for t in range(n):
                m = t % 7
                if m == 1:
                    v[b, :, t, :] = 0.25 * (t % 5) - 0.5              # constant row
                elif m == 2:
                    v[b, :, t, :] = 0.0
                    v[b, :, t, ::2] = -0.0                            # zero row with -0
                elif m == 3:
                    v[b, :, t, :] = rng.integers(0, 9, (Hkv, D)) * 2.0 ** -24
                elif m == 4:
                    v[b, :, t, :G] = 3.0                              # one constant group
                elif m == 5:
                    v[b, :, t, :] = 1e-5 * rng.standard_normal((Hkv, D))
        elif r == 1:
            for j in range(-(-n // G)):
                t0, t1 = j * G, min(n, (j + 1) * G)
                c = 8 + j % 4
                k[b, :, t0:t1, c] = rng.uniform(-huge, huge, (Hkv, t1 - t0))
                k[b, :, t0, c] = -huge
                k[b, :, t1 - 1, c] = huge
                k[b, :, t0:t1, c + 8] = huge
                k[b, :, t0 + (j % (t1 - t0)), c + 8] = -huge
        elif r == 2:
            ng = D // G
            for t in range(n):
                if t % 23 == 5:
                    gm = (t // 23) % ng
                    v[b, :, t, gm * G:(gm + 1) * G] = rng.uniform(-huge, huge, (Hkv, G))
                    v[b, :, t, gm * G] = -huge
                    v[b, :, t, gm * G + 1] = huge
    return k.astype(np.float16), v.astype(np.float16)


Q_SCALES = {0: (1.0,), 1: (1e-3, 0.0, 2.0 ** -20, 1e-3), 2: (1.0,), 3: (100.0, 1e-3, 100.0, 1.0)}


def edge_q(rng, B, Hq, D, T=None):
    """fp16 queries [B][Hq][D] (or [B][T][Hq][D]); head h of sequence b is
    scaled by Q_SCALES[b % 4][h % 4]."""
    shape = (B, Hq, D) if T is None else (B, T, Hq, D)
    q = rng.standard_normal(shape)
    for b in range(B):
        sc = Q_SCALES[b % 4]
        for h in range(Hq):
            f = sc[h % len(sc)]
            if T is None:
                q[b, h] *= f
            else:
                q[b, :, h] *= f
    return q.astype(np.float16)


# --------------------------------------------- plain fp32 reference ----
def _seq_fp32_head(K, V, q, scale):
    """One head: sequential fp32 dot products over channels, fp32 softmax,
    sequential fp32 weighted sum over tokens, fp16 result (float64 array)."""
    f32 = np.float32
    s = np.zeros(K.shape[0], f32)
    for c in range(K.shape[1]):
        s = (s + K[:, c].astype(f32) * f32(q[c])).astype(f32)
    s = (s * f32(scale)).astype(f32)
    if s.size == 0:
        return np.zeros(V.shape[1])
    p = np.exp((s - s.max()).astype(f32)).astype(f32)
    acc = np.zeros(V.shape[1], f32)
    l = f32(0)
    for t in range(K.shape[0]):
        acc = (acc + p[t] * V[t].astype(f32)).astype(f32)
        l = f32(l + p[t])
    return (acc / l).astype(np.float16).astype(np.float64)


def fp32_reference(og, oc, q, lens, scale, T=1):
    """The plain fp32 implementation's outputs on the oracle's dequantized
    cache (same shape as the oracle's decode output)."""
    lens = np.asarray(lens)
    gq = og.n_q_heads // og.n_kv_heads
    out = np.zeros(q.shape)
    for b in range(q.shape[0]):
        # the cache as it represents sequence b's own positions
        K, V = oracle.cache_kv(og, oc, int(lens[b]))
        for i in range(T):
            vis = int(lens[b]) - T + 1 + i  # positions this query token sees
            for h in range(og.n_q_heads):
                qh = q[b, h] if T == 1 else q[b, i, h]
                o = _seq_fp32_head(K[b, h // gq, :vis], V[b, h // gq, :vis],
                                   qh.astype(np.float32), scale)
                if T == 1:
                    out[b, h] = o
                else:
                    out[b, i, h] = o
    return out


def assert_close_cond(got, ref, ref32, what, tol=1e-3):
    """|got - ref| <= tol (1 + |ref|) elementwise, after checking that the
    plain fp32 implementation ref32 meets the same bound on these inputs."""
    lim = tol * (1.0 + np.abs(ref))
    r32 = float(np.max(np.abs(ref32 - ref) / lim)) if ref.size else 0.0
    assert r32 <= 1.0, f"{what}: ill-conditioned input (plain fp32 at {r32:.2f} of the tolerance)"
    err = assert_close(got, ref, what=what, tol=tol)
    if isinstance(got, torch.Tensor):
        got = got.float().cpu().numpy()
    r = float(np.max(np.abs(got.astype(np.float64) - ref) / lim)) if ref.size else 0.0
    _say(f"  {what}: max err {err:.2e}, {r:.2f} of the tolerance (plain fp32 {r32:.2f})")


# ------------------------------------------------------- guarded buffers ----
class Guarded:
    """A device tensor of the given shape and dtype between two guard bands,
    all filled with the canary."""

    def __init__(self, shape, dtype):
        self.shape, self.dtype = tuple(shape), dtype
        es = torch.empty((), dtype=dtype).element_size()
        self.pad = PAD * 2 // es                        # PAD fp16-sized elements of guard
        n = int(np.prod(shape))
        self.raw = torch.empty(n + 2 * self.pad, dtype=dtype, device="cuda")
        self.raw.view(torch.int16).fill_(CANARY16)
        self.t = self.raw[self.pad:self.pad + n].view(self.shape)

    def check_guards(self, what):
        torch.cuda.synchronize()
        g16 = self.raw.view(torch.int16).cpu().numpy().view(np.uint16)
        per = self.raw.element_size() // 2
        lo, hi = g16[:self.pad * per], g16[len(g16) - self.pad * per:]
        assert np.all(lo == CANARY16) and np.all(hi == CANARY16), f"{what}: guard band written"


def guarded_cache(g):
    """A kvq.Cache whose six tensors sit in guarded, canary-filled buffers."""
    B, H, C, D = g.batch, g.n_kv_heads, g.capacity, g.head_dim
    blocks = C // 32
    shapes = {
        "k_codes": ((B, H, blocks, 64, 2, D * g.k_bits // 128), torch.int32),
        "v_codes": ((B, H, blocks, 64, D * g.v_bits // 64), torch.int32),
        "k_meta": ((B, H, C // g.group, D // 8, 8, 2), torch.int16),
        "v_meta": ((B, H, blocks, 4, D // g.group, 8, 2), torch.int16),
        "k_res": ((B, H, g.residual, D), torch.float16),
        "v_res": ((B, H, g.rv // 32, D // 16, 64, 8), torch.float16),
    }
    c = kvq.Cache.__new__(kvq.Cache)
    c.g = g
    c.guards = {}
    for name, (shape, dt) in shapes.items():
        gb = Guarded(shape, dt)
        setattr(c, name, gb.t)
        c.guards[name] = gb
    sizes = kvq.kvq_cache_bytes(g)
    for t, s in zip(c.tensors(), sizes):
        assert t.numel() * t.element_size() == s
    return c


def canary_oracle_cache(og):
    oc = oracle.Cache(og)
    for a in oc.arrays():
        a.view(np.uint16)[...] = CANARY16
    return oc


def assert_whole_cache(cache, oc, what):
    """Every word of every buffer equal (canaries included), guards intact."""
    torch.cuda.synchronize()
    for name, t, o in zip(NAMES, cache.tensors(), oc.arrays()):
        got = t.cpu().numpy().view(o.dtype).reshape(o.shape)
        bad = np.argwhere(got != o)
        assert bad.size == 0, f"{what} {name}: {len(bad)} words differ, first at {bad[0]}"
        cache.guards[name].check_guards(f"{what} {name}")


def _decode_guarded(g, cache, q, lens, scale, T=1, ws_fn=None):
    lens = np.asarray(lens, np.int32)
    msl = int(lens.max())
    D = getattr(g, "head_dim", 64)  # the rotated format's head dim is 64
    shape = (g.batch, g.n_q_heads, D) if T == 1 else (g.batch, T, g.n_q_heads, D)
    out = Guarded(shape, torch.float16)
    nbytes = ws_fn(msl)
    ws = Guarded((nbytes // 4,), torch.float32)
    return out, ws, msl


# ---------------------------------------------------------------- dense -----
DENSE = [
    # Hq, Hkv, D, bK, bV, G, R, lens (one sequence per regime)
    (8, 2, 128, 2, 4, 32, 128, [300, 257, 385, 200]),     # GQA 4, K2V4
    (8, 8, 128, 2, 2, 32, 64, [300, 129, 230, 97]),       # MHA
    (16, 2, 64, 4, 4, 64, 64, [320, 129, 260, 200]),      # GQA 8, D64
    (8, 4, 128, 8, 8, 32, 32, [300, 257, 185, 64]),       # GQA 2, 8-bit
    (16, 1, 128, 4, 2, 128, 128, [513, 300, 385, 129]),   # GQA 16, G128
    (8, 2, 64, 2, 8, 32, 32, [200, 33, 161, 96]),         # D64, K2V8
    (4, 1, 128, 8, 4, 64, 128, [400, 129, 256, 300]),     # GQA 4, K8V4, G64
    (8, 2, 128, 4, 8, 64, 64, [256, 300, 129, 65]),       # K4V8 G64
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: f"D{c[2]}K{c[3]}V{c[4]}G{c[5]}R{c[6]}gq{c[0] // c[1]}")
def test_edge_decode_dense(case):
    Hq, Hkv, D, bK, bV, G, R, lens = case
    B = len(lens)
    nmax = max(lens)
    C = (nmax // R + 2) * R
    _say(f"edge dense {case}")
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(1000 + D + 10 * bK + bV + G + R)
    k, v = edge_kv(rng, B, Hkv, nmax, D, G)
    q = edge_q(rng, B, Hq, D)
    cache = guarded_cache(g)
    oc = canary_oracle_cache(og)
    for b, n in enumerate(lens):
        sub = cache.view(b, b + 1)
        kvq.kvq_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        ob = oracle.Geom(1, Hq, Hkv, D, bK, bV, G, R, C)
        c1 = canary_oracle_cache(ob)
        oracle.prefill(ob, c1, k[b:b + 1, :, :n], v[b:b + 1, :, :n], n)
        for dst, src in zip(oc.arrays(), c1.arrays()):
            dst[b] = src[0]
    assert_whole_cache(cache, oc, "edge prefill")
    scale = 1.0 / math.sqrt(D)
    out, ws, msl = _decode_guarded(g, cache, q, lens, scale,
                                   ws_fn=lambda m: kvq.kvq_decode_workspace_bytes(g, m))
    kvq.kvq_decode_attn(g, dev(q), cache, dev(np.asarray(lens, np.int32)), msl, scale,
                        ws.t, out.t)
    torch.cuda.synchronize()
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), float(np.float32(scale)))
    out.check_guards("out")
    ws.check_guards("workspace")
    assert_whole_cache(cache, oc, "after decode")  # decode writes nothing in the cache
    got = out.t.float().cpu().numpy()
    assert np.all(np.isfinite(got)), "non-finite output (a canary was read)"
    ref32 = fp32_reference(og, oc, q, lens, float(np.float32(scale)))
    for b in range(B):
        assert_close_cond(got[b], ref[b], ref32[b], f"edge dense {case} seq {b} (regime {b % 4})")


# ------------------------------------------- append / flush write set -------
APPEND = [
    # Hq, Hkv, D, bK, bV, G, R, Rv, lens0, steps
    (8, 2, 128, 2, 4, 32, 64, 0, [60, 128, 1, 100], 70),
    (4, 2, 64, 8, 2, 64, 64, 0, [63, 64, 130, 10], 68),
    (8, 2, 128, 4, 8, 32, 32, 64, [31, 64, 95, 0], 70),
]


@pytest.mark.parametrize("case", APPEND, ids=lambda c: f"D{c[2]}K{c[3]}V{c[4]}G{c[5]}R{c[6]}Rv{c[7]}")
def test_edge_append_write_set(case):
    """Appends of edge-valued tokens through flushes: after every step the
    whole cache (canaries included) equals the oracle's, guards intact; the
    decode after the last step within tolerance."""
    Hq, Hkv, D, bK, bV, G, R, Rv, lens0, steps = case
    B = len(lens0)
    lens0 = np.asarray(lens0, np.int32)
    final = lens0 + steps
    Rmax = max(R, Rv)
    C = (int(final.max()) // Rmax + 2) * Rmax
    _say(f"edge append {case}")
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C, Rv)
    rng = np.random.default_rng(77 + D + bK + R)
    k, v = edge_kv(rng, B, Hkv, int(final.max()), D, G)
    cache = guarded_cache(g)
    oc = canary_oracle_cache(og)
    for b, n in enumerate(lens0.tolist()):
        if n == 0:
            continue
        sub = cache.view(b, b + 1)
        kvq.kvq_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        ob = oracle.Geom(1, Hq, Hkv, D, bK, bV, G, R, C, residual_v=Rv)
        c1 = canary_oracle_cache(ob)
        oracle.prefill(ob, c1, k[b:b + 1, :, :n], v[b:b + 1, :, :n], n)
        for dst, src in zip(oc.arrays(), c1.arrays()):
            dst[b] = src[0]
    assert_whole_cache(cache, oc, "append prefill")
    lens = lens0.copy()
    for s in range(steps):
        kn = np.ascontiguousarray(k[np.arange(B), :, lens])
        vn = np.ascontiguousarray(v[np.arange(B), :, lens])
        kvq.kvq_append(g, dev(kn), dev(vn), dev(lens), cache)
        oracle.append(og, oc, kn, vn, lens)
        lens = lens + 1
        flushed = np.any((lens - 1 > 0) & (((lens - 1) % R == 0) | ((lens - 1) % g.rv == 0)))
        if flushed or s == steps - 1 or s % 16 == 0:
            assert_whole_cache(cache, oc, f"append step {s} (lens {lens.tolist()})")
    q = edge_q(rng, B, Hq, D)
    scale = 1.0 / math.sqrt(D)
    out, ws, msl = _decode_guarded(g, cache, q, lens, scale,
                                   ws_fn=lambda m: kvq.kvq_decode_workspace_bytes(g, m))
    kvq.kvq_decode_attn(g, dev(q), cache, dev(lens), msl, scale, ws.t, out.t)
    ref = oracle.decode_attn(og, oc, q, lens, float(np.float32(scale)))
    out.check_guards("out")
    ws.check_guards("workspace")
    ref32 = fp32_reference(og, oc, q, lens, float(np.float32(scale)))
    assert_close_cond(out.t, ref, ref32, f"edge append decode {case}")


def test_edge_append_tokens_write_set():
    """kvq_append_tokens (T = 3) of edge tokens through flushes: the whole cache
    equals the oracle's T single appends after every call."""
    B, Hq, Hkv, D, bK, bV, G, R, T = 4, 8, 2, 128, 2, 4, 32, 32, 3
    lens0 = np.array([30, 64, 1, 95], np.int32)
    calls = 24
    final = lens0 + T * calls
    C = (int(final.max()) // R + 2) * R
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(4242)
    k, v = edge_kv(rng, B, Hkv, int(final.max()), D, G)
    cache = guarded_cache(g)
    oc = canary_oracle_cache(og)
    for b, n in enumerate(lens0.tolist()):
        if n == 0:
            continue
        sub = cache.view(b, b + 1)
        kvq.kvq_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        ob = oracle.Geom(1, Hq, Hkv, D, bK, bV, G, R, C)
        c1 = canary_oracle_cache(ob)
        oracle.prefill(ob, c1, k[b:b + 1, :, :n], v[b:b + 1, :, :n], n)
        for dst, src in zip(oc.arrays(), c1.arrays()):
            dst[b] = src[0]
    lens = lens0.copy()
    for s in range(calls):
        idx = lens[:, None] + np.arange(T)[None, :]                     # [B][T]
        kt = np.ascontiguousarray(k[np.arange(B)[:, None], :, idx])     # [B][T][Hkv][D]
        vt = np.ascontiguousarray(v[np.arange(B)[:, None], :, idx])
        kvq.kvq_append_tokens(g, T, dev(kt), dev(vt), dev(lens), cache)
        for j in range(T):
            oracle.append(og, oc, np.ascontiguousarray(kt[:, j]), np.ascontiguousarray(vt[:, j]),
                          lens + j)
        lens = lens + T
        assert_whole_cache(cache, oc, f"append_tokens call {s} (lens {lens.tolist()})")


# ---------------------------------------------------------------- paged -----
PAGED = [
    # Hq, Hkv, D, bK, bV, G, R, P, lens
    (8, 2, 128, 2, 4, 32, 128, 128, [300, 257, 385, 200]),
    (16, 2, 64, 4, 2, 64, 64, 64, [320, 129, 260, 200]),
    (8, 4, 128, 8, 8, 32, 32, 32, [300, 257, 185, 64]),
]


@pytest.mark.parametrize("case", PAGED, ids=lambda c: f"D{c[2]}K{c[3]}V{c[4]}G{c[5]}P{c[7]}")
def test_edge_decode_paged(case):
    Hq, Hkv, D, bK, bV, G, R, P, lens = case
    B = len(lens)
    nmax = max(lens)
    C = (nmax // R + 2) * R
    C = -(-C // P) * P
    _say(f"edge paged {case}")
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(2000 + D + bK + P)
    k, v = edge_kv(rng, B, Hkv, nmax, D, G)
    q = edge_q(rng, B, Hq, D)
    table, npages = _table(rng, B, C // P, _pages_needed(lens, R, P))
    pc = kvq.PagedCache(g, P, npages, dev(table))
    for b, n in enumerate(lens):
        sub = pc.view(b, b + 1)
        kvq.kvq_paged_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
    oc = oracle.Cache(og)
    for b, n in enumerate(lens):
        ob = oracle.Geom(1, Hq, Hkv, D, bK, bV, G, R, C)
        c1 = oracle.Cache(ob)
        oracle.prefill(ob, c1, k[b:b + 1, :, :n], v[b:b + 1, :, :n], n)
        for dst, src in zip(oc.arrays(), c1.arrays()):
            dst[b] = src[0]
    from kvq_testutil import assert_cache_equal
    assert_cache_equal(_gather(pc, table, g), oc, lens, what="edge paged prefill")
    scale = 1.0 / math.sqrt(D)
    out, ws, msl = _decode_guarded(g, pc, q, lens, scale,
                                   ws_fn=lambda m: kvq.kvq_paged_decode_workspace_bytes(g, 1, m))
    kvq.kvq_paged_decode_attn(g, dev(q), pc, dev(np.asarray(lens, np.int32)), msl, scale,
                              ws.t, out.t)
    torch.cuda.synchronize()
    out.check_guards("out")
    ws.check_guards("workspace")
    ref = oracle.decode_attn(og, oc, q, np.asarray(lens, np.int32), float(np.float32(scale)))
    ref32 = fp32_reference(og, oc, q, lens, float(np.float32(scale)))
    assert_close_cond(out.t, ref, ref32, f"edge paged {case}")


# ----------------------------------------------------- several query tokens --
MULTI = [
    # Hq, Hkv, D, bK, bV, G, R, T, lens
    (8, 2, 128, 2, 4, 32, 128, 4, [300, 257, 385, 131]),   # 16 rows per KV head
    (4, 2, 64, 4, 2, 64, 64, 4, [320, 129, 66, 200]),      # 8 rows
    (8, 4, 128, 8, 8, 32, 32, 2, [300, 33, 185, 64]),      # 4 rows, 8-bit
    (8, 8, 128, 2, 2, 32, 64, 2, [300, 129, 66, 200]),     # MHA, 2 rows: split value columns
]


@pytest.mark.parametrize("case", MULTI, ids=lambda c: f"D{c[2]}K{c[3]}V{c[4]}G{c[5]}T{c[7]}")
def test_edge_decode_multi(case):
    Hq, Hkv, D, bK, bV, G, R, T, lens = case
    B = len(lens)
    nmax = max(lens)
    C = (nmax // R + 2) * R
    _say(f"edge multi {case}")
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(3000 + D + bK + T)
    k, v = edge_kv(rng, B, Hkv, nmax, D, G)
    q = edge_q(rng, B, Hq, D, T=T)
    cache = guarded_cache(g)
    oc = canary_oracle_cache(og)
    for b, n in enumerate(lens):
        sub = cache.view(b, b + 1)
        kvq.kvq_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        ob = oracle.Geom(1, Hq, Hkv, D, bK, bV, G, R, C)
        c1 = canary_oracle_cache(ob)
        oracle.prefill(ob, c1, k[b:b + 1, :, :n], v[b:b + 1, :, :n], n)
        for dst, src in zip(oc.arrays(), c1.arrays()):
            dst[b] = src[0]
    scale = 1.0 / math.sqrt(D)
    out, ws, msl = _decode_guarded(g, cache, q, lens, scale, T=T,
                                   ws_fn=lambda m: kvq.kvq_decode_multi_workspace_bytes(g, T, m))
    kvq.kvq_decode_attn_multi(g, dev(q), cache, dev(np.asarray(lens, np.int32)), T, msl, scale,
                              ws.t, out.t)
    torch.cuda.synchronize()
    out.check_guards("out")
    ws.check_guards("workspace")
    assert_whole_cache(cache, oc, "after multi decode")
    ref = oracle.decode_attn_multi(og, oc, q, np.asarray(lens, np.int32), T,
                                   float(np.float32(scale)))
    ref32 = fp32_reference(og, oc, q, lens, float(np.float32(scale)), T=T)
    assert_close_cond(out.t, ref, ref32, f"edge multi {case}")


# ----------------------------------------------- rotated 2-bit format -------
def bq2_edge_kv(rng, B, Hkv, n, huge=8000.0):
    """Regimes of the rotated format (head dim 64; inputs below 8188 in
    magnitude keep the rotated entries inside fp16): 0 zero, constant, tiny
    (range below the 1e-6 scale floor) and subnormal rows; 1 huge key rows; 2
    huge value rows; 3 ordinary rows (queries x100 / x1e-3)."""
    D = 64
    k = rng.standard_normal((B, Hkv, n, D)) * rng.lognormal(0, 0.5, (1, Hkv, 1, D))
    v = rng.standard_normal((B, Hkv, n, D))
    for b in range(B):
        r = b % 4
        for t in range(n):
            if r == 0:
                m = t % 6
                if m == 1:
                    k[b, :, t] = 0.0
                    v[b, :, t] = 0.0
                elif m == 2:
                    k[b, :, t] = 0.5
                    v[b, :, t] = -1.25
                elif m == 3:
                    k[b, :, t] = 1e-8 * rng.standard_normal((Hkv, D))
                    v[b, :, t] = 1e-8 * rng.standard_normal((Hkv, D))
                elif m == 4:
                    k[b, :, t] = rng.integers(0, 5, (Hkv, D)) * 2.0 ** -24
                    v[b, :, t] = rng.integers(0, 5, (Hkv, D)) * 2.0 ** -24
            elif r == 1 and t % 5 == 2:
                k[b, :, t] = rng.uniform(-huge, huge, (Hkv, D))
            elif r == 2 and t % 3 == 0:
                v[b, :, t] = rng.uniform(-huge, huge, (Hkv, D))
    return k.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("Hq,Hkv,lens", [(8, 2, [300, 257, 385, 200]), (4, 4, [129, 64, 5, 100]),
                                         (8, 4, [1, 40, 3, 260])])
def test_edge_decode_bq2(Hq, Hkv, lens):
    B = len(lens)
    nmax = max(lens)
    C = (nmax // 32 + 2) * 32
    _say(f"edge bq2 Hq={Hq} Hkv={Hkv} lens {lens}")
    g, og = kvq.Bq2Geom(B, Hq, Hkv, C), oracle.Bq2Geom(B, Hq, Hkv, C)
    rng = np.random.default_rng(5000 + Hq + Hkv)
    k, v = bq2_edge_kv(rng, B, Hkv, nmax)
    q = edge_q(rng, B, Hq, 64)
    from test_gpu_bq2 import _assert_state, _prefill_both
    cache, oc = _prefill_both(g, og, k, v, lens)
    _assert_state(g, og, cache, oc, lens, what="edge bq2 prefill")
    scale = 0.125
    out, ws, msl = _decode_guarded(g, cache, q, lens, scale,
                                   ws_fn=lambda m: kvq.kvq_bq2_decode_workspace_bytes(g, m))
    out_t = out.t
    kvq.kvq_bq2_decode_attn(g, dev(q), cache, dev(np.asarray(lens, np.int32)), msl, scale,
                            ws.t, out_t)
    torch.cuda.synchronize()
    out.check_guards("out")
    ws.check_guards("workspace")
    ref = oracle.bq2_decode_attn(og, oc, q, np.asarray(lens, np.int32), float(np.float32(scale)))
    got = out_t.float().cpu().numpy()
    for b in range(B):
        err = assert_close(got[b], ref[b], what=f"edge bq2 seq {b} (regime {b % 4})")
        _say(f"  seq {b} regime {b % 4}: max err {err:.2e}, max|o| {np.abs(ref[b]).max():.3g}")
