"""Shared helpers of the GPU parity tests: run the same seeded inputs through
libkvq (via its C ABI binding) and through the CPU oracle, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_decode_attention_amd as kvq

NAMES = ("k_codes", "v_codes", "k_meta", "v_meta", "k_res", "v_res")


def geoms(B, Hq, Hkv, D, bK, bV, G, R, C, Rv=0):
    """Library and oracle geometry; Rv: a value window of its own (0: R)."""
    return (kvq.Geom(B, Hq, Hkv, D, bK, bV, G, R, C, Rv),
            oracle.Geom(B, Hq, Hkv, D, bK, bV, G, R, C, residual_v=Rv))


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cache_np(cache: kvq.Cache, like: oracle.Cache):
    torch.cuda.synchronize()
    out = {}
    for name, t, o in zip(NAMES, cache.tensors(), like.arrays()):
        out[name] = t.cpu().numpy().view(o.dtype).reshape(o.shape)
    return out


def assert_cache_equal(cache: kvq.Cache, oc: oracle.Cache, lens=None, what=""):
    """Packed state bit-exact; with lens given, only each sequence's packed
    prefix and live residual slots are compared (the rest is unspecified)."""
    got = cache_np(cache, oc)
    g = oc.g
    if lens is None:
        for name, o in zip(NAMES, oc.arrays()):
            bad = np.argwhere(got[name] != o)
            assert bad.size == 0, f"{what} {name}: {len(bad)} mismatches, first at {bad[0]}"
        return
    for b, n in enumerate(np.asarray(lens).tolist()):
        lqk, lqv = oracle.packed_len(n, g.rk), oracle.packed_len(n, g.rv)
        sl = {
            "k_codes": (slice(b, b + 1), slice(None), slice(0, lqk // 32)),
            "k_meta": (slice(b, b + 1), slice(None), slice(0, lqk // g.group)),
            "v_codes": (slice(b, b + 1), slice(None), slice(0, lqv // 32)),
            "v_meta": (slice(b, b + 1), slice(None), slice(0, lqv // 32)),
        }
        for name, idx in sl.items():
            o = getattr(oc, name)[idx]
            gg = got[name][idx]
            bad = np.argwhere(gg != o)
            assert bad.size == 0, f"{what} seq {b} {name}: {len(bad)} mismatches, first {bad[0]}"
        res = {"k_res": (got["k_res"], oc.k_res, lqk, g.rk),
               "v_res": (oracle.value_res_rows(g, got["v_res"]),
                         oracle.value_res_rows(g, oc.v_res), lqv, g.rv)}
        for name, (ga, oa, lq, R) in res.items():
            for t in range(lq, n):
                s = t % R
                assert np.array_equal(ga[b, :, s], oa[b, :, s]), \
                    f"{what} seq {b} {name} slot {s}"


def assert_close(got: torch.Tensor | np.ndarray, ref: np.ndarray, what="", tol=1e-3):
    """|gpu - oracle| <= tol * (1 + |oracle|) elementwise."""
    if isinstance(got, torch.Tensor):
        got = got.float().cpu().numpy()
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    lim = tol * (1.0 + np.abs(ref))
    bad = np.argwhere(~(err <= lim))
    assert bad.size == 0, (f"{what}: {len(bad)} of {err.size} outside tolerance; first at "
                           f"{bad[0]} got {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]}; "
                           f"max err {np.nanmax(err):.3e}")
    return float(np.max(err)) if err.size else 0.0


def prefill_both(g, og, k, v, lens):
    """Per-sequence prefill on both sides; k, v fp16 [B][Hkv][>=max n][D]."""
    cache = kvq.Cache(g)
    oc = oracle.Cache(og)
    lens = np.asarray(lens).tolist()
    if all(n == lens[0] for n in lens):
        n = lens[0]
        kvq.kvq_prefill(g, dev(k[:, :, :n]), dev(v[:, :, :n]), n, cache)
        oracle.prefill(og, oc, k[:, :, :n], v[:, :, :n], n)
        return cache, oc
    for b, n in enumerate(lens):
        sub = cache.view(b, b + 1)
        kvq.kvq_prefill(sub.g, dev(k[b:b + 1, :, :n]), dev(v[b:b + 1, :, :n]), n, sub)
        ob = oracle.Geom(1, og.n_q_heads, og.n_kv_heads, og.head_dim, og.k_bits, og.v_bits,
                         og.group, og.residual, og.capacity,
                         residual_v=og.residual_v)
        c1 = oracle.Cache(ob)
        oracle.prefill(ob, c1, k[b:b + 1, :, :n], v[b:b + 1, :, :n], n)
        for dst, src in zip(oc.arrays(), c1.arrays()):
            dst[b] = src[0]
    return cache, oc


def decode_both(g, og, cache, oc, q, lens, max_seq_len=None, scale=None):
    lens = np.asarray(lens, dtype=np.int32)
    msl = int(lens.max()) if max_seq_len is None else max_seq_len
    scale = 1.0 / np.sqrt(g.head_dim) if scale is None else scale
    out = torch.empty((g.batch, g.n_q_heads, g.head_dim), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_workspace(g, msl)
    kvq.kvq_decode_attn(g, dev(q), cache, dev(lens), msl, scale, ws, out)
    torch.cuda.synchronize()
    ref = oracle.decode_attn(og, oc, q, lens, float(np.float32(scale)))
    return out, ref
