"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantization, no attention), so both the GPU path and the CPU
oracle can take their inputs from it.

Value structure (a stand-in for real K/V activations, which need model
weights): queries and values are fp16 N(0, 1); keys are fp16 N(0, 1) times a
per-(KV head, channel) scale and a few outlier channels per head, because the
KIVI pages explain per-channel key quantization by outliers that live in fixed
channels.  The channel structure is a property of the head, shared by every
sequence, token and decode step.

Streams: numpy PCG64 seeded by SeedSequence([20261203, config, layer, stream]);
stream 0 = head structure, 1 = prefill keys, 2 = prefill values, 3 = queries,
4 = sequence lengths, 1000 + step = the step's new key/value/query.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20261203


@dataclass(frozen=True)
class Workload:
    """One of the pages' workload shapes."""
    name: str
    cfg: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    k_bits: int
    v_bits: int
    group: int
    residual: int
    context: int            # n at attention time (incl. the current token)
    layers: int = 1
    ctx_range: tuple | None = None   # variable length: uniform integers [lo, hi]
    lognormal_sigma: float = 0.5     # per-channel key scale spread (0: none)
    n_outliers: int = 4
    outlier_lo: float = 10.0
    outlier_hi: float = 20.0
    steps: int = 1
    fmt: str = "kivi"               # "kivi" or "bq2" (rotated per-token 2-bit)

    def max_context(self) -> int:
        return self.ctx_range[1] if self.ctx_range else self.context


WORKLOADS = {
    # Tiny: parity focus.
    1: Workload("tiny_b1_h2_d64_k2v2_g32_r32_n256", 1, 1, 2, 2, 64, 2, 2, 32, 32,
                256, lognormal_sigma=0.0, n_outliers=2, outlier_lo=10.0,
                outlier_hi=10.0),
    # Llama-2-7B-shaped MHA layer.
    2: Workload("llama2_7b_mha_b8_n4096_k2v2_g32_r128", 2, 8, 32, 32, 128, 2, 2,
                32, 128, 4096),
    # Llama-3-8B-shaped GQA layer (group 4), asymmetric K2/V4.
    3: Workload("llama3_8b_gqa_b32_n8192_k2v4_g32_r128", 3, 32, 32, 8, 128, 2, 4,
                32, 128, 8192),
    # Long-context variable length.
    4: Workload("longctx_gqa_b4_n16k-64k_k2v2_g64_r128", 4, 4, 32, 8, 128, 2, 2,
                64, 128, 65536, ctx_range=(16384, 65536)),
    # Full-stack decode: 32 layers, 256 steps from a 4096-token prefix.
    5: Workload("fullstack_32l_gqa_b64_n4096_k4v2_g64_r64_256steps", 5, 64, 32,
                8, 128, 4, 2, 64, 64, 4096, layers=32, steps=256),
    # KV1-shaped attention layer (32 query heads, 8 KV heads, head dim 64, 32K
    # context) in the rotated per-token 2-bit format with 4 fp16 sinks; keys
    # carry the same channel structure before rotation.
    6: Workload("kv1_bq2_gqa_b16_n32768_d64", 6, 16, 32, 8, 64, 2, 2, 64, 0, 32768,
                fmt="bq2"),
}


def rng(cfg: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cfg, layer, stream])))


def _normal_f16(gen: np.random.Generator, shape) -> np.ndarray:
    return gen.standard_normal(size=shape, dtype=np.float32).astype(np.float16)


def head_structure(w: Workload, layer: int = 0) -> np.ndarray:
    """Per-(KV head, channel) key multiplier, float32 [Hkv][D]."""
    g = rng(w.cfg, layer, 0)
    H, D = w.n_kv_heads, w.head_dim
    if w.lognormal_sigma > 0:
        s = g.lognormal(mean=0.0, sigma=w.lognormal_sigma, size=(H, D))
    else:
        s = np.ones((H, D))
    for h in range(H):
        ch = g.choice(D, size=w.n_outliers, replace=False)
        s[h, ch] *= g.uniform(w.outlier_lo, w.outlier_hi, size=w.n_outliers)
    return s.astype(np.float32)


def keys(w: Workload, n_tok: int, layer: int = 0, stream: int = 1,
         batch: int | None = None) -> np.ndarray:
    """fp16 [B][Hkv][n_tok][D] keys with the head's channel structure."""
    B = w.batch if batch is None else batch
    z = rng(w.cfg, layer, stream).standard_normal(
        size=(B, w.n_kv_heads, n_tok, w.head_dim), dtype=np.float32)
    z *= head_structure(w, layer)[None, :, None, :]
    return z.astype(np.float16)


def values(w: Workload, n_tok: int, layer: int = 0, stream: int = 2,
           batch: int | None = None) -> np.ndarray:
    B = w.batch if batch is None else batch
    return _normal_f16(rng(w.cfg, layer, stream),
                       (B, w.n_kv_heads, n_tok, w.head_dim))


def queries(w: Workload, layer: int = 0, stream: int = 3,
            batch: int | None = None) -> np.ndarray:
    B = w.batch if batch is None else batch
    return _normal_f16(rng(w.cfg, layer, stream), (B, w.n_q_heads, w.head_dim))


def seq_lens(w: Workload, layer: int = 0) -> np.ndarray:
    """int32 [B] context lengths (incl. the current token)."""
    if w.ctx_range is None:
        return np.full(w.batch, w.context, np.int32)
    lo, hi = w.ctx_range
    return rng(w.cfg, layer, 4).integers(lo, hi, size=w.batch,
                                         endpoint=True).astype(np.int32)


def step_token(w: Workload, step: int, layer: int = 0, batch: int | None = None):
    """The new token of a decode step: (k_new, v_new fp16 [B][Hkv][D],
    q fp16 [B][Hq][D])."""
    B = w.batch if batch is None else batch
    g = rng(w.cfg, layer, 1000 + step)
    k = g.standard_normal(size=(B, w.n_kv_heads, w.head_dim), dtype=np.float32)
    k *= head_structure(w, layer)[None]
    v = g.standard_normal(size=(B, w.n_kv_heads, w.head_dim), dtype=np.float32)
    q = g.standard_normal(size=(B, w.n_q_heads, w.head_dim), dtype=np.float32)
    return k.astype(np.float16), v.astype(np.float16), q.astype(np.float16)


def capacity_for(w: Workload, extra_tokens: int = 0) -> int:
    """Smallest multiple of R (of 32 for the rotated format) holding the
    longest context plus extra tokens."""
    need = w.max_context() + extra_tokens
    R = w.residual if w.fmt == "kivi" else 32
    return ((need + R - 1) // R) * R
