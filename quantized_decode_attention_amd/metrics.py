"""Byte accounting of the packed cache and of one decode step.

Algorithmic bytes are the bytes the method itself must move: every packed code
once, each key group's fp16 (scale, min) row once per G tokens, each token's
value (scale, min) pairs once, the fp16 residual window, the query and the
output.  Split partials and any re-reads are not counted (they count against
the kernels).  The per-token formula reproduces the KV1 model card's "Memory"
table (fp16 / 3.5-bit / BQ2_0 per token and at 8K and 32K context), which is
the pin used by the tests.
"""
from __future__ import annotations

import numpy as np


def packed_bytes_per_token(head_dim: int, k_bits: int, v_bits: int, group: int) -> float:
    """Bytes per packed token per KV head: codes, key meta amortized over the
    group's G tokens (4 bytes per channel), value meta (4 bytes per group)."""
    D, G = head_dim, group
    return D * (k_bits + v_bits) / 8 + 4 * D / G + 4 * D / G


def fp16_bytes_per_token(head_dim: int) -> int:
    return 2 * 2 * head_dim


def packed_len(n: int, residual: int) -> int:
    """Packed tokens of a sequence of n tokens under the lazy flush rule."""
    return 0 if n <= 0 else n - (((n - 1) % residual) + 1)


def decode_step_bytes(seq_lens, n_q_heads: int, n_kv_heads: int, head_dim: int,
                      k_bits: int, v_bits: int, group: int, residual: int,
                      residual_v: int | None = None) -> float:
    """Algorithmic bytes of one decode-attention launch over sequences of the
    given lengths (current token included).  residual is the key window;
    residual_v the value window (default: the same)."""
    D, G = head_dim, group
    Rk = residual
    Rv = residual if residual_v is None else residual_v
    key_tok = D * k_bits / 8 + 4 * D / G      # codes + (scale, min) per channel / G
    val_tok = D * v_bits / 8 + 4 * D / G      # codes + (scale, min) per group of G
    total = 0.0
    for n in np.asarray(seq_lens).tolist():
        n = int(n)
        lk, lv = packed_len(n, Rk), packed_len(n, Rv)
        total += n_kv_heads * (lk * key_tok + (n - lk) * 2 * D
                               + lv * val_tok + (n - lv) * 2 * D)
    B = len(np.asarray(seq_lens))
    total += 2 * 2 * B * n_q_heads * D       # q in, out
    total += 4 * B                            # seq_lens
    return total


def append_bytes(batch: int, n_kv_heads: int, head_dim: int) -> int:
    """Bytes of one append without a flush: new K, V read and written."""
    return 2 * 2 * 2 * batch * n_kv_heads * head_dim


def flush_bytes(n_flush_units: int, residual: int, head_dim: int, k_bits: int,
                v_bits: int, group: int, residual_v: int | None = None) -> float:
    """Bytes of flushing full residual windows of n units: the fp16 window
    read, the packed rows written.  With separate windows (residual for keys,
    residual_v for values) this counts one flush of each."""
    D, G = head_dim, group
    Rk = residual
    Rv = residual if residual_v is None else residual_v
    key_tok = D * k_bits / 8 + 4 * D / G
    val_tok = D * v_bits / 8 + 4 * D / G
    return n_flush_units * (Rk * (2 * D + key_tok) + Rv * (2 * D + val_tok))


# ---- rotated per-token 2-bit format ([KV1] Quantization Format) ------------
BQ2_BLOCK_BYTES = 20   # fp16 d, fp16 m, 16 bytes of 2-bit codes per 64 values
BQ2_SINKS = 4


def bq2_bytes_per_token() -> int:
    """Bytes per position per KV head: one block each for K and V."""
    return 2 * BQ2_BLOCK_BYTES


def bq2_decode_step_bytes(seq_lens, n_q_heads: int, n_kv_heads: int) -> float:
    """Algorithmic bytes of one decode-attention launch in the rotated format:
    packed blocks of positions >= 4, fp16 sinks, query in and output out."""
    D = 64
    total = 0.0
    for n in np.asarray(seq_lens).tolist():
        n = int(n)
        sinks = min(n, BQ2_SINKS)
        total += n_kv_heads * ((n - sinks) * bq2_bytes_per_token()
                               + sinks * fp16_bytes_per_token(D))
    B = len(np.asarray(seq_lens))
    total += 2 * 2 * B * n_q_heads * D
    total += 4 * B
    return total


def bq2_append_bytes(batch: int, n_kv_heads: int) -> int:
    """One append: new K, V read (fp16) and their blocks written."""
    return batch * n_kv_heads * (2 * 2 * 64 + bq2_bytes_per_token())
