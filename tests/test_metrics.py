"""Byte accounting pinned to the KV1 model card's "Memory" table.

At head_dim 64 with groups of 64 the packed format spends 2-bit codes plus an
fp16 scale and min per 64 values on keys and on values alike, i.e. the 2.5
bits/value of the card's BQ2_0 cache (and 3.5 bits/value for 3-bit codes).
"""
import os

import pytest

from quantized_decode_attention_amd import metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv1_memory_table.txt")
LAYERS, KV_HEADS, D = 6, 8, 64


def _rows():
    out = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            ctx, unit, f16, b3, b2, prec = [p.strip() for p in line.split("|")]
            out.append((int(ctx), unit, float(f16), float(b3), float(b2), float(prec)))
    return out


@pytest.mark.parametrize("row", _rows(), ids=lambda r: str(r[0]))
def test_kv1_memory_table(row):
    ctx, unit, f16, b3, b2, prec = row
    div = 1024 if unit == "KiB" else 1024 * 1024
    per_tok = {
        "fp16": LAYERS * KV_HEADS * metrics.fp16_bytes_per_token(D),
        "3bit": LAYERS * KV_HEADS * metrics.packed_bytes_per_token(D, 3, 3, 64),
        "bq2_0": LAYERS * KV_HEADS * metrics.packed_bytes_per_token(D, 2, 2, 64),
    }
    for key, expect in (("fp16", f16), ("3bit", b3), ("bq2_0", b2)):
        got = per_tok[key] * ctx / div
        assert abs(got - expect) <= prec, (key, got, expect)


def test_bits_per_value():
    # 2.5 bits/value at G = 64 (KV1 card: 2.5 bits per value, ~6.4x below fp16)
    assert metrics.packed_bytes_per_token(64, 2, 2, 64) * 8 / (2 * 64) == 2.5
    assert metrics.packed_bytes_per_token(128, 2, 2, 64) * 8 / (2 * 128) == 2.5
    assert abs(16 / 2.5 - 6.4) < 1e-12


def test_decode_step_bytes_closed_form():
    # config-3 shape: B32, 32/8, D128, K2/V4, G32, R128, n = 8192 -> 8064 packed
    b = metrics.decode_step_bytes([8192] * 32, 32, 8, 128, 2, 4, 32, 128)
    per_packed = 128 * 6 / 8 + 2 * 4 * 128 / 32
    assert per_packed == 128
    expect = 32 * 8 * (8064 * 128 + 128 * 512) + 4 * 32 * 32 * 128 + 4 * 32
    assert b == expect
    assert metrics.packed_len(8192, 128) == 8064
    assert metrics.packed_len(8193, 128) == 8192
    assert metrics.packed_len(1, 128) == 0
    assert metrics.packed_len(128, 128) == 0
    assert metrics.packed_len(129, 128) == 128


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N with N != 1 prints one JSON line
    naming the reason and exits with status 2 (before touching any device)."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_decode_step_bytes_of_the_benchmarked_workload():
    """The Llama-3-8B GQA workload (B32, 32/8, D128, K2/V4, G32, R128) at n = 8192: per KV head
    8064 packed tokens of 32 + 64 + 16 + 16 bytes and 128 fp16 tokens of 512
    bytes, plus q in and out (4 bytes per query value) and the lengths."""
    n = [8192] * 32
    got = metrics.decode_step_bytes(n, 32, 8, 128, 2, 4, 32, 128)
    per_head = 8064 * (32 + 64 + 16 + 16) + 128 * 512
    assert got == 32 * 8 * per_head + 4 * 32 * 32 * 128 + 4 * 32


def test_separate_key_and_value_windows():
    """Key window 128, value window 64 at n = 8192 (B32, 32/8, D128, K2/V4,
    G32): keys hold 8064 packed + 128 fp16 tokens, values 8128 packed + 64 fp16
    tokens.  Packed key token: 32 code bytes + 4 * 128 / 32 meta bytes; packed
    value token: 64 code bytes + 16 meta bytes; an fp16 K or V row is 256
    bytes."""
    n = [8192] * 32
    got = metrics.decode_step_bytes(n, 32, 8, 128, 2, 4, 32, 128, residual_v=64)
    per_head = 8064 * 48 + 128 * 256 + 8128 * 80 + 64 * 256
    assert got == 32 * 8 * per_head + 4 * 32 * 32 * 128 + 4 * 32
    # one window each: the same as the single-window call
    assert metrics.decode_step_bytes(n, 32, 8, 128, 2, 4, 32, 128, residual_v=128) == \
        metrics.decode_step_bytes(n, 32, 8, 128, 2, 4, 32, 128)
    # flushing one unit: 128 key rows read (256 B) and packed (48 B), 64 value rows (256 + 80 B)
    assert metrics.flush_bytes(1, 128, 128, 2, 4, 32, residual_v=64) == 128 * 304 + 64 * 336
    assert metrics.flush_bytes(3, 128, 128, 2, 4, 32) == 3 * 128 * (512 + 128)
