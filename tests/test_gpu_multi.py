"""GPU parity of attention for several query tokens per sequence
(kvq_decode_attn_multi) against the CPU oracle, through the C ABI.

Query token i of the last T attends causally to positions [0, n - T + i] of
the cache at length n.  Outputs must satisfy |gpu - oracle| <= 1e-3 * (1 +
|oracle|).  Lengths are chosen so that the causal mask falls in the fp16
window, in the newest packed chunk (T larger than the window's fill), and on
chunk boundaries; T = 1 must equal kvq_decode_attn bit for bit.
"""
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


def _run(g, og, cache, oc, q, lens, T, scale=0.125, max_len=None):
    lens = np.asarray(lens, np.int32)
    msl = int(lens.max()) if max_len is None else max_len
    out = torch.empty((g.batch, T, g.n_q_heads, g.head_dim), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_multi_workspace(g, T, msl)
    kvq.kvq_decode_attn_multi(g, dev(q), cache, dev(lens), T, msl, scale, ws, out)
    torch.cuda.synchronize()
    ref = oracle.decode_attn_multi(og, oc, q, lens, T, float(np.float32(scale)))
    return out, ref


CASES = [
    # (D, bK, bV, G, R, Hq, Hkv, T, lengths)
    (128, 2, 4, 32, 128, 8, 2, 4, [4, 5, 31, 33, 129, 130, 131, 200, 257, 259]),
    (128, 2, 4, 32, 128, 8, 2, 2, [2, 64, 128, 129, 130, 300]),
    (128, 2, 2, 64, 64, 4, 1, 4, [65, 66, 67, 68, 128, 129, 190]),
    (64, 4, 2, 32, 32, 2, 2, 16, [16, 17, 33, 47, 48, 64, 100]),
    (128, 4, 4, 32, 64, 16, 2, 2, [2, 65, 66, 97, 160]),
    (64, 2, 2, 64, 64, 2, 1, 8, [8, 64, 65, 70, 71, 72, 129]),
    (128, 8, 8, 32, 128, 8, 2, 4, [4, 131, 257, 300]),
    # MHA with several query tokens: 2 or 4 rows per KV head, so the value
    # weights' hi and lo parts take neighbouring MFMA columns
    (128, 2, 4, 32, 128, 4, 4, 2, [2, 64, 129, 200]),
    (128, 4, 2, 64, 64, 4, 4, 4, [4, 65, 130, 191]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"D{c[0]}K{c[1]}V{c[2]}G{c[3]}R{c[4]}gq{c[5] // c[6]}T{c[7]}")
def test_multi_token_parity(case):
    D, bK, bV, G, R, Hq, Hkv, T, lens = case
    B = len(lens)
    C = ((max(lens) + R) // R + 1) * R
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(sum(lens) + T)
    k = (rng.standard_normal((B, Hkv, max(lens), D)) *
         rng.lognormal(0, 0.5, (1, Hkv, 1, D))).astype(np.float16)
    v = rng.standard_normal((B, Hkv, max(lens), D)).astype(np.float16)
    q = rng.standard_normal((B, T, Hq, D)).astype(np.float16)
    _say(f"multi T={T} gq={Hq // Hkv} D={D} K{bK}V{bV} G{G} R{R} lens {lens}")
    cache, oc = prefill_both(g, og, k, v, lens)
    out, ref = _run(g, og, cache, oc, q, lens, T)
    assert_close(out, ref, what=f"T={T}")


def test_single_token_equals_decode_attn():
    g, og = geoms(3, 8, 2, 128, 2, 4, 32, 128, 512)
    lens = [1, 200, 385]
    rng = np.random.default_rng(7)
    k = rng.standard_normal((3, 2, 385, 128)).astype(np.float16)
    v = rng.standard_normal((3, 2, 385, 128)).astype(np.float16)
    q = rng.standard_normal((3, 1, 8, 128)).astype(np.float16)
    cache, oc = prefill_both(g, og, k, v, lens)
    out, _ = _run(g, og, cache, oc, q, lens, 1)
    one = torch.empty((3, 8, 128), dtype=torch.float16, device="cuda")
    ws = kvq.alloc_workspace(g, 385)
    kvq.kvq_decode_attn(g, dev(np.ascontiguousarray(q[:, 0])), cache, dev(np.array(lens, np.int32)),
                        385, 0.125, ws, one)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0].view(torch.int16), one.view(torch.int16))


def test_rows_that_see_nothing_are_zero():
    g, og = geoms(2, 4, 2, 64, 2, 2, 32, 32, 64)
    lens = [2, 40]  # T = 4: tokens 0, 1 of sequence 0 see no position
    rng = np.random.default_rng(8)
    k = rng.standard_normal((2, 2, 40, 64)).astype(np.float16)
    v = rng.standard_normal((2, 2, 40, 64)).astype(np.float16)
    q = rng.standard_normal((2, 4, 4, 64)).astype(np.float16)
    cache, oc = prefill_both(g, og, k, v, lens)
    out, ref = _run(g, og, cache, oc, q, lens, 4)
    o = out.float().cpu().numpy()
    assert np.all(o[0, :2] == 0)
    assert_close(o, ref, what="n < T")


def test_multi_token_llama3_shape():
    """The Llama-3-8B-shaped GQA layer (K2/V4, G32, R128) at context 8192 for 4
    sequences, T = 4 (16 rows per KV head), sampled sequences by the oracle."""
    w = synth.WORKLOADS[3]
    B, T = 4, 4
    lens = np.array([8192, 8193, 8195, 8320], np.int32)  # window fill 128, 1, 3, 128
    C = synth.capacity_for(w, 256)
    g, og = geoms(B, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_bits, w.v_bits, w.group,
                  w.residual, C)
    k = synth.keys(w, int(lens.max()), batch=B)
    v = synth.values(w, int(lens.max()), batch=B)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((B, T, w.n_q_heads, w.head_dim)).astype(np.float16)
    _say(f"multi llama3 shape T={T} lens {lens.tolist()}")
    cache, oc = prefill_both(g, og, k, v, lens)
    out, ref = _run(g, og, cache, oc, q, lens, T, scale=1 / math.sqrt(w.head_dim))
    assert_close(out, ref, what="llama3 T=4")
