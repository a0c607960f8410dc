"""kvq_decode_attn_noalloc (decode attention with the library's static
partials buffer, for callers that cannot allocate) against kvq_decode_attn with
a caller-allocated workspace, through the C ABI.  Both run the same kernels, so
the outputs must agree bit for bit; both are also held to |gpu - oracle| <=
1e-3 * (1 + |oracle|) against the CPU oracle.  Calls come in a row on one
device, the second with a smaller input than the first, so a stale partial
left in the shared buffer by the first call would show up in the second."""
import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_amd as kvq

from kvq_testutil import assert_close, dev, geoms, prefill_both

pytestmark = pytest.mark.gpu

CANARY16 = 0x7E5A  # a NaN pattern: an output element left unwritten shows


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(B, Hq, Hkv, D, bK, bV, G, R, lens, seed):
    lens = np.asarray(lens, np.int32)
    C = ((int(lens.max()) + R - 1) // R + 1) * R
    g, og = geoms(B, Hq, Hkv, D, bK, bV, G, R, C)
    rng = np.random.default_rng(seed)
    n = int(lens.max())
    k = (rng.standard_normal((B, Hkv, n, D)) *
         rng.lognormal(0, 0.5, (1, Hkv, 1, D))).astype(np.float16)
    v = rng.standard_normal((B, Hkv, n, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    cache, oc = prefill_both(g, og, k, v, lens)
    return g, og, cache, oc, q, lens


def _both(g, og, cache, oc, q, lens, what):
    msl = int(lens.max())
    scale = 1.0 / np.sqrt(g.head_dim)
    qd, ld = dev(q), dev(lens)
    shape = (g.batch, g.n_q_heads, g.head_dim)
    ref_out = torch.empty(shape, dtype=torch.float16, device="cuda")
    ws = kvq.alloc_workspace(g, msl)
    kvq.kvq_decode_attn(g, qd, cache, ld, msl, scale, ws, ref_out)
    got = torch.full(shape, CANARY16, dtype=torch.int16, device="cuda").view(torch.float16)
    _say(f"noalloc {what}: B={g.batch} Hq={g.n_q_heads} Hkv={g.n_kv_heads} D={g.head_dim} "
         f"K{g.k_bits}V{g.v_bits} G{g.group} R{g.residual} lens {lens.min()}..{lens.max()}")
    kvq.kvq_decode_attn_noalloc(g, qd, cache, ld, msl, scale, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16)), \
        f"{what}: noalloc differs from kvq_decode_attn"
    ref = oracle.decode_attn(og, oc, q, lens, float(np.float32(scale)))
    assert_close(got, ref, what=what)


def test_noalloc_two_calls_in_a_row_second_smaller():
    # Llama-3-8B-shaped GQA layer, ragged lengths across chunk and window edges
    big = _case(32, 32, 8, 128, 2, 4, 32, 128,
                [1, 31, 32, 33, 127, 128, 129, 255, 256, 257] + list(range(1000, 3200, 100)),
                seed=11)
    small = _case(3, 8, 2, 64, 4, 2, 32, 32, [1, 40, 97], seed=12)
    _both(*big, "first call (large)")
    _both(*small, "second call (smaller)")
    _both(*big, "third call (large again)")


def test_noalloc_rejects_a_geometry_beyond_its_buffer():
    # 256 x 8 units of 16 query rows: the partials alone need 256*8*16*132*4
    # bytes (17.3 MB), above the 16 MiB static buffer
    g = kvq.Geom(256, 128, 8, 128, 2, 2, 32, 32, 32)
    need = kvq.kvq_decode_workspace_bytes(g, 32)
    assert need > kvq._lib.NOALLOC_SCRATCH_BYTES
    cache = kvq.Cache(g)
    q = torch.zeros((256, 128, 128), dtype=torch.float16, device="cuda")
    out = torch.zeros_like(q)
    lens = torch.full((256,), 32, dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn_noalloc(g, q, cache, lens, 32, 0.125, out)
    assert e.value.status == kvq._lib.KVQ_ERR_WORKSPACE and "static buffer" in str(e.value)
    torch.cuda.synchronize()
    assert not torch.any(out != 0)
