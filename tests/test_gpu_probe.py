"""The measurement aids of kvq_probe.h: the plain stream read and the decode
kernel's chunk stream without its arithmetic.  They are no part of the method;
these tests check that they run and that the chunk stream's arguments are
validated before anything is launched (that part needs no GPU)."""
import ctypes

import pytest

import quantized_decode_attention_amd as kvq
from quantized_decode_attention_amd import _lib


def _chunk_call(pieces, n_chunks=64, spin=0, ptr=16):
    p = ctypes.c_void_p(ptr)  # never dereferenced: every case below fails validation
    return kvq.lib().kvq_probe_chunk_stream(p, p, p, p, n_chunks, *pieces, spin, p,
                                            ctypes.c_void_p(0))


@pytest.mark.parametrize("pieces,n_chunks,spin", [
    ((1024, 2048, 512, 600), 64, 0),      # not a multiple of 512
    ((2048, 2048, 512, 512), 64, 0),      # more than 4096 bytes per chunk
    ((0, 0, 0, 0), 64, 0),                # empty chunk
    ((1024, 2048, 512, 512), 0, 0),       # no chunks
    ((1024, 2048, 512, 512), 64, 5000),   # spin out of range
    ((-512, 2048, 512, 512), 64, 0),      # negative piece
])
def test_chunk_stream_rejects_bad_sizes(pieces, n_chunks, spin):
    assert _chunk_call(pieces, n_chunks, spin) == _lib.KVQ_ERR_RANGE


def test_chunk_stream_rejects_null_buffers():
    L = kvq.lib()
    p = ctypes.c_void_p(16)
    st = L.kvq_probe_chunk_stream(None, p, p, p, 64, 1024, 2048, 512, 512, 0, p, None)
    assert st == _lib.KVQ_ERR_NULL


@pytest.mark.gpu
def test_stream_read_runs():
    r = kvq.stream_read_gbs(nbytes=64 << 20, reps=3)
    assert r["gbs"] > 0


@pytest.mark.gpu
def test_chunk_stream_runs():
    # a small stream in the Llama-3-8B GQA layer's chunk shape; more spin is not faster
    rows = kvq.chunk_stream([1024, 2048, 512, 512], 8192, [0, 256], copies=2, reps=3)
    assert all(r["gbs"] > 0 for r in rows)
    assert rows[1]["median_us"] > 0.5 * rows[0]["median_us"]
