"""libkvq: KIVI-style quantized KV cache + fused single-token decode attention
for AMD Instinct MI355X (gfx950).

The computation lives in libkvq.so (hand-written HIP kernels behind the C ABI
in include/kvq.h); this package is its thin ctypes binding plus the seeded
synthetic workloads and the byte accounting used by the benchmark.
"""
from ._lib import (  # noqa: F401
    ABI_VERSION, LAYOUT_VERSION, Cache, Geom, KvqError, alloc_workspace,
    kvq_abi_version, kvq_append, kvq_cache_bytes, kvq_decode_attn,
    kvq_decode_combine, kvq_decode_partial, kvq_decode_workers,
    kvq_decode_workspace_bytes, kvq_layout_version, kvq_prefill,
    kvq_quantize_keys_perchannel, kvq_quantize_values_pertoken,
    kvq_validate_geom, last_error, lib, status_str)
