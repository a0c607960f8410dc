"""libkvq: KIVI-style quantized KV cache + fused single-token decode attention
for AMD Instinct MI355X (gfx950), and the rotated per-token 2-bit format of
KV1 (BQ2_0).

The computation lives in libkvq.so (hand-written HIP kernels behind the C ABI
in include/kvq.h, include/kvq_paged.h and include/kvq_bq2.h); this package is
its thin ctypes binding plus the seeded synthetic workloads and the byte
accounting used by the benchmark.
"""
from ._lib import (  # noqa: F401
    ABI_VERSION, LAYOUT_VERSION, Cache, Geom, KvqError, alloc_workspace,
    kvq_abi_version, kvq_append, kvq_append_tokens, kvq_cache_bytes, kvq_decode_attn,
    kvq_decode_combine, kvq_decode_partial, kvq_decode_workers,
    kvq_decode_workspace_bytes, kvq_layout_version, kvq_prefill,
    kvq_quantize_keys_perchannel, kvq_quantize_values_pertoken,
    kvq_validate_geom, last_error, lib, status_str)
from ._lib import (  # noqa: F401
    alloc_multi_workspace, kvq_decode_attn_multi, kvq_decode_multi_workspace_bytes)
from ._lib import (  # noqa: F401
    Bq2Cache, Bq2Geom, alloc_bq2_workspace, kvq_bq2_append, kvq_bq2_cache_bytes,
    kvq_bq2_decode_attn, kvq_bq2_decode_combine, kvq_bq2_decode_partial,
    kvq_bq2_decode_workers, kvq_bq2_decode_workspace_bytes, kvq_bq2_prefill,
    kvq_bq2_validate_geom)
from ._lib import (  # noqa: F401
    PagedCache, alloc_paged_workspace, kvq_paged_append, kvq_paged_append_tokens,
    kvq_paged_cache_bytes,
    kvq_paged_decode_attn, kvq_paged_decode_attn_multi, kvq_paged_decode_combine,
    kvq_paged_decode_partial, kvq_paged_decode_workspace_bytes, kvq_paged_prefill,
    kvq_paged_validate)
from ._lib import kvq_decode_attn_noalloc  # noqa: F401
from ._lib import chunk_stream, stream_read_gbs, stream_read_sweep  # noqa: F401  (measurement aids)
