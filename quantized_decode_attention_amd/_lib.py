"""ctypes binding of libkvq (argument marshalling only).

Every function here has the name of a C entry point in include/kvq.h or
include/kvq_bq2.h and does
nothing but check the torch tensors it is handed (device, dtype, contiguity,
shape), pass their data pointers and the current HIP stream, and turn a
non-zero status into an exception.  All computation runs in the library's HIP
kernels; there is no fallback.  PyTorch only provides device memory and
streams.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

ABI_VERSION = 2
LAYOUT_VERSION = 3
VBLOCK = 32

# status codes (include/kvq.h)
KVQ_OK = 0
KVQ_ERR_NULL = -1
KVQ_ERR_GEOM = -2
KVQ_ERR_BITS = -3
KVQ_ERR_ALIGN = -4
KVQ_ERR_WORKSPACE = -5
KVQ_ERR_RANGE = -6
KVQ_ERR_HIP = -7
KVQ_ERR_INTERNAL = -8
NOALLOC_SCRATCH_BYTES = 16 << 20  # KVQ_NOALLOC_SCRATCH_BYTES

EXPORTS = [
    "kvq_abi_version", "kvq_layout_version", "kvq_status_str", "kvq_last_error",
    "kvq_validate_geom", "kvq_cache_bytes", "kvq_decode_workers",
    "kvq_decode_workspace_bytes", "kvq_quantize_keys_perchannel",
    "kvq_quantize_values_pertoken", "kvq_prefill", "kvq_append", "kvq_append_tokens",
    "kvq_decode_attn", "kvq_decode_partial", "kvq_decode_combine",
    "kvq_decode_multi_workspace_bytes", "kvq_decode_attn_multi", "kvq_decode_attn_noalloc",
]
EXPORTS_BQ2 = [
    "kvq_bq2_validate_geom", "kvq_bq2_cache_bytes", "kvq_bq2_decode_workers",
    "kvq_bq2_decode_workspace_bytes", "kvq_bq2_prefill", "kvq_bq2_append",
    "kvq_bq2_decode_attn", "kvq_bq2_decode_partial", "kvq_bq2_decode_combine",
]
EXPORTS_PAGED = [
    "kvq_paged_validate", "kvq_paged_cache_bytes", "kvq_paged_decode_workspace_bytes",
    "kvq_paged_prefill", "kvq_paged_append", "kvq_paged_append_tokens", "kvq_paged_decode_attn",
    "kvq_paged_decode_partial", "kvq_paged_decode_combine", "kvq_paged_decode_attn_multi",
]
EXPORTS_PROBE = ["kvq_probe_stream_read", "kvq_probe_sink_words", "kvq_probe_stream_read_sweep",
                 "kvq_probe_chunk_stream"]
BQ2_HEAD_DIM = 64
BQ2_SINKS = 4


class kvq_geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "k_bits", "v_bits",
        "group", "residual", "capacity", "residual_v")]


class kvq_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_codes", "v_codes", "k_meta", "v_meta", "k_res", "v_res")]


class kvq_bq2_geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "n_q_heads", "n_kv_heads", "capacity")]


class kvq_bq2_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_codes", "v_codes", "k_meta", "v_meta", "k_sink", "v_sink")]


class kvq_paged_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_codes", "v_codes", "k_meta", "v_meta", "k_res", "v_res", "block_table")] + [
        (n, ctypes.c_int32) for n in ("page_size", "max_pages", "num_pages")]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what} failed: {detail or status_str(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Loads the in-tree libkvq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -c "
                "'import __graft_entry__; __graft_entry__.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        G = ctypes.POINTER(kvq_geom)
        C = ctypes.POINTER(kvq_cache)
        G2 = ctypes.POINTER(kvq_bq2_geom)
        C2 = ctypes.POINTER(kvq_bq2_cache)
        f32 = ctypes.c_float
        CP = ctypes.POINTER(kvq_paged_cache)
        sig = {
            "kvq_probe_stream_read": (ctypes.c_int, [P, sz, P, P]),
            "kvq_probe_sink_words": (ctypes.c_int, [ctypes.POINTER(i32)]),
            "kvq_probe_stream_read_sweep": (ctypes.c_int, [P, sz, P, i32, i32, i32, P]),
            "kvq_probe_chunk_stream": (ctypes.c_int, [P, P, P, P, ctypes.c_int64, i32, i32, i32,
                                                      i32, i32, P, P]),
            "kvq_paged_validate": (ctypes.c_int, [G, CP]),
            "kvq_paged_cache_bytes": (ctypes.c_int, [G, i32, i32, ctypes.POINTER(sz)]),
            "kvq_paged_decode_workspace_bytes": (ctypes.c_int, [G, i32, i32, ctypes.POINTER(sz)]),
            "kvq_paged_prefill": (ctypes.c_int, [G, P, P, i32, CP, P]),
            "kvq_paged_append": (ctypes.c_int, [G, P, P, P, CP, P]),
            "kvq_paged_append_tokens": (ctypes.c_int, [G, ctypes.c_int32, P, P, P, CP, P]),
            "kvq_paged_decode_attn": (ctypes.c_int, [G, P, CP, P, i32, f32, P, sz, P, P]),
            "kvq_paged_decode_partial": (ctypes.c_int, [G, P, CP, P, i32, f32, P, sz, P, P]),
            "kvq_paged_decode_combine": (ctypes.c_int, [G, P, CP, P, i32, f32, P, sz, P, P]),
            "kvq_paged_decode_attn_multi": (ctypes.c_int, [G, P, CP, P, i32, i32, f32, P, sz, P,
                                                           P]),
            "kvq_abi_version": (ctypes.c_int, []),
            "kvq_layout_version": (ctypes.c_int, []),
            "kvq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "kvq_last_error": (ctypes.c_char_p, []),
            "kvq_validate_geom": (ctypes.c_int, [G]),
            "kvq_cache_bytes": (ctypes.c_int, [G, ctypes.POINTER(sz)]),
            "kvq_decode_workers": (ctypes.c_int, [G, ctypes.POINTER(i32)]),
            "kvq_decode_workspace_bytes": (ctypes.c_int, [G, i32, ctypes.POINTER(sz)]),
            "kvq_quantize_keys_perchannel": (ctypes.c_int, [G, P, i32, i32, P, P, P]),
            "kvq_quantize_values_pertoken": (ctypes.c_int, [G, P, i32, i32, P, P, P]),
            "kvq_prefill": (ctypes.c_int, [G, P, P, i32, C, P]),
            "kvq_append": (ctypes.c_int, [G, P, P, P, C, P]),
            "kvq_append_tokens": (ctypes.c_int, [G, ctypes.c_int32, P, P, P, C, P]),
            "kvq_decode_attn": (ctypes.c_int, [G, P, C, P, i32, ctypes.c_float, P, sz, P, P]),
            "kvq_decode_partial": (ctypes.c_int, [G, P, C, P, i32, ctypes.c_float, P, sz, P, P]),
            "kvq_decode_combine": (ctypes.c_int, [G, P, C, P, i32, ctypes.c_float, P, sz, P, P]),
            "kvq_decode_attn_noalloc": (ctypes.c_int, [G, P, C, P, i32, f32, P, P]),
            "kvq_decode_multi_workspace_bytes": (ctypes.c_int, [G, i32, i32, ctypes.POINTER(sz)]),
            "kvq_decode_attn_multi": (ctypes.c_int, [G, P, C, P, i32, i32, f32, P, sz, P, P]),
            "kvq_bq2_validate_geom": (ctypes.c_int, [G2]),
            "kvq_bq2_cache_bytes": (ctypes.c_int, [G2, ctypes.POINTER(sz)]),
            "kvq_bq2_decode_workers": (ctypes.c_int, [G2, ctypes.POINTER(i32)]),
            "kvq_bq2_decode_workspace_bytes": (ctypes.c_int, [G2, i32, ctypes.POINTER(sz)]),
            "kvq_bq2_prefill": (ctypes.c_int, [G2, P, P, i32, C2, P]),
            "kvq_bq2_append": (ctypes.c_int, [G2, P, P, P, C2, P]),
            "kvq_bq2_decode_attn": (ctypes.c_int, [G2, P, C2, P, i32, f32, P, sz, P, P]),
            "kvq_bq2_decode_partial": (ctypes.c_int, [G2, P, C2, P, i32, f32, P, sz, P, P]),
            "kvq_bq2_decode_combine": (ctypes.c_int, [G2, P, C2, P, i32, f32, P, sz, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().kvq_status_str(status).decode()


def last_error() -> str:
    return lib().kvq_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, what, last_error())


@dataclass(frozen=True)
class Geom:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    k_bits: int
    v_bits: int
    group: int
    residual: int
    capacity: int
    residual_v: int = 0  # value window length; 0: the same as residual

    @property
    def rv(self) -> int:
        """Value window length."""
        return self.residual_v or self.residual

    def c(self) -> kvq_geom:
        return kvq_geom(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                        self.k_bits, self.v_bits, self.group, self.residual,
                        self.capacity, self.residual_v)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor | None, name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


_F16 = (torch.float16, torch.int16)
_I32 = (torch.int32,)


# ---------------------------------------------------------------- queries --
def kvq_abi_version() -> int:
    return lib().kvq_abi_version()


def kvq_layout_version() -> int:
    return lib().kvq_layout_version()


def kvq_validate_geom(g: Geom) -> None:
    gc = g.c()
    _check(lib().kvq_validate_geom(ctypes.byref(gc)), "kvq_validate_geom")


def kvq_cache_bytes(g: Geom) -> list[int]:
    gc = g.c()
    out = (ctypes.c_size_t * 6)()
    _check(lib().kvq_cache_bytes(ctypes.byref(gc), out), "kvq_cache_bytes")
    return list(out)


def kvq_decode_workers(g: Geom) -> int:
    gc = g.c()
    nw = ctypes.c_int32()
    _check(lib().kvq_decode_workers(ctypes.byref(gc), ctypes.byref(nw)),
           "kvq_decode_workers")
    return nw.value


def kvq_decode_workspace_bytes(g: Geom, max_seq_len: int) -> int:
    gc = g.c()
    out = ctypes.c_size_t()
    _check(lib().kvq_decode_workspace_bytes(ctypes.byref(gc), max_seq_len,
                                            ctypes.byref(out)), "kvq_decode_workspace_bytes")
    return out.value


# ------------------------------------------------------------------ cache --
class Cache:
    """The six cache buffers of one layer as torch device tensors (allocated
    here with torch, sized by kvq_cache_bytes, laid out as include/kvq.h
    specifies)."""

    def __init__(self, g: Geom, device="cuda"):
        B, H, C, D = g.batch, g.n_kv_heads, g.capacity, g.head_dim
        self.g = g
        z = dict(device=device)
        blocks = C // VBLOCK
        self.k_codes = torch.zeros((B, H, blocks, 64, 2, D * g.k_bits // 128),
                                   dtype=torch.int32, **z)
        self.v_codes = torch.zeros((B, H, blocks, 64, D * g.v_bits // 64),
                                   dtype=torch.int32, **z)
        self.k_meta = torch.zeros((B, H, C // g.group, D // 8, 8, 2), dtype=torch.int16, **z)
        self.v_meta = torch.zeros((B, H, blocks, 4, D // g.group, 8, 2),
                                  dtype=torch.int16, **z)
        self.k_res = torch.zeros((B, H, g.residual, D), dtype=torch.float16, **z)
        self.v_res = torch.zeros((B, H, g.rv // 32, D // 16, 64, 8),
                                 dtype=torch.float16, **z)
        sizes = kvq_cache_bytes(g)
        for t, s in zip(self.tensors(), sizes):
            assert t.numel() * t.element_size() == s

    def tensors(self):
        return (self.k_codes, self.v_codes, self.k_meta, self.v_meta, self.k_res,
                self.v_res)

    def view(self, b0: int, b1: int) -> "Cache":
        """Sequences [b0, b1) as a cache of batch b1 - b0 sharing this memory
        (the layout is batch-major, so a batch slice is one contiguous piece)."""
        c = Cache.__new__(Cache)
        c.g = Geom(b1 - b0, *[getattr(self.g, f) for f in (
            "n_q_heads", "n_kv_heads", "head_dim", "k_bits", "v_bits", "group",
            "residual", "capacity", "residual_v")])
        for name in ("k_codes", "v_codes", "k_meta", "v_meta", "k_res", "v_res"):
            setattr(c, name, getattr(self, name)[b0:b1])
        return c

    def c(self) -> kvq_cache:
        return kvq_cache(*[t.data_ptr() for t in self.tensors()])


def _cache_arg(cache: Cache):
    for t in cache.tensors():
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("cache tensors must be contiguous device tensors")
    return cache.c()


# ------------------------------------------------------------- operations --
def kvq_quantize_keys_perchannel(g: Geom, k: torch.Tensor, pos0: int,
                                 k_codes: torch.Tensor, k_meta: torch.Tensor,
                                 stream=None) -> None:
    n_tok = k.shape[2]
    gc = g.c()
    _check(lib().kvq_quantize_keys_perchannel(
        ctypes.byref(gc),
        _ptr(k, "k", _F16, (g.batch, g.n_kv_heads, n_tok, g.head_dim)), pos0, n_tok,
        _ptr(k_codes, "k_codes"), _ptr(k_meta, "k_meta"), _stream(stream)),
        "kvq_quantize_keys_perchannel")


def kvq_quantize_values_pertoken(g: Geom, v: torch.Tensor, pos0: int,
                                 v_codes: torch.Tensor, v_meta: torch.Tensor,
                                 stream=None) -> None:
    n_tok = v.shape[2]
    gc = g.c()
    _check(lib().kvq_quantize_values_pertoken(
        ctypes.byref(gc),
        _ptr(v, "v", _F16, (g.batch, g.n_kv_heads, n_tok, g.head_dim)), pos0, n_tok,
        _ptr(v_codes, "v_codes"), _ptr(v_meta, "v_meta"), _stream(stream)),
        "kvq_quantize_values_pertoken")


def kvq_prefill(g: Geom, k: torch.Tensor, v: torch.Tensor, n: int, cache: Cache,
                stream=None) -> None:
    shape = (g.batch, g.n_kv_heads, n, g.head_dim)
    gc = g.c()
    cc = _cache_arg(cache)
    _check(lib().kvq_prefill(ctypes.byref(gc), _ptr(k, "k", _F16, shape),
                             _ptr(v, "v", _F16, shape), n, ctypes.byref(cc),
                             _stream(stream)), "kvq_prefill")


def kvq_append(g: Geom, k_new: torch.Tensor, v_new: torch.Tensor,
               seq_lens: torch.Tensor, cache: Cache, stream=None) -> None:
    shape = (g.batch, g.n_kv_heads, g.head_dim)
    gc = g.c()
    cc = _cache_arg(cache)
    _check(lib().kvq_append(ctypes.byref(gc), _ptr(k_new, "k_new", _F16, shape),
                            _ptr(v_new, "v_new", _F16, shape),
                            _ptr(seq_lens, "seq_lens", _I32, (g.batch,)),
                            ctypes.byref(cc), _stream(stream)), "kvq_append")


def kvq_append_tokens(g: Geom, T: int, k_new: torch.Tensor, v_new: torch.Tensor,
                      seq_lens: torch.Tensor, cache: Cache, stream=None) -> None:
    """T new tokens per sequence, k_new / v_new [B][T][Hkv][D], in one launch."""
    shape = (g.batch, T, g.n_kv_heads, g.head_dim)
    gc = g.c()
    cc = _cache_arg(cache)
    _check(lib().kvq_append_tokens(ctypes.byref(gc), T, _ptr(k_new, "k_new", _F16, shape),
                                   _ptr(v_new, "v_new", _F16, shape),
                                   _ptr(seq_lens, "seq_lens", _I32, (g.batch,)),
                                   ctypes.byref(cc), _stream(stream)), "kvq_append_tokens")


def _decode_args(g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out):
    gc = g.c()
    cc = _cache_arg(cache)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (ctypes.byref(gc),
            _ptr(q, "q", _F16, (g.batch, g.n_q_heads, g.head_dim)),
            ctypes.byref(cc), _ptr(seq_lens, "seq_lens", _I32, (g.batch,)),
            int(max_seq_len), float(sm_scale), _ptr(workspace, "workspace"),
            ws_bytes, _ptr(out, "out", _F16, (g.batch, g.n_q_heads, g.head_dim))), (gc, cc)


def kvq_decode_attn(g: Geom, q: torch.Tensor, cache: Cache, seq_lens: torch.Tensor,
                    max_seq_len: int, sm_scale: float, workspace: torch.Tensor | None,
                    out: torch.Tensor, stream=None) -> None:
    args, keep = _decode_args(g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out)
    _check(lib().kvq_decode_attn(*args, _stream(stream)), "kvq_decode_attn")


def kvq_decode_attn_noalloc(g: Geom, q: torch.Tensor, cache: Cache, seq_lens: torch.Tensor,
                            max_seq_len: int, sm_scale: float, out: torch.Tensor,
                            stream=None) -> None:
    """kvq_decode_attn with the library's static partials buffer (no workspace)."""
    gc = g.c()
    cc = _cache_arg(cache)
    _check(lib().kvq_decode_attn_noalloc(
        ctypes.byref(gc), _ptr(q, "q", _F16, (g.batch, g.n_q_heads, g.head_dim)),
        ctypes.byref(cc), _ptr(seq_lens, "seq_lens", _I32, (g.batch,)), int(max_seq_len),
        float(sm_scale), _ptr(out, "out", _F16, (g.batch, g.n_q_heads, g.head_dim)),
        _stream(stream)), "kvq_decode_attn_noalloc")


def kvq_decode_partial(g: Geom, q: torch.Tensor, cache: Cache, seq_lens: torch.Tensor,
                       max_seq_len: int, sm_scale: float, workspace: torch.Tensor | None,
                       out: torch.Tensor, stream=None) -> None:
    args, keep = _decode_args(g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out)
    _check(lib().kvq_decode_partial(*args, _stream(stream)), "kvq_decode_partial")


def kvq_decode_combine(g: Geom, q: torch.Tensor, cache: Cache, seq_lens: torch.Tensor,
                       max_seq_len: int, sm_scale: float, workspace: torch.Tensor | None,
                       out: torch.Tensor, stream=None) -> None:
    args, keep = _decode_args(g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out)
    _check(lib().kvq_decode_combine(*args, _stream(stream)), "kvq_decode_combine")


def kvq_decode_multi_workspace_bytes(g: Geom, T: int, max_seq_len: int) -> int:
    gc = g.c()
    out = ctypes.c_size_t()
    _check(lib().kvq_decode_multi_workspace_bytes(ctypes.byref(gc), T, max_seq_len,
                                                  ctypes.byref(out)),
           "kvq_decode_multi_workspace_bytes")
    return out.value


def kvq_decode_attn_multi(g: Geom, q: torch.Tensor, cache: Cache, seq_lens: torch.Tensor,
                          T: int, max_seq_len: int, sm_scale: float,
                          workspace: torch.Tensor | None, out: torch.Tensor,
                          stream=None) -> None:
    gc = g.c()
    cc = _cache_arg(cache)
    shape = (g.batch, T, g.n_q_heads, g.head_dim)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kvq_decode_attn_multi(
        ctypes.byref(gc), _ptr(q, "q", _F16, shape), ctypes.byref(cc),
        _ptr(seq_lens, "seq_lens", _I32, (g.batch,)), int(T), int(max_seq_len),
        float(sm_scale), _ptr(workspace, "workspace"), ws_bytes, _ptr(out, "out", _F16, shape),
        _stream(stream)), "kvq_decode_attn_multi")


def alloc_multi_workspace(g: Geom, T: int, max_seq_len: int, device="cuda") -> torch.Tensor:
    n = kvq_decode_multi_workspace_bytes(g, T, max_seq_len)
    return torch.empty(n // 4, dtype=torch.float32, device=device)


# ------------------------------------------------------------ paged cache --
class PagedCache:
    """Page pools, per-sequence residual windows and block table of one layer
    (include/kvq_paged.h): pools of `num_pages` pages of `page_size` positions
    for every KV head; block_table is a device int32 [B][max_pages] tensor
    (entry [b][j]: the pool page holding positions [j P, (j+1) P) of sequence b)."""

    def __init__(self, g: Geom, page_size: int, num_pages: int, block_table: torch.Tensor,
                 device="cuda"):
        P, H, D, G = page_size, g.n_kv_heads, g.head_dim, g.group
        self.g, self.page_size, self.num_pages = g, page_size, num_pages
        z = dict(device=device)
        self.k_codes = torch.zeros((num_pages, H, P // VBLOCK, 64, 2, D * g.k_bits // 128),
                                   dtype=torch.int32, **z)
        self.v_codes = torch.zeros((num_pages, H, P // VBLOCK, 64, D * g.v_bits // 64),
                                   dtype=torch.int32, **z)
        self.k_meta = torch.zeros((num_pages, H, P // G, D // 8, 8, 2), dtype=torch.int16, **z)
        self.v_meta = torch.zeros((num_pages, H, P // VBLOCK, 4, D // G, 8, 2),
                                  dtype=torch.int16, **z)
        self.k_res = torch.zeros((g.batch, H, g.residual, D), dtype=torch.float16, **z)
        self.v_res = torch.zeros((g.batch, H, g.rv // 32, D // 16, 64, 8),
                                 dtype=torch.float16, **z)
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
                block_table.shape[0] != g.batch or not block_table.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 [batch][max_pages] tensor")
        self.block_table = block_table
        self.max_pages = block_table.shape[1]
        sizes = kvq_paged_cache_bytes(g, page_size, num_pages)
        for t, n in zip(self.tensors(), sizes):
            assert t.numel() * t.element_size() == n

    def tensors(self):
        return (self.k_codes, self.v_codes, self.k_meta, self.v_meta, self.k_res,
                self.v_res)

    def view(self, b0: int, b1: int) -> "PagedCache":
        """Sequences [b0, b1) as a paged cache of batch b1 - b0: the same pools,
        those sequences' residual windows and table rows."""
        c = PagedCache.__new__(PagedCache)
        c.g = Geom(b1 - b0, *[getattr(self.g, f) for f in (
            "n_q_heads", "n_kv_heads", "head_dim", "k_bits", "v_bits", "group",
            "residual", "capacity", "residual_v")])
        c.page_size, c.num_pages, c.max_pages = self.page_size, self.num_pages, self.max_pages
        c.k_codes, c.v_codes, c.k_meta, c.v_meta = (self.k_codes, self.v_codes, self.k_meta,
                                                    self.v_meta)
        c.k_res, c.v_res = self.k_res[b0:b1], self.v_res[b0:b1]
        c.block_table = self.block_table[b0:b1]
        return c

    def c(self) -> kvq_paged_cache:
        for t in self.tensors() + (self.block_table,):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("paged cache tensors must be contiguous device tensors")
        return kvq_paged_cache(*[t.data_ptr() for t in self.tensors()],
                               self.block_table.data_ptr(), self.page_size, self.max_pages,
                               self.num_pages)


def kvq_paged_validate(g: Geom, page_size: int, max_pages: int, num_pages: int) -> None:
    gc = g.c()
    cc = kvq_paged_cache(None, None, None, None, None, None, None, page_size, max_pages,
                         num_pages)
    _check(lib().kvq_paged_validate(ctypes.byref(gc), ctypes.byref(cc)), "kvq_paged_validate")


def kvq_paged_cache_bytes(g: Geom, page_size: int, num_pages: int) -> list[int]:
    gc = g.c()
    out = (ctypes.c_size_t * 6)()
    _check(lib().kvq_paged_cache_bytes(ctypes.byref(gc), page_size, num_pages, out),
           "kvq_paged_cache_bytes")
    return list(out)


def kvq_paged_decode_workspace_bytes(g: Geom, T: int, max_seq_len: int) -> int:
    gc = g.c()
    out = ctypes.c_size_t()
    _check(lib().kvq_paged_decode_workspace_bytes(ctypes.byref(gc), T, max_seq_len,
                                                  ctypes.byref(out)),
           "kvq_paged_decode_workspace_bytes")
    return out.value


def alloc_paged_workspace(g: Geom, T: int, max_seq_len: int, device="cuda") -> torch.Tensor:
    n = kvq_paged_decode_workspace_bytes(g, T, max_seq_len)
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def kvq_paged_prefill(g: Geom, k: torch.Tensor, v: torch.Tensor, n: int, cache: PagedCache,
                      stream=None) -> None:
    shape = (g.batch, g.n_kv_heads, n, g.head_dim)
    gc = g.c()
    cc = cache.c()
    _check(lib().kvq_paged_prefill(ctypes.byref(gc), _ptr(k, "k", _F16, shape),
                                   _ptr(v, "v", _F16, shape), n, ctypes.byref(cc),
                                   _stream(stream)), "kvq_paged_prefill")


def kvq_paged_append(g: Geom, k_new: torch.Tensor, v_new: torch.Tensor,
                     seq_lens: torch.Tensor, cache: PagedCache, stream=None) -> None:
    shape = (g.batch, g.n_kv_heads, g.head_dim)
    gc = g.c()
    cc = cache.c()
    _check(lib().kvq_paged_append(ctypes.byref(gc), _ptr(k_new, "k_new", _F16, shape),
                                  _ptr(v_new, "v_new", _F16, shape),
                                  _ptr(seq_lens, "seq_lens", _I32, (g.batch,)),
                                  ctypes.byref(cc), _stream(stream)), "kvq_paged_append")


def kvq_paged_append_tokens(g: Geom, T: int, k_new: torch.Tensor, v_new: torch.Tensor,
                            seq_lens: torch.Tensor, cache: PagedCache, stream=None) -> None:
    shape = (g.batch, T, g.n_kv_heads, g.head_dim)
    gc = g.c()
    cc = cache.c()
    _check(lib().kvq_paged_append_tokens(ctypes.byref(gc), T, _ptr(k_new, "k_new", _F16, shape),
                                         _ptr(v_new, "v_new", _F16, shape),
                                         _ptr(seq_lens, "seq_lens", _I32, (g.batch,)),
                                         ctypes.byref(cc), _stream(stream)),
           "kvq_paged_append_tokens")


def kvq_paged_decode_attn_multi(g: Geom, q: torch.Tensor, cache: PagedCache,
                                seq_lens: torch.Tensor, T: int, max_seq_len: int,
                                sm_scale: float, workspace: torch.Tensor | None,
                                out: torch.Tensor, stream=None) -> None:
    gc = g.c()
    cc = cache.c()
    shape = (g.batch, T, g.n_q_heads, g.head_dim)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kvq_paged_decode_attn_multi(
        ctypes.byref(gc), _ptr(q, "q", _F16, shape), ctypes.byref(cc),
        _ptr(seq_lens, "seq_lens", _I32, (g.batch,)), int(T), int(max_seq_len),
        float(sm_scale), _ptr(workspace, "workspace"), ws_bytes, _ptr(out, "out", _F16, shape),
        _stream(stream)), "kvq_paged_decode_attn_multi")


def _paged_call(name, g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out, stream):
    gc = g.c()
    cc = cache.c()
    shape = (g.batch, g.n_q_heads, g.head_dim)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(getattr(lib(), name)(
        ctypes.byref(gc), _ptr(q, "q", _F16, shape), ctypes.byref(cc),
        _ptr(seq_lens, "seq_lens", _I32, (g.batch,)), int(max_seq_len), float(sm_scale),
        _ptr(workspace, "workspace"), ws_bytes, _ptr(out, "out", _F16, shape),
        _stream(stream)), name)


def kvq_paged_decode_attn(g: Geom, q: torch.Tensor, cache: PagedCache, seq_lens: torch.Tensor,
                          max_seq_len: int, sm_scale: float, workspace: torch.Tensor | None,
                          out: torch.Tensor, stream=None) -> None:
    _paged_call("kvq_paged_decode_attn", g, q, cache, seq_lens, max_seq_len, sm_scale,
                workspace, out, stream)


def kvq_paged_decode_partial(g: Geom, q: torch.Tensor, cache: PagedCache,
                             seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float,
                             workspace: torch.Tensor | None, out: torch.Tensor,
                             stream=None) -> None:
    _paged_call("kvq_paged_decode_partial", g, q, cache, seq_lens, max_seq_len, sm_scale,
                workspace, out, stream)


def kvq_paged_decode_combine(g: Geom, q: torch.Tensor, cache: PagedCache,
                             seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float,
                             workspace: torch.Tensor | None, out: torch.Tensor,
                             stream=None) -> None:
    _paged_call("kvq_paged_decode_combine", g, q, cache, seq_lens, max_seq_len, sm_scale,
                workspace, out, stream)


def stream_read_gbs(nbytes: int = 2 << 30, reps: int = 20, device="cuda") -> dict:
    """HBM read rate of kvq_probe_stream_read over a buffer of nbytes (well
    beyond the 256 MB Infinity Cache), HIP events around each of reps reads
    (a measurement aid: the practical ceiling of a read-only stream)."""
    words = ctypes.c_int32()
    _check(lib().kvq_probe_sink_words(ctypes.byref(words)), "kvq_probe_sink_words")
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    sink = torch.zeros(words.value, dtype=torch.int32, device=device)
    st = torch.cuda.current_stream()
    times = []
    for r in range(reps + 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        _check(lib().kvq_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                           ctypes.c_void_p(sink.data_ptr()),
                                           ctypes.c_void_p(st.cuda_stream)),
               "kvq_probe_stream_read")
        b.record(st)
        b.synchronize()
        if r >= 2:
            times.append(a.elapsed_time(b) / 1e3)
    del buf
    t = float(np.median(times))
    return {"gbs": round(nbytes / t / 1e9, 1), "bytes": nbytes, "reps": reps,
            "median_us": round(t * 1e6, 2)}


def stream_read_sweep(shapes, nbytes: int = 2 << 30, reps: int = 10, device="cuda") -> list:
    """HBM read rate of kvq_probe_stream_read_sweep for each (waves_per_simd,
    loads_per_lane, nontemporal) in shapes: the median of reps reads of nbytes
    (HIP events around each).  A measurement aid."""
    words = ctypes.c_int32()
    _check(lib().kvq_probe_sink_words(ctypes.byref(words)), "kvq_probe_sink_words")
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    sink = torch.zeros(words.value, dtype=torch.int32, device=device)
    st = torch.cuda.current_stream()
    out = []
    for wps, loads, nt in shapes:
        times = []
        for r in range(reps + 2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            _check(lib().kvq_probe_stream_read_sweep(
                ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                int(wps), int(loads), int(nt), ctypes.c_void_p(st.cuda_stream)),
                "kvq_probe_stream_read_sweep")
            b.record(st)
            b.synchronize()
            if r >= 2:
                times.append(a.elapsed_time(b) / 1e3)
        t = float(np.median(times))
        out.append({"waves_per_simd": wps, "loads_per_lane": loads,
                    "load": ("plain", "nontemporal", "lds nontemporal", "lds plain")[nt],
                    "bytes_in_flight_per_wave": [64 * 16 * loads, 2 * 64 * 16 * loads],
                    "gbs": round(nbytes / t / 1e9, 1), "median_us": round(t * 1e6, 2)})
    del buf
    return out


def chunk_stream(piece_bytes, n_chunks: int, spins, copies: int = 4, reps: int = 20,
                 device="cuda") -> list:
    """Rate of kvq_probe_chunk_stream (the decode partial kernel's load stream
    without its arithmetic) for chunks of the four given piece sizes, for each
    spin (dependent multiply-adds per chunk).  Launches run back to back in
    rounds of 2 x copies, rotating over copies buffer sets so that the Infinity
    Cache holds none of a launch's bytes, with HIP events around each round
    (as the decode kernel is timed); the median round / launches is reported.
    A measurement aid."""
    words = ctypes.c_int32()
    _check(lib().kvq_probe_sink_words(ctypes.byref(words)), "kvq_probe_sink_words")
    sets = [[torch.ones(n_chunks * b // 4, dtype=torch.int32, device=device) for b in piece_bytes]
            for _ in range(copies)]
    sink = torch.zeros(words.value, dtype=torch.int32, device=device)
    st = torch.cuda.current_stream()

    def launch(k, spin):
        _check(lib().kvq_probe_chunk_stream(
            *[ctypes.c_void_p(x.data_ptr()) for x in sets[k % copies]], int(n_chunks),
            *[int(x) for x in piece_bytes], int(spin), ctypes.c_void_p(sink.data_ptr()),
            ctypes.c_void_p(st.cuda_stream)), "kvq_probe_chunk_stream")

    out = []
    per_round = 2 * copies
    for spin in spins:
        for k in range(copies):
            launch(k, spin)
        times = []
        for r in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            for k in range(per_round):
                launch(k, spin)
            b.record(st)
            b.synchronize()
            times.append(a.elapsed_time(b) / 1e3 / per_round)
        t = float(np.median(times))
        nbytes = n_chunks * sum(piece_bytes)
        out.append({"spin": spin, "median_us": round(t * 1e6, 2),
                    "gbs": round(nbytes / t / 1e9, 1)})
    del sets
    return out


def alloc_workspace(g: Geom, max_seq_len: int, device="cuda") -> torch.Tensor | None:
    n = kvq_decode_workspace_bytes(g, max_seq_len)
    if n == 0:
        return None
    return torch.empty(n // 4, dtype=torch.float32, device=device)


# ------------------------------------------- rotated per-token 2-bit format --
@dataclass(frozen=True)
class Bq2Geom:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    capacity: int

    def c(self) -> kvq_bq2_geom:
        return kvq_bq2_geom(self.batch, self.n_q_heads, self.n_kv_heads, self.capacity)


def kvq_bq2_validate_geom(g: Bq2Geom) -> None:
    gc = g.c()
    _check(lib().kvq_bq2_validate_geom(ctypes.byref(gc)), "kvq_bq2_validate_geom")


def kvq_bq2_cache_bytes(g: Bq2Geom) -> list[int]:
    gc = g.c()
    out = (ctypes.c_size_t * 6)()
    _check(lib().kvq_bq2_cache_bytes(ctypes.byref(gc), out), "kvq_bq2_cache_bytes")
    return list(out)


def kvq_bq2_decode_workers(g: Bq2Geom) -> int:
    gc = g.c()
    nw = ctypes.c_int32()
    _check(lib().kvq_bq2_decode_workers(ctypes.byref(gc), ctypes.byref(nw)),
           "kvq_bq2_decode_workers")
    return nw.value


def kvq_bq2_decode_workspace_bytes(g: Bq2Geom, max_seq_len: int) -> int:
    gc = g.c()
    out = ctypes.c_size_t()
    _check(lib().kvq_bq2_decode_workspace_bytes(ctypes.byref(gc), max_seq_len,
                                                ctypes.byref(out)),
           "kvq_bq2_decode_workspace_bytes")
    return out.value


class Bq2Cache:
    """The six buffers of one layer's cache in the rotated format, as torch
    device tensors laid out as include/kvq_bq2.h specifies."""

    def __init__(self, g: Bq2Geom, device="cuda"):
        B, H, C = g.batch, g.n_kv_heads, g.capacity
        self.g = g
        z = dict(device=device)
        self.k_codes = torch.zeros((B, H, C // 32, 64, 2), dtype=torch.int32, **z)
        self.v_codes = torch.zeros((B, H, C // 32, 64, 2), dtype=torch.int32, **z)
        self.k_meta = torch.zeros((B, H, C, 2), dtype=torch.int16, **z)
        self.v_meta = torch.zeros((B, H, C, 2), dtype=torch.int16, **z)
        self.k_sink = torch.zeros((B, H, BQ2_SINKS, BQ2_HEAD_DIM), dtype=torch.float16, **z)
        self.v_sink = torch.zeros((B, H, BQ2_HEAD_DIM, BQ2_SINKS), dtype=torch.float16, **z)
        for t, n in zip(self.tensors(), kvq_bq2_cache_bytes(g)):
            assert t.numel() * t.element_size() == n

    def tensors(self):
        return (self.k_codes, self.v_codes, self.k_meta, self.v_meta, self.k_sink,
                self.v_sink)

    def c(self) -> kvq_bq2_cache:
        for t in self.tensors():
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("cache tensors must be contiguous device tensors")
        return kvq_bq2_cache(*[t.data_ptr() for t in self.tensors()])


def kvq_bq2_prefill(g: Bq2Geom, k: torch.Tensor, v: torch.Tensor, n: int, cache: Bq2Cache,
                    stream=None) -> None:
    shape = (g.batch, g.n_kv_heads, n, BQ2_HEAD_DIM)
    gc, cc = g.c(), cache.c()
    _check(lib().kvq_bq2_prefill(ctypes.byref(gc), _ptr(k, "k", _F16, shape),
                                 _ptr(v, "v", _F16, shape), n, ctypes.byref(cc),
                                 _stream(stream)), "kvq_bq2_prefill")


def kvq_bq2_append(g: Bq2Geom, k_new: torch.Tensor, v_new: torch.Tensor,
                   seq_lens: torch.Tensor, cache: Bq2Cache, stream=None) -> None:
    shape = (g.batch, g.n_kv_heads, BQ2_HEAD_DIM)
    gc, cc = g.c(), cache.c()
    _check(lib().kvq_bq2_append(ctypes.byref(gc), _ptr(k_new, "k_new", _F16, shape),
                                _ptr(v_new, "v_new", _F16, shape),
                                _ptr(seq_lens, "seq_lens", _I32, (g.batch,)),
                                ctypes.byref(cc), _stream(stream)), "kvq_bq2_append")


def _bq2_decode_args(g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out):
    gc, cc = g.c(), cache.c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    shape = (g.batch, g.n_q_heads, BQ2_HEAD_DIM)
    return (ctypes.byref(gc), _ptr(q, "q", _F16, shape), ctypes.byref(cc),
            _ptr(seq_lens, "seq_lens", _I32, (g.batch,)), int(max_seq_len),
            float(sm_scale), _ptr(workspace, "workspace"), ws_bytes,
            _ptr(out, "out", _F16, shape)), (gc, cc)


def kvq_bq2_decode_attn(g: Bq2Geom, q, cache: Bq2Cache, seq_lens, max_seq_len: int,
                        sm_scale: float, workspace, out, stream=None) -> None:
    args, keep = _bq2_decode_args(g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out)
    _check(lib().kvq_bq2_decode_attn(*args, _stream(stream)), "kvq_bq2_decode_attn")


def kvq_bq2_decode_partial(g: Bq2Geom, q, cache: Bq2Cache, seq_lens, max_seq_len: int,
                           sm_scale: float, workspace, out, stream=None) -> None:
    args, keep = _bq2_decode_args(g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out)
    _check(lib().kvq_bq2_decode_partial(*args, _stream(stream)), "kvq_bq2_decode_partial")


def kvq_bq2_decode_combine(g: Bq2Geom, q, cache: Bq2Cache, seq_lens, max_seq_len: int,
                           sm_scale: float, workspace, out, stream=None) -> None:
    args, keep = _bq2_decode_args(g, q, cache, seq_lens, max_seq_len, sm_scale, workspace, out)
    _check(lib().kvq_bq2_decode_combine(*args, _stream(stream)), "kvq_bq2_decode_combine")


def alloc_bq2_workspace(g: Bq2Geom, max_seq_len: int, device="cuda") -> torch.Tensor:
    n = kvq_bq2_decode_workspace_bytes(g, max_seq_len)
    return torch.empty(n // 4, dtype=torch.float32, device=device)
