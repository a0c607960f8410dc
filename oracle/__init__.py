"""CPU oracle for KIVI-style quantized KV caches and decode attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the library under test never does.  The
arithmetic lives in ``kvq_oracle.c`` (plain C, fp32 quantizer as the KV1 model
card's "Quantization Format" section fixes it, fp64 dequantization and
attention); this module only builds it and marshals numpy arrays.  Nothing here
is shared with the GPU library: the packed layout and fp16 rounding are
restated independently.

Every function cites the page passage it follows in ``kvq_oracle.c``.  Pins
(tests marked ``not gpu``) tie it to the pages and to independent mathematics.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_SRC_BQ2 = os.path.join(_HERE, "bq2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a separately built library (the sanitizer test loads an instrumented build)
_LIB_OVERRIDE = os.environ.get("KVQ_ORACLE_LIB")

VBLOCK = 32  # tokens per value-code block (layout restated in kvq_oracle.c)


def build_sanitized(out: str) -> str:
    """The same library with AddressSanitizer and UndefinedBehaviorSanitizer
    (host code, gcc; any report aborts), for tests that run the oracle under
    them."""
    cmd = [
        "gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
        "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, _SRC_BQ2, "-o", out, "-lm",
    ]
    subprocess.run(cmd, check=True)
    return out


def build(force: bool = True) -> str:
    """Compiles liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = [
            "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
            "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, _SRC_BQ2,
            "-o", _LIB + ".tmp", "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_half_to_float.restype = ctypes.c_float
        L.orc_half_to_float.argtypes = [ctypes.c_uint16]
        L.orc_float_to_half.restype = ctypes.c_uint16
        L.orc_float_to_half.argtypes = [ctypes.c_float]
        L.orc_float_to_half_array.argtypes = [P, P, i64]
        L.orc_half_to_float_array.argtypes = [P, P, i64]
        L.orc_quantize_group.argtypes = [P, i64, i64, ctypes.c_int, P, P, P, i64]
        L.orc_quantize_keys.argtypes = [ctypes.c_int] * 5 + [i64, P, i64, i64, P, P]
        L.orc_quantize_values.argtypes = [ctypes.c_int] * 5 + [i64, P, i64, i64, P, P]
        L.orc_packed_len.restype = i64
        L.orc_packed_len.argtypes = [i64, ctypes.c_int]
        L.orc_append.argtypes = [ctypes.c_int] * 8 + [i64] + [P] * 9
        L.orc_cache_kv.argtypes = [ctypes.c_int] * 8 + [i64] + [P] * 6 + [i64, P, P]
        L.orc_decode_attn.argtypes = [ctypes.c_int] * 9 + [i64] + [P] * 8 + [f64, P]
        L.orc_decode_attn_multi.argtypes = ([ctypes.c_int] * 9 + [i64, ctypes.c_int] + [P] * 8
                                            + [f64, P])
        L.orc_unpack.argtypes = [ctypes.c_int] * 6 + [i64] + [P] * 8
        L.orc_key_residual_store.argtypes = [ctypes.c_int] * 4 + [P, i64, i64, P]
        L.orc_value_residual_store.argtypes = [ctypes.c_int] * 4 + [P, i64, i64, P]
        L.orc_value_res_rows.argtypes = [ctypes.c_int] * 4 + [P, P]
        L.orc_bq2_hadamard.restype = f64
        L.orc_bq2_hadamard.argtypes = [ctypes.c_int, ctypes.c_int]
        L.orc_bq2_rotate.argtypes = [P, P]
        L.orc_bq2_quantize.argtypes = [P, P, P, P]
        L.orc_bq2_block.argtypes = [ctypes.c_uint16, ctypes.c_uint16, P, P]
        L.orc_bq2_prefill.argtypes = [ctypes.c_int, ctypes.c_int, i64, P, P, i64] + [P] * 6
        L.orc_bq2_append.argtypes = [ctypes.c_int, ctypes.c_int, i64, P, P, P] + [P] * 6
        L.orc_bq2_unpack.argtypes = [ctypes.c_int, ctypes.c_int, i64] + [P] * 4
        L.orc_bq2_cache_kv.argtypes = [ctypes.c_int, ctypes.c_int, i64] + [P] * 6 + [i64, P, P]
        L.orc_bq2_decode_attn.argtypes = ([ctypes.c_int] * 3 + [i64] + [P] * 8 + [f64, P])
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a: np.ndarray) -> np.ndarray:
    """fp16 or uint16 array -> contiguous uint16 view."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


# ---------------------------------------------------------------- fp16 -----
def float_to_half_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().orc_float_to_half_array(_p(x), _p(y), x.size)
    return y


def half_bits_to_float(h: np.ndarray) -> np.ndarray:
    h = _u16(h)
    y = np.empty(h.shape, np.float32)
    lib().orc_half_to_float_array(_p(h), _p(y), h.size)
    return y


# ------------------------------------------------------------ quantizer ----
def quantize_group(x: np.ndarray, bits: int):
    """One group: returns (scale_bits, min_bits, codes uint8[n])."""
    x = _u16(x).ravel().copy()
    n = x.size
    codes = np.zeros(n, np.uint8)
    d = ctypes.c_uint16()
    m = ctypes.c_uint16()
    lib().orc_quantize_group(_p(x), n, 1, bits, ctypes.byref(d), ctypes.byref(m),
                             _p(codes), 1)
    return int(d.value), int(m.value), codes


@dataclass
class Geom:
    """Cache geometry (the oracle's own restatement; plain ints)."""
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
    def rk(self) -> int:
        """Key window length."""
        return self.residual

    @property
    def rv(self) -> int:
        """Value window length."""
        return self.residual_v or self.residual


class Cache:
    """The six packed-cache arrays on the host, laid out as the specification
    states (see kvq_oracle.c)."""

    def __init__(self, g: Geom):
        B, H, C, D = g.batch, g.n_kv_heads, g.capacity, g.head_dim
        self.g = g
        blocks = C // VBLOCK
        self.k_codes = np.zeros((B, H, blocks, 64, 2, D * g.k_bits // 128), np.uint32)
        self.v_codes = np.zeros((B, H, blocks, 64, D * g.v_bits // 64), np.uint32)
        self.k_meta = np.zeros((B, H, C // g.group, D // 8, 8, 2), np.uint16)
        self.v_meta = np.zeros((B, H, blocks, 4, D // g.group, 8, 2), np.uint16)
        self.k_res = np.zeros((B, H, g.rk, D), np.uint16)
        self.v_res = np.zeros((B, H, g.rv // 32, D // 16, 64, 8), np.uint16)

    def arrays(self):
        return (self.k_codes, self.v_codes, self.k_meta, self.v_meta,
                self.k_res, self.v_res)


def quantize_keys(g: Geom, cache: Cache, k: np.ndarray, pos0: int) -> None:
    """k fp16 [B][Hkv][n_tok][D] -> key groups of positions [pos0, pos0+n_tok)."""
    k = _u16(k)
    n_tok = k.shape[2]
    lib().orc_quantize_keys(g.batch, g.n_kv_heads, g.head_dim, g.k_bits, g.group,
                            g.capacity, _p(k), pos0, n_tok, _p(cache.k_codes),
                            _p(cache.k_meta))


def quantize_values(g: Geom, cache: Cache, v: np.ndarray, pos0: int) -> None:
    v = _u16(v)
    n_tok = v.shape[2]
    lib().orc_quantize_values(g.batch, g.n_kv_heads, g.head_dim, g.v_bits,
                              g.group, g.capacity, _p(v), pos0, n_tok,
                              _p(cache.v_codes), _p(cache.v_meta))


def packed_len(n: int, R: int) -> int:
    return int(lib().orc_packed_len(n, R))


def prefill(g: Geom, cache: Cache, k: np.ndarray, v: np.ndarray, n: int) -> None:
    """State after n single-token appends: keys [0, Lq(n, Rk)) packed and the
    rest in the key window; values likewise with Rv."""
    k = _u16(k)
    v = _u16(v)
    lqk, lqv = packed_len(n, g.rk), packed_len(n, g.rv)
    if lqk > 0:
        quantize_keys(g, cache, np.ascontiguousarray(k[:, :, :lqk]), 0)
    if lqv > 0:
        quantize_values(g, cache, np.ascontiguousarray(v[:, :, :lqv]), 0)
    if n > lqk:
        kr = np.ascontiguousarray(k[:, :, lqk:n])
        lib().orc_key_residual_store(g.batch, g.n_kv_heads, g.head_dim, g.rk, _p(kr), lqk,
                                     n - lqk, _p(cache.k_res))
    if n > lqv:
        vr = np.ascontiguousarray(v[:, :, lqv:n])
        lib().orc_value_residual_store(g.batch, g.n_kv_heads, g.head_dim, g.rv, _p(vr), lqv,
                                       n - lqv, _p(cache.v_res))


def value_res_rows(g: Geom, v_res: np.ndarray) -> np.ndarray:
    """A v_res array (any array of the cache's v_res layout and batch) in
    natural order [B][Hkv][R][D] (tests only)."""
    B = v_res.shape[0]
    v_res = np.ascontiguousarray(v_res).view(np.uint16)
    out = np.zeros((B, g.n_kv_heads, g.rv, g.head_dim), np.uint16)
    lib().orc_value_res_rows(B, g.n_kv_heads, g.head_dim, g.rv, _p(v_res), _p(out))
    return out


def append(g: Geom, cache: Cache, k_new: np.ndarray, v_new: np.ndarray,
           seq_lens_before: np.ndarray) -> None:
    k_new = _u16(k_new)
    v_new = _u16(v_new)
    sl = np.ascontiguousarray(seq_lens_before, dtype=np.int32)
    lib().orc_append(g.batch, g.n_kv_heads, g.head_dim, g.k_bits, g.v_bits,
                     g.group, g.rk, g.rv, g.capacity, _p(k_new), _p(v_new),
                     _p(sl), *[_p(a) for a in cache.arrays()])


def cache_kv(g: Geom, cache: Cache, n: int):
    """(K, V) fp64 [B][Hkv][n][D] as the cache represents positions < n."""
    shape = (g.batch, g.n_kv_heads, n, g.head_dim)
    ok = np.zeros(shape, np.float64)
    ov = np.zeros(shape, np.float64)
    lib().orc_cache_kv(g.batch, g.n_kv_heads, g.head_dim, g.k_bits, g.v_bits,
                       g.group, g.rk, g.rv, g.capacity,
                       *[_p(a) for a in cache.arrays()], n, _p(ok), _p(ov))
    return ok, ov


def decode_attn(g: Geom, cache: Cache, q: np.ndarray, seq_lens: np.ndarray,
                sm_scale: float) -> np.ndarray:
    """fp64 [B][Hq][D] attention outputs; seq_lens include the current token."""
    q = _u16(q)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.zeros((g.batch, g.n_q_heads, g.head_dim), np.float64)
    lib().orc_decode_attn(g.batch, g.n_q_heads, g.n_kv_heads, g.head_dim,
                          g.k_bits, g.v_bits, g.group, g.rk, g.rv, g.capacity,
                          _p(q), *[_p(a) for a in cache.arrays()], _p(sl),
                          float(sm_scale), _p(out))
    return out


def decode_attn_multi(g: Geom, cache: Cache, q: np.ndarray, seq_lens: np.ndarray, T: int,
                      sm_scale: float) -> np.ndarray:
    """fp64 [B][T][Hq][D]: query token i of the last T attends causally to
    positions [0, n - T + i]; seq_lens include all T tokens."""
    q = _u16(q)
    assert q.shape == (g.batch, T, g.n_q_heads, g.head_dim)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.zeros((g.batch, T, g.n_q_heads, g.head_dim), np.float64)
    lib().orc_decode_attn_multi(g.batch, g.n_q_heads, g.n_kv_heads, g.head_dim, g.k_bits,
                                g.v_bits, g.group, g.rk, g.rv, g.capacity, T, _p(q),
                                *[_p(a) for a in cache.arrays()], _p(sl), float(sm_scale),
                                _p(out))
    return out


def unpack(g: Geom, cache: Cache):
    """The cache's codes and (scale, min) bits in natural order (tests only):
    k_code, v_code uint8 [B][Hkv][C][D]; k_sm uint16 [B][Hkv][C/G][D][2]
    (per key group and channel); v_sm uint16 [B][Hkv][C][D/G][2] (per token
    and channel group)."""
    B, H, C, D, G = g.batch, g.n_kv_heads, g.capacity, g.head_dim, g.group
    k_code = np.zeros((B, H, C, D), np.uint8)
    v_code = np.zeros((B, H, C, D), np.uint8)
    k_sm = np.zeros((B, H, C // G, D, 2), np.uint16)
    v_sm = np.zeros((B, H, C, D // G, 2), np.uint16)
    lib().orc_unpack(B, H, D, g.k_bits, g.v_bits, G, C, _p(cache.k_codes),
                     _p(cache.v_codes), _p(cache.k_meta), _p(cache.v_meta),
                     _p(k_code), _p(v_code), _p(k_sm), _p(v_sm))
    return k_code, v_code, k_sm, v_sm


# --------------------------------------------- rotated 2-bit format (BQ2_0) --
BQ2_D = 64       # head dim of the format ([KV1] Quantization Format)
BQ2_SINKS = 4    # positions kept in fp16


def bq2_hadamard() -> np.ndarray:
    """The oracle's normalized 64x64 Sylvester Hadamard matrix (fp64)."""
    return np.array([[lib().orc_bq2_hadamard(r, c) for c in range(BQ2_D)]
                     for r in range(BQ2_D)])


def bq2_rotate(x: np.ndarray) -> np.ndarray:
    """fp16 [..., 64] -> fp32 rotated vectors (exact product, one rounding)."""
    x = _u16(x)
    flat = x.reshape(-1, BQ2_D)
    out = np.empty(flat.shape, np.float32)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        lib().orc_bq2_rotate(_p(row), _p(out[r]))
    return out.reshape(x.shape)


def bq2_quantize(x: np.ndarray):
    """One block of 64 fp32 values -> (d bits, m bits, codes uint8[64])."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    assert x.size == BQ2_D
    codes = np.zeros(BQ2_D, np.uint8)
    d = ctypes.c_uint16()
    m = ctypes.c_uint16()
    lib().orc_bq2_quantize(_p(x), ctypes.byref(d), ctypes.byref(m), _p(codes))
    return int(d.value), int(m.value), codes


def bq2_block(d: int, m: int, codes: np.ndarray) -> bytes:
    """The page's 20-byte block for (d, m, codes)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros(20, np.uint8)
    lib().orc_bq2_block(d, m, _p(codes), _p(out))
    return out.tobytes()


@dataclass
class Bq2Geom:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    capacity: int


class Bq2Cache:
    """Host arrays of the rotated 2-bit format, laid out as bq2_oracle.c states."""

    def __init__(self, g: Bq2Geom):
        B, H, C = g.batch, g.n_kv_heads, g.capacity
        self.g = g
        self.k_codes = np.zeros((B, H, C // 32, 64, 2), np.uint32)
        self.v_codes = np.zeros((B, H, C // 32, 64, 2), np.uint32)
        self.k_meta = np.zeros((B, H, C, 2), np.uint16)
        self.v_meta = np.zeros((B, H, C, 2), np.uint16)
        self.k_sink = np.zeros((B, H, BQ2_SINKS, BQ2_D), np.uint16)
        self.v_sink = np.zeros((B, H, BQ2_D, BQ2_SINKS), np.uint16)

    def arrays(self):
        return (self.k_codes, self.v_codes, self.k_meta, self.v_meta,
                self.k_sink, self.v_sink)


def bq2_prefill(g: Bq2Geom, cache: Bq2Cache, k: np.ndarray, v: np.ndarray, n: int) -> None:
    """Positions [0, n) from fp16 rows k, v [B][Hkv][n][64] (unrotated)."""
    k = np.ascontiguousarray(_u16(k)[:, :, :n])
    v = np.ascontiguousarray(_u16(v)[:, :, :n])
    lib().orc_bq2_prefill(g.batch, g.n_kv_heads, g.capacity, _p(k), _p(v), n,
                          *[_p(a) for a in cache.arrays()])


def bq2_append(g: Bq2Geom, cache: Bq2Cache, k_new: np.ndarray, v_new: np.ndarray,
               seq_lens_before: np.ndarray) -> None:
    k_new = np.ascontiguousarray(_u16(k_new))
    v_new = np.ascontiguousarray(_u16(v_new))
    sl = np.ascontiguousarray(seq_lens_before, dtype=np.int32)
    lib().orc_bq2_append(g.batch, g.n_kv_heads, g.capacity, _p(k_new), _p(v_new), _p(sl),
                         *[_p(a) for a in cache.arrays()])


def bq2_unpack(g: Bq2Geom, cache: Bq2Cache):
    """Codes in natural order (tests): k_code, v_code uint8 [B][Hkv][C][64]."""
    shape = (g.batch, g.n_kv_heads, g.capacity, BQ2_D)
    kc = np.zeros(shape, np.uint8)
    vc = np.zeros(shape, np.uint8)
    lib().orc_bq2_unpack(g.batch, g.n_kv_heads, g.capacity, _p(cache.k_codes),
                         _p(cache.v_codes), _p(kc), _p(vc))
    return kc, vc


def bq2_cache_kv(g: Bq2Geom, cache: Bq2Cache, n: int):
    """Rotated (K, V) fp64 [B][Hkv][n][64] as the cache represents positions < n."""
    shape = (g.batch, g.n_kv_heads, n, BQ2_D)
    ok = np.zeros(shape, np.float64)
    ov = np.zeros(shape, np.float64)
    lib().orc_bq2_cache_kv(g.batch, g.n_kv_heads, g.capacity,
                           *[_p(a) for a in cache.arrays()], n, _p(ok), _p(ov))
    return ok, ov


def bq2_decode_attn(g: Bq2Geom, cache: Bq2Cache, q: np.ndarray, seq_lens: np.ndarray,
                    sm_scale: float) -> np.ndarray:
    """fp64 [B][Hq][64] outputs (rotated back); seq_lens include the current token."""
    q = np.ascontiguousarray(_u16(q))
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.zeros((g.batch, g.n_q_heads, BQ2_D), np.float64)
    lib().orc_bq2_decode_attn(g.batch, g.n_q_heads, g.n_kv_heads, g.capacity, _p(q),
                              *[_p(a) for a in cache.arrays()], _p(sl), float(sm_scale),
                              _p(out))
    return out


def max_threads() -> int:
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    lib().orc_set_threads(n)
