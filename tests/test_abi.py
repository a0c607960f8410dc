"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/kvq.h declares, and
reject invalid arguments with the documented status before any launch.  The
byte sizes it reports are tied to the layout and to the KV1 model card's
"Memory" table.  Calls with made-up pointers below are all invalid in some
other argument, so none of them reaches a launch.
"""
import ctypes
import os
import re

import pytest

import quantized_decode_attention_amd as kvq
from quantized_decode_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")
HEADER_BQ2 = os.path.join(ROOT, "include", "kvq_bq2.h")
HEADER_PAGED = os.path.join(ROOT, "include", "kvq_paged.h")
HEADER_PROBE = os.path.join(ROOT, "include", "kvq_probe.h")
GOOD = dict(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128, k_bits=2, v_bits=4,
            group=32, residual=128, capacity=1024)


def _declared(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = kvq.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.EXPORTS) == names


def test_exports_every_declared_bq2_symbol():
    L = kvq.lib()
    names = _declared(HEADER_BQ2)
    assert len(names) == 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.EXPORTS_BQ2) == names


def test_exports_every_declared_paged_symbol():
    L = kvq.lib()
    names = _declared(HEADER_PAGED)
    assert len(names) == 10
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.EXPORTS_PAGED) == names


def test_exports_every_declared_probe_symbol():
    L = kvq.lib()
    names = _declared(HEADER_PROBE)
    assert sorted(_lib.EXPORTS_PROBE) == names
    for n in names:
        assert hasattr(L, n), n


def test_headers_compile_as_plain_c(tmp_path):
    """The public headers are C (no C++ in the boundary): a C99 translation
    unit that includes all of them and takes every entry point's address
    compiles with gcc -Wall -Werror."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    names = sorted(set(_declared(HEADER) + _declared(HEADER_BQ2) + _declared(HEADER_PAGED) +
                       _declared(HEADER_PROBE)))
    src = tmp_path / "abi.c"
    src.write_text(
        '#include "kvq.h"\n#include "kvq_paged.h"\n#include "kvq_bq2.h"\n'
        '#include "kvq_probe.h"\n'
        "void *entry_points[] = {\n" + ",\n".join(f"  (void *)&{n}" for n in names) + "\n};\n")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-Wno-pedantic", "-I", os.path.join(ROOT, "include"), "-c", str(src),
                        "-o", str(tmp_path / "abi.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_include_headers_are_all_checked():
    """Every public header's declarations are covered by an export test."""
    hdrs = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert hdrs == ["kvq.h", "kvq_bq2.h", "kvq_paged.h", "kvq_probe.h"]


@pytest.mark.parametrize("page_size,max_pages,num_pages,ok", [
    (128, 8, 100, True), (32, 32, 1, True), (1024, 1, 4, True), (64, 16, 10, True),
    (16, 64, 10, False),   # below one 32-position chunk
    (96, 11, 10, False),   # not a power of two
    (128, 7, 10, False),   # 7 pages of 128 do not cover capacity 1024
    (128, 8, 0, False),    # empty pool
    (0, 8, 10, False),
])
def test_paged_validation(page_size, max_pages, num_pages, ok):
    g = kvq.Geom(**GOOD)
    if ok:
        kvq.kvq_paged_validate(g, page_size, max_pages, num_pages)
        return
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_paged_validate(g, page_size, max_pages, num_pages)
    assert e.value.status == -2


def test_paged_page_smaller_than_key_group():
    g = kvq.Geom(**{**GOOD, "group": 64, "residual": 128})
    kvq.kvq_paged_validate(g, 64, 16, 4)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_paged_validate(g, 32, 32, 4)
    assert e.value.status == -2


@pytest.mark.parametrize("geom", [GOOD, {**GOOD, "head_dim": 64, "k_bits": 4, "v_bits": 2,
                                         "group": 64, "residual": 64}])
def test_paged_cache_bytes_are_dense_bytes_per_page(geom):
    """A pool of N pages of P positions takes the bytes of a dense cache of N
    sequences of capacity P (each page is a dense unit per KV head); the
    residual windows are per sequence, as in the dense cache."""
    g = kvq.Geom(**geom)
    for P, N in [(128, 3), (256, 10), (1024, 2)]:
        pools = kvq.kvq_paged_cache_bytes(g, P, N)
        dense_pages = kvq.kvq_cache_bytes(kvq.Geom(**{**geom, "batch": N, "capacity": P}))
        dense = kvq.kvq_cache_bytes(g)
        assert pools[:4] == dense_pages[:4]
        assert pools[4:] == dense[4:]


def test_paged_calls_reject_before_launch():
    """Invalid page parameters or null buffers fail on the host."""
    g = kvq.Geom(**GOOD)
    gc = g.c()
    L = kvq.lib()
    cc = _lib.kvq_paged_cache(16, 16, 16, 16, 16, 16, None, 128, 8, 4)
    st = L.kvq_paged_append(ctypes.byref(gc), 16, 16, 16, ctypes.byref(cc), None)
    assert st == -1 and "block_table" in kvq.last_error()
    cc = _lib.kvq_paged_cache(16, 16, 16, 16, 16, 16, 16, 100, 8, 4)
    st = L.kvq_paged_decode_attn(ctypes.byref(gc), 16, ctypes.byref(cc), 16, 1, 1.0, 16, 1 << 30,
                                 16, None)
    assert st == -2
    cc = _lib.kvq_paged_cache(16, 16, 16, 16, 16, 16, 16, 128, 8, 4)
    st = L.kvq_paged_prefill(ctypes.byref(gc), 16, 16, 2000, ctypes.byref(cc), None)
    assert st == -6


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("n_kv_heads", 0), ("n_q_heads", 12), ("n_q_heads", 64), ("n_q_heads", 128),
    ("capacity", 0), ("capacity", 100), ("capacity", 1 << 25),
])
def test_bq2_geometry_validation(field, value):
    good = dict(batch=2, n_q_heads=32, n_kv_heads=8, capacity=1024)
    kvq.kvq_bq2_validate_geom(kvq.Bq2Geom(**good))
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_bq2_validate_geom(kvq.Bq2Geom(**{**good, field: value}))
    assert e.value.status == -2


def test_bq2_cache_bytes_and_memory_table():
    """Per position and KV head: two 20-byte BQ2_0 blocks ([KV1] Quantization
    Format); 6 layers x 8 KV heads at 32K context give the card's 60 MiB (plus
    the sinks, 4 fp16 positions per head)."""
    g = kvq.Bq2Geom(1, 32, 8, 32768)
    kc, vc, km, vm, ks, vs = kvq.kvq_bq2_cache_bytes(g)
    assert kc == vc == 8 * 32768 * 16
    assert km == vm == 8 * 32768 * 4
    assert ks == vs == 8 * 4 * 64 * 2
    assert 6 * (kc + vc + km + vm) == 60 * 2**20


def test_versions_and_status_strings():
    assert kvq.kvq_abi_version() == kvq.ABI_VERSION == 2
    assert kvq.kvq_layout_version() == kvq.LAYOUT_VERSION == 3
    for s in range(-8, 1):
        assert kvq.status_str(s) and kvq.status_str(s) != "unknown status"
    assert kvq.status_str(5) == "unknown status"



@pytest.mark.parametrize("field,value,status", [
    ("k_bits", 3, -3), ("v_bits", 16, -3), ("k_bits", 1, -3), ("batch", 0, -2),
    ("n_q_heads", 12, -2),
    ("n_q_heads", 24, -2), ("head_dim", 96, -2), ("group", 16, -2), ("group", 48, -2),
    ("residual", 48, -2), ("residual", 0, -2), ("capacity", 1000, -2),
    ("capacity", 1 << 25, -2), ("n_kv_heads", 0, -2),
])
def test_geometry_validation(field, value, status):
    kvq.kvq_validate_geom(kvq.Geom(**GOOD))
    bad = dict(GOOD)
    bad[field] = value
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_validate_geom(kvq.Geom(**bad))
    assert e.value.status == status
    assert kvq.last_error()


@pytest.mark.parametrize("rv,ok", [(0, True), (32, True), (256, True), (64, True),
                                   (48, False), (-32, False), (384, False)])
def test_value_window_validation(rv, ok):
    """residual_v: 0 (the key window's length) or a multiple of group that
    divides capacity (1024 here)."""
    g = kvq.Geom(**{**GOOD, "residual_v": rv})
    if ok:
        kvq.kvq_validate_geom(g)
        return
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_validate_geom(g)
    assert e.value.status == -2


def test_value_window_bytes():
    g = kvq.Geom(**{**GOOD, "residual_v": 256})
    kc, vc, km, vm, kr, vr = kvq.kvq_cache_bytes(g)
    assert kr == 2 * 8 * 128 * 128 * 2
    assert vr == 2 * 8 * 256 * 128 * 2
    assert kvq.kvq_paged_cache_bytes(g, 128, 4)[4:] == [kr, vr]


def test_group_larger_than_head_dim():
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_validate_geom(kvq.Geom(**{**GOOD, "head_dim": 64, "group": 128,
                                          "residual": 128}))
    assert e.value.status == -2


def test_cache_bytes_layout():
    g = kvq.Geom(**GOOD)
    kc, vc, km, vm, kr, vr = kvq.kvq_cache_bytes(g)
    B, H, C, D = 2, 8, 1024, 128
    assert kc == B * H * C * D * 2 // 8
    assert vc == B * H * C * D * 4 // 8
    assert km == B * H * (C // 32) * D * 4
    assert vm == B * H * C * (D // 32) * 4
    assert kr == vr == B * H * 128 * D * 2


def test_cache_bytes_kv1_memory_table():
    """At head dim 64, group 64, 2-bit keys and values, the packed part of the
    cache for the KV1 model's 6 attention layers x 8 KV heads at 32K context is
    the card's 60 MiB (KV1-1.2B card, "Memory"); 8K gives 15 MiB."""
    for ctx, mib in ((32768, 60), (8192, 15)):
        g = kvq.Geom(1, 32, 8, 64, 2, 2, 64, 64, ctx)
        kc, vc, km, vm, kr, vr = kvq.kvq_cache_bytes(g)
        assert 6 * (kc + vc + km + vm) == mib * 1024 * 1024


def test_invalid_arguments_are_rejected_before_launch():
    L = kvq.lib()
    g = kvq.Geom(**GOOD).c()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10004)
    # pos0 / n_tok not multiples of the group, or past capacity
    assert L.kvq_quantize_keys_perchannel(ctypes.byref(g), fake, 16, 32, fake, fake, None) == -6
    assert L.kvq_quantize_keys_perchannel(ctypes.byref(g), fake, 0, 33, fake, fake, None) == -6
    assert L.kvq_quantize_keys_perchannel(ctypes.byref(g), fake, 1024, 32, fake, fake, None) == -6
    assert L.kvq_quantize_values_pertoken(ctypes.byref(g), fake, -32, 32, fake, fake, None) == -6
    # null / misaligned pointers
    assert L.kvq_quantize_keys_perchannel(ctypes.byref(g), None, 0, 32, fake, fake, None) == -1
    assert L.kvq_quantize_keys_perchannel(ctypes.byref(g), odd, 0, 32, fake, fake, None) == -4
    c = _lib.kvq_cache(0x10000, 0x10000, 0x10000, None, 0x10000, 0x10000)
    assert L.kvq_append(ctypes.byref(g), fake, fake, fake, ctypes.byref(c), None) == -1
    c = _lib.kvq_cache(0x10000, 0x10000, 0x10008, 0x10000, 0x10000, 0x10000)
    assert L.kvq_append(ctypes.byref(g), fake, fake, fake, ctypes.byref(c), None) == -4
    assert "k_meta" in kvq.last_error()
    # prefill length out of range
    c = _lib.kvq_cache(*([0x10000] * 6))
    assert L.kvq_prefill(ctypes.byref(g), fake, fake, 1025, ctypes.byref(c), None) == -6
    # a T-token append needs T >= 1, and the usual pointers
    assert L.kvq_append_tokens(ctypes.byref(g), 0, fake, fake, fake, ctypes.byref(c), None) == -6
    assert "T must be" in kvq.last_error()
    assert L.kvq_append_tokens(ctypes.byref(g), 4, None, fake, fake, ctypes.byref(c), None) == -1
    assert L.kvq_append_tokens(ctypes.byref(g), 4, fake, odd, fake, ctypes.byref(c), None) == -4
    # bad geometry is reported first
    bad = kvq.Geom(**{**GOOD, "k_bits": 3}).c()
    assert L.kvq_decode_attn(ctypes.byref(bad), fake, ctypes.byref(c), fake, 8, 0.1,
                             None, 0, fake, None) == -3
    # non-finite scale
    assert L.kvq_decode_attn(ctypes.byref(g), fake, ctypes.byref(c), fake, 8,
                             float("nan"), None, 0, fake, None) == -6
    assert L.kvq_cache_bytes(None, None) == -1


def test_build_scratch_guard_reads_the_resource_remarks():
    """The build rejects a decode partial kernel (either format) that the
    compiler reports with scratch; other kernels and zero scratch pass."""
    from quantized_decode_attention_amd import build
    remarks = "\n".join([
        "x.hip:1:1: remark: Function Name: _ZN3kvq12_GLOBAL__N_121decode_partial_kernelILi128E",
        "x.hip:1:1: remark:     VGPRs: 201",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0",
        "x.hip:2:1: remark: Function Name: _ZN3kvq12_GLOBAL__N_118bq2_partial_kernelILi4E",
        "x.hip:2:1: remark:     ScratchSize [bytes/lane]: 28",
        "x.hip:3:1: remark: Function Name: _ZN3kvq12_GLOBAL__N_121decode_combine_kernel",
        "x.hip:3:1: remark:     ScratchSize [bytes/lane]: 16",
    ])
    assert build.scratch_kernels(remarks) == [
        ("_ZN3kvq12_GLOBAL__N_118bq2_partial_kernelILi4E", 28)]
    assert build.scratch_kernels(remarks.replace(": 28", ": 0")) == []


def test_noalloc_buffer_size_matches_the_header():
    """The binding's copy of KVQ_NOALLOC_SCRATCH_BYTES is the header's."""
    text = open(HEADER).read()
    m = re.search(r"#define KVQ_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m, "KVQ_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
