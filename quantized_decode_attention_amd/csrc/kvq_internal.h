// kvq_internal.h — device helpers and launch declarations shared by the libkvq
// translation units (not part of the public ABI).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/kvq.h"
#include "../../include/kvq_bq2.h"
#include "../../include/kvq_paged.h"
#include "../../include/kvq_probe.h"

namespace kvq {

constexpr int kThreads = 256;   // threads per workgroup of every kernel
constexpr int kVBlock = KVQ_VBLOCK;

// fp16 bits -> fp32 (exact widening).
__device__ __forceinline__ float h2f(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}
// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f2h(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

// Geometry as kernels see it (validated on the host).  Packed 32-position
// chunks are addressed through chunk slots (chunk_slot below): with table ==
// nullptr the cache is dense (kvq.h), otherwise paged (kvq_paged.h) with
// pages of 32 << cpp_log2 positions.
struct Geom {
  int B, Hq, Hkv, D, bK, bV, G, R, C;
  int Rv;                // value window length (R is the key window's)
  const int32_t* table;  // block table [B][maxp], or nullptr (dense)
  int cpp_log2;          // log2 of the 32-position chunks per page
  int maxp;              // table entries per sequence
  int npages;            // pages in the pools
};

inline Geom to_geom(const kvq_geom& g) {
  return Geom{g.batch, g.n_q_heads, g.n_kv_heads, g.head_dim, g.k_bits,
              g.v_bits, g.group, g.residual, g.capacity,
              g.residual_v > 0 ? g.residual_v : g.residual, nullptr, 0, 0, 0};
}

inline Geom to_geom(const kvq_geom& g, const kvq_paged_cache& c) {
  Geom r = to_geom(g);
  r.table = c.block_table;
  r.cpp_log2 = __builtin_ctz((unsigned)c.page_size / KVQ_VBLOCK);
  r.maxp = c.max_pages;
  r.npages = c.num_pages;
  return r;
}

// The dense buffers of kvq_cache standing for a paged cache's pools and
// residual windows (every launcher addresses packed data by chunk slot).
inline kvq_cache pool_view(const kvq_paged_cache& c) {
  return kvq_cache{c.k_codes, c.v_codes, c.k_meta, c.v_meta, c.k_res, c.v_res};
}

// Slot of 32-position chunk k of unit (b, hkv) = b * Hkv + hkv in the packed
// buffers: rows of 32 positions, one after the other.  The dense layout is the
// paged one with a single page of C positions per unit; a paged cache puts the
// chunk in page table[b][k / chunks per page], whose Hkv units are stored one
// after the other.  -1 if the table entry is not a page of the pool.  The key
// group starting at position p (a multiple of G) has meta slot
// chunk_slot(p / 32) * 32 / G, as every page holds whole key groups.
__device__ __forceinline__ int64_t chunk_slot(const Geom& g, int64_t unit, int k) {
  if (g.table == nullptr) return unit * (g.C / KVQ_VBLOCK) + k;
  const int64_t b = unit / g.Hkv, hkv = unit % g.Hkv;
  const int pg = g.table[b * g.maxp + (k >> g.cpp_log2)];
  if (pg < 0 || pg >= g.npages) return -1;
  return (((int64_t)pg * g.Hkv + hkv) << g.cpp_log2) + (k & ((1 << g.cpp_log2) - 1));
}

// 64-bit element offsets into the cache buffers.
__host__ __device__ inline int64_t kcodes_words(const Geom& g) {
  return (int64_t)g.D * g.bK / 32;
}

// ---- launchers (defined in the .hip files; all enqueue only) -------------
hipError_t launch_quantize_keys(const Geom& g, const uint16_t* src,
                                int64_t src_unit_stride, int32_t pos0,
                                int32_t n_tok, uint32_t* k_codes,
                                uint16_t* k_meta, hipStream_t st);
hipError_t launch_quantize_values(const Geom& g, const uint16_t* src,
                                  int64_t src_unit_stride, int32_t pos0,
                                  int32_t n_tok, uint32_t* v_codes,
                                  uint16_t* v_meta, hipStream_t st);
// Positions [pos0, pos0 + n_tok) of key (values = false) or value rows into
// their window slots.
hipError_t launch_residual_copy(const Geom& g, const uint16_t* src, int64_t src_unit_stride,
                                int32_t pos0, int32_t n_tok, uint16_t* window, bool values,
                                hipStream_t st);
hipError_t launch_append(const Geom& g, const uint16_t* k_new,
                         const uint16_t* v_new, const int32_t* seq_lens,
                         const kvq_cache& cache, hipStream_t st);
// T new tokens per sequence ([B][T][Hkv][D]) in one launch: the same result
// as T launch_append calls with seq_lens + t.
hipError_t launch_append_tokens(const Geom& g, int T, const uint16_t* k_new,
                                const uint16_t* v_new, const int32_t* seq_lens,
                                const kvq_cache& c, hipStream_t st);

struct DecodeLaunch {
  Geom g;
  const uint16_t* q;  // [B][T][Hq][D]
  kvq_cache cache;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t T;          // query tokens per sequence (the last T positions)
  int32_t gq;         // rows per KV head: T * Hq / Hkv (query token major)
  int32_t n_workers;  // worker waves of the partial kernel
  int32_t rw;         // work units of a residual chunk (its bytes / a packed chunk's)
  float scale_log2;   // sm_scale * log2(e)
  float* ws;          // partials [n_workers + B*Hkv][gq][D + 4]
  uint16_t* out;      // [B][T][Hq][D]
};
// Worker waves of the partial kernel for gq rows per KV head on the current
// device (dense or paged as g.table says).
hipError_t decode_workers(const Geom& g, int gq, int cus, int* workers);
// The partial kernels by head dim, key bits and cache form (one instantiation
// set each): op 0 launches, op 1 puts the worker count in *workers.
#define KVQ_DECODE_SETS(X)                                                          \
  X(decode_partial_d64_k2) X(decode_partial_d64_k4) X(decode_partial_d64_k8)         \
  X(decode_partial_d128_k2) X(decode_partial_d128_k4) X(decode_partial_d128_k8)      \
  X(decode_partial_paged_d64_k2) X(decode_partial_paged_d64_k4)                      \
  X(decode_partial_paged_d64_k8) X(decode_partial_paged_d128_k2)                     \
  X(decode_partial_paged_d128_k4) X(decode_partial_paged_d128_k8)
#define KVQ_DECLARE_SET(name) \
  hipError_t name(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st);
KVQ_DECODE_SETS(KVQ_DECLARE_SET)
#undef KVQ_DECLARE_SET
hipError_t launch_decode_partial(const DecodeLaunch& L, hipStream_t st);
hipError_t launch_decode_combine(const DecodeLaunch& L, hipStream_t st);

// ---- rotated per-token 2-bit format (kvq_bq2.h) ---------------------------
struct Bq2Geom {
  int B, Hq, Hkv, C;
};

inline Bq2Geom to_geom(const kvq_bq2_geom& g) {
  return Bq2Geom{g.batch, g.n_q_heads, g.n_kv_heads, g.capacity};
}

// Positions [0, n) of every unit from rows k, v [B][Hkv][n][64].
hipError_t launch_bq2_prefill(const Bq2Geom& g, const uint16_t* k, const uint16_t* v,
                              int32_t n, const kvq_bq2_cache& cache, hipStream_t st);
// One position per sequence (seq_lens[b] = positions held before it).
hipError_t launch_bq2_append(const Bq2Geom& g, const uint16_t* k_new, const uint16_t* v_new,
                             const int32_t* seq_lens, const kvq_bq2_cache& cache,
                             hipStream_t st);

struct Bq2Launch {
  Bq2Geom g;
  const uint16_t* q;
  kvq_bq2_cache cache;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t n_workers;  // worker waves of the partial kernel
  int32_t rw;         // work units of the sink chunk
  float scale_log2;   // sm_scale * log2(e)
  float* ws;          // partials [n_workers + B*Hkv][Hq/Hkv][64 + 4]
  uint16_t* out;      // [B][Hq][64]
};
hipError_t bq2_decode_workers(const Bq2Geom& g, int cus, int* workers);
hipError_t launch_bq2_decode_partial(const Bq2Launch& L, hipStream_t st);
hipError_t launch_bq2_decode_combine(const Bq2Launch& L, hipStream_t st);

// ---- kvq_decode_attn_noalloc's partials (kvq_noalloc.hip) -----------------
// This device's copy of the library's static partials array and its size.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// ---- measurement aid (kvq_probe.h) ----------------------------------------
int probe_sink_words();
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_stream_read_sweep(const void* buf, size_t bytes, uint32_t* sink, int waves,
                                    int loads, int mode, hipStream_t st);

}  // namespace kvq
