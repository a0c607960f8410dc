// kvq_api.cpp — host side of the libkvq C ABI: argument validation, size and
// workspace queries, split sizing, kernel launches.  Every entry point only
// enqueues work on the caller's stream; nothing here synchronizes or allocates.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kvq_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_geom(const kvq_geom* g) {
  if (!g) return fail(KVQ_ERR_NULL, "geometry is NULL");
  if (g->k_bits != 2 && g->k_bits != 4 && g->k_bits != 8)
    return fail(KVQ_ERR_BITS, "k_bits must be 2, 4 or 8 (got %d)", g->k_bits);
  if (g->v_bits != 2 && g->v_bits != 4 && g->v_bits != 8)
    return fail(KVQ_ERR_BITS, "v_bits must be 2, 4 or 8 (got %d)", g->v_bits);
  if (g->batch < 1 || g->n_kv_heads < 1 || g->n_q_heads < 1)
    return fail(KVQ_ERR_GEOM, "batch and head counts must be >= 1");
  if (g->n_q_heads % g->n_kv_heads != 0)
    return fail(KVQ_ERR_GEOM, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                g->n_q_heads, g->n_kv_heads);
  const int gq = g->n_q_heads / g->n_kv_heads;
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8 && gq != 16)
    return fail(KVQ_ERR_GEOM, "query heads per KV head must be 1, 2, 4, 8 or 16 (got %d)", gq);
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(KVQ_ERR_GEOM, "head_dim must be 64 or 128 (got %d)", g->head_dim);
  if (g->group != 32 && g->group != 64 && g->group != 128)
    return fail(KVQ_ERR_GEOM, "group must be 32, 64 or 128 (got %d)", g->group);
  if (g->group > g->head_dim || g->head_dim % g->group != 0)
    return fail(KVQ_ERR_GEOM, "group (%d) must divide head_dim (%d)", g->group, g->head_dim);
  if (g->residual < g->group || g->residual % g->group != 0)
    return fail(KVQ_ERR_GEOM, "residual (%d) must be a positive multiple of group (%d)",
                g->residual, g->group);
  if (g->capacity < g->residual || g->capacity % g->residual != 0 || g->capacity > (1 << 24))
    return fail(KVQ_ERR_GEOM, "capacity (%d) must be a multiple of residual (%d), <= 2^24",
                g->capacity, g->residual);
  if (g->residual_v < 0 || (g->residual_v > 0 && g->residual_v % g->group != 0))
    return fail(KVQ_ERR_GEOM, "residual_v (%d) must be 0 or a positive multiple of group (%d)",
                g->residual_v, g->group);
  if (g->residual_v > 0 && g->capacity % g->residual_v != 0)
    return fail(KVQ_ERR_GEOM, "capacity (%d) must be a multiple of residual_v (%d)",
                g->capacity, g->residual_v);
  return KVQ_OK;
}

int check_cache(const kvq_cache* c) {
  if (!c) return fail(KVQ_ERR_NULL, "cache is NULL");
  const void* p[6] = {c->k_codes, c->v_codes, c->k_meta, c->v_meta, c->k_res, c->v_res};
  static const char* names[6] = {"k_codes", "v_codes", "k_meta", "v_meta", "k_res", "v_res"};
  for (int i = 0; i < 6; ++i) {
    if (!p[i]) return fail(KVQ_ERR_NULL, "cache.%s is NULL", names[i]);
    if (!aligned16(p[i])) return fail(KVQ_ERR_ALIGN, "cache.%s is not 16-byte aligned", names[i]);
  }
  return KVQ_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(KVQ_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(KVQ_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return KVQ_OK;
}

// seq_lens is an int32 array; 4-byte alignment is enough.
int check_lens(const int32_t* p) {
  if (!p) return fail(KVQ_ERR_NULL, "seq_lens is NULL");
  if (reinterpret_cast<uintptr_t>(p) & 3u)
    return fail(KVQ_ERR_ALIGN, "seq_lens is not 4-byte aligned");
  return KVQ_OK;
}

int packed_len(int n, int R) { return n <= 0 ? 0 : n - (((n - 1) % R) + 1); }

// Compute units of the current device, cached per device.
int cu_count(int* out) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return KVQ_OK;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
  if (dev >= 0 && dev < 64) cache[dev] = cus;
  *out = cus;
  return KVQ_OK;
}

// Worker waves of the persistent partial kernel (resident waves x CUs) for
// T query tokens per sequence, over a dense cache or a paged one (pc).
int workers_for(const kvq_geom* g, int32_t* n_workers, int T = 1, bool paged = false) {
  int cus = 0;
  int st = cu_count(&cus);
  if (st != KVQ_OK) return st;
  int w = 0;
  kvq::Geom kg = kvq::to_geom(*g);
  static const int32_t kAnyTable = 0;  // a non-null table selects the paged kernels
  if (paged) kg.table = &kAnyTable;
  hipError_t e = kvq::decode_workers(kg, T * (g->n_q_heads / g->n_kv_heads), cus, &w);
  if (e != hipSuccess) return hip_fail(e, "occupancy query");
  *n_workers = w;
  return KVQ_OK;
}

int check_max_len(const kvq_geom* g, int32_t max_seq_len) {
  if (max_seq_len < 1 || max_seq_len > g->capacity)
    return fail(KVQ_ERR_RANGE, "max_seq_len (%d) must be in [1, capacity=%d]",
                max_seq_len, g->capacity);
  return KVQ_OK;
}

// Partials: one per (worker wave, unit) pair that occurs, at most
// n_workers + B*Hkv, each [T * Hq/Hkv][head_dim + 4] floats.
size_t workspace_need(const kvq_geom* g, int32_t n_workers, int T = 1) {
  const size_t gq = (size_t)T * (g->n_q_heads / g->n_kv_heads);
  return ((size_t)n_workers + (size_t)g->batch * g->n_kv_heads) * gq *
         (g->head_dim + 4) * sizeof(float);
}

int check_workspace(const kvq_geom* g, int32_t n_workers, const void* ws, size_t bytes,
                    int T = 1) {
  const size_t need = workspace_need(g, n_workers, T);
  if (!ws) return fail(KVQ_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(KVQ_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", bytes, need);
  return KVQ_OK;
}

// Query tokens per sequence: T >= 1 with T * Hq/Hkv in {1, 2, 4, 8, 16}.
int check_tokens(const kvq_geom* g, int32_t T) {
  const int rows = T * (g->n_q_heads / g->n_kv_heads);
  if (T < 1 || (rows != 1 && rows != 2 && rows != 4 && rows != 8 && rows != 16))
    return fail(KVQ_ERR_RANGE,
                "T=%d query tokens: T * n_q_heads / n_kv_heads must be 1, 2, 4, 8 or 16", T);
  return KVQ_OK;
}

// Page parameters of a paged cache (kvq_paged.h); buffers too if `buffers`.
int check_paged(const kvq_geom* g, const kvq_paged_cache* c, bool buffers) {
  if (!c) return fail(KVQ_ERR_NULL, "cache is NULL");
  const int P = c->page_size;
  if (P < 32 || (P & (P - 1)) != 0 || P < g->group)
    return fail(KVQ_ERR_GEOM, "page_size (%d) must be a power of two >= 32 and >= group (%d)", P,
                g->group);
  if (c->max_pages < 1 || (int64_t)c->max_pages * P < g->capacity)
    return fail(KVQ_ERR_GEOM, "max_pages (%d) * page_size (%d) must cover capacity (%d)",
                c->max_pages, P, g->capacity);
  if (c->num_pages < 1) return fail(KVQ_ERR_GEOM, "num_pages (%d) must be >= 1", c->num_pages);
  if (!buffers) return KVQ_OK;
  const void* p[6] = {c->k_codes, c->v_codes, c->k_meta, c->v_meta, c->k_res, c->v_res};
  static const char* names[6] = {"k_codes", "v_codes", "k_meta", "v_meta", "k_res", "v_res"};
  for (int i = 0; i < 6; ++i) {
    if (!p[i]) return fail(KVQ_ERR_NULL, "cache.%s is NULL", names[i]);
    if (!aligned16(p[i])) return fail(KVQ_ERR_ALIGN, "cache.%s is not 16-byte aligned", names[i]);
  }
  if (!c->block_table) return fail(KVQ_ERR_NULL, "cache.block_table is NULL");
  if (reinterpret_cast<uintptr_t>(c->block_table) & 3u)
    return fail(KVQ_ERR_ALIGN, "cache.block_table is not 4-byte aligned");
  return KVQ_OK;
}

// Launch parameters of decode over a dense cache, or over a paged one when
// pc is given (then `cache` is its pool view).
int decode_setup(const kvq_geom* geom, const uint16_t* q, const kvq_cache* cache,
                 const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                 void* workspace, size_t workspace_bytes, uint16_t* out,
                 kvq::DecodeLaunch* L, int32_t T = 1, const kvq_paged_cache* pc = nullptr) {
  int st = check_geom(geom);
  if (st != KVQ_OK) return st;
  if (pc && (st = check_paged(geom, pc, true)) != KVQ_OK) return st;
  if ((st = check_tokens(geom, T)) != KVQ_OK) return st;
  if (T > max_seq_len)
    return fail(KVQ_ERR_RANGE, "T=%d exceeds max_seq_len=%d", T, max_seq_len);
  if ((st = check_cache(cache)) != KVQ_OK) return st;
  if ((st = check_ptr(q, "q")) != KVQ_OK) return st;
  if ((st = check_lens(seq_lens)) != KVQ_OK) return st;
  if ((st = check_ptr(out, "out")) != KVQ_OK) return st;
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_huge_valf() ||
      sm_scale == -__builtin_huge_valf())
    return fail(KVQ_ERR_RANGE, "sm_scale must be finite");
  if ((st = check_max_len(geom, max_seq_len)) != KVQ_OK) return st;
  int32_t n_workers = 0;
  if ((st = workers_for(geom, &n_workers, T, pc != nullptr)) != KVQ_OK) return st;
  if ((st = check_workspace(geom, n_workers, workspace, workspace_bytes, T)) != KVQ_OK)
    return st;
  L->g = pc ? kvq::to_geom(*geom, *pc) : kvq::to_geom(*geom);
  L->q = q;
  L->cache = *cache;
  L->seq_lens = seq_lens;
  L->max_seq_len = max_seq_len;
  L->T = T;
  L->gq = T * (geom->n_q_heads / geom->n_kv_heads);
  L->n_workers = n_workers;
  {
    // a residual (fp16) chunk moves rw times the bytes of a packed chunk
    const int64_t D = geom->head_dim;
    const int64_t packed = D * (geom->k_bits + geom->v_bits) / 8 + 8 * D / geom->group;
    L->rw = (int32_t)((4 * D + packed - 1) / packed);
  }
  L->scale_log2 = sm_scale * 1.4426950408889634f;
  L->ws = static_cast<float*>(workspace);
  L->out = out;
  return KVQ_OK;
}


// ---- rotated per-token 2-bit format (kvq_bq2.h) ---------------------------

int check_bq2_geom(const kvq_bq2_geom* g) {
  if (!g) return fail(KVQ_ERR_NULL, "geometry is NULL");
  if (g->batch < 1 || g->n_kv_heads < 1 || g->n_q_heads < 1)
    return fail(KVQ_ERR_GEOM, "batch and head counts must be >= 1");
  if (g->n_q_heads % g->n_kv_heads != 0)
    return fail(KVQ_ERR_GEOM, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                g->n_q_heads, g->n_kv_heads);
  const int gq = g->n_q_heads / g->n_kv_heads;
  if (gq != 1 && gq != 2 && gq != 4)
    return fail(KVQ_ERR_GEOM, "query heads per KV head must be 1, 2 or 4 (got %d)", gq);
  if (g->capacity < 32 || g->capacity % 32 != 0 || g->capacity > (1 << 24))
    return fail(KVQ_ERR_GEOM, "capacity (%d) must be a positive multiple of 32, <= 2^24",
                g->capacity);
  return KVQ_OK;
}

int check_bq2_cache(const kvq_bq2_cache* c) {
  if (!c) return fail(KVQ_ERR_NULL, "cache is NULL");
  const void* p[6] = {c->k_codes, c->v_codes, c->k_meta, c->v_meta, c->k_sink, c->v_sink};
  static const char* names[6] = {"k_codes", "v_codes", "k_meta", "v_meta", "k_sink", "v_sink"};
  for (int i = 0; i < 6; ++i) {
    if (!p[i]) return fail(KVQ_ERR_NULL, "cache.%s is NULL", names[i]);
    if (!aligned16(p[i])) return fail(KVQ_ERR_ALIGN, "cache.%s is not 16-byte aligned", names[i]);
  }
  return KVQ_OK;
}

int bq2_workers_for(const kvq_bq2_geom* g, int32_t* n_workers) {
  int cus = 0;
  int st = cu_count(&cus);
  if (st != KVQ_OK) return st;
  int w = 0;
  hipError_t e = kvq::bq2_decode_workers(kvq::to_geom(*g), cus, &w);
  if (e != hipSuccess) return hip_fail(e, "occupancy query");
  *n_workers = w;
  return KVQ_OK;
}

int check_bq2_max_len(const kvq_bq2_geom* g, int32_t max_seq_len) {
  if (max_seq_len < 1 || max_seq_len > g->capacity)
    return fail(KVQ_ERR_RANGE, "max_seq_len (%d) must be in [1, capacity=%d]", max_seq_len,
                g->capacity);
  return KVQ_OK;
}

// Partials: at most n_workers + B*Hkv, each [Hq/Hkv][64 + 4] floats.
size_t bq2_workspace_need(const kvq_bq2_geom* g, int32_t n_workers) {
  const size_t gq = g->n_q_heads / g->n_kv_heads;
  return ((size_t)n_workers + (size_t)g->batch * g->n_kv_heads) * gq *
         (KVQ_BQ2_HEAD_DIM + 4) * sizeof(float);
}

int bq2_decode_setup(const kvq_bq2_geom* geom, const uint16_t* q, const kvq_bq2_cache* cache,
                     const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                     void* workspace, size_t workspace_bytes, uint16_t* out,
                     kvq::Bq2Launch* L) {
  int st = check_bq2_geom(geom);
  if (st != KVQ_OK) return st;
  if ((st = check_bq2_cache(cache)) != KVQ_OK) return st;
  if ((st = check_ptr(q, "q")) != KVQ_OK) return st;
  if ((st = check_lens(seq_lens)) != KVQ_OK) return st;
  if ((st = check_ptr(out, "out")) != KVQ_OK) return st;
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_huge_valf() ||
      sm_scale == -__builtin_huge_valf())
    return fail(KVQ_ERR_RANGE, "sm_scale must be finite");
  if ((st = check_bq2_max_len(geom, max_seq_len)) != KVQ_OK) return st;
  int32_t n_workers = 0;
  if ((st = bq2_workers_for(geom, &n_workers)) != KVQ_OK) return st;
  const size_t need = bq2_workspace_need(geom, n_workers);
  if (!workspace) return fail(KVQ_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(workspace)) return fail(KVQ_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  L->g = kvq::to_geom(*geom);
  L->q = q;
  L->cache = *cache;
  L->seq_lens = seq_lens;
  L->max_seq_len = max_seq_len;
  L->n_workers = n_workers;
  // the sink chunk: 4 fp16 positions (K and V: 1 KB) against a packed chunk's
  // 32 x 40 bytes, i.e. one work unit
  L->rw = 1;
  L->scale_log2 = sm_scale * 1.4426950408889634f;
  L->ws = static_cast<float*>(workspace);
  L->out = out;
  return KVQ_OK;
}

}  // namespace

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }
int kvq_layout_version(void) { return KVQ_LAYOUT_VERSION; }

const char* kvq_status_str(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "null pointer";
    case KVQ_ERR_GEOM: return "invalid geometry";
    case KVQ_ERR_BITS: return "unsupported bit width";
    case KVQ_ERR_ALIGN: return "misaligned pointer";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_RANGE: return "argument out of range";
    case KVQ_ERR_HIP: return "HIP runtime error";
    case KVQ_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

int kvq_validate_geom(const kvq_geom* geom) {
  try {
    return check_geom(geom);
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_cache_bytes(const kvq_geom* geom, size_t out[6]) {
  int st = check_geom(geom);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_ERR_NULL, "out is NULL");
  const size_t B = geom->batch, H = geom->n_kv_heads, C = geom->capacity,
               D = geom->head_dim, G = geom->group, R = geom->residual;
  out[0] = B * H * C * (D * geom->k_bits / 32) * 4;               // k_codes
  out[1] = B * H * (C / KVQ_VBLOCK) * D * geom->v_bits * 4;      // v_codes
  out[2] = B * H * (C / G) * D * 2 * 2;                          // k_meta
  out[3] = B * H * C * (D / G) * 2 * 2;                          // v_meta
  const size_t Rv = geom->residual_v > 0 ? geom->residual_v : R;
  out[4] = B * H * R * D * 2;                                    // k_res
  out[5] = B * H * Rv * D * 2;                                   // v_res
  return KVQ_OK;
}

int kvq_decode_workers(const kvq_geom* geom, int32_t* n_workers) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if (!n_workers) return fail(KVQ_ERR_NULL, "n_workers is NULL");
    return workers_for(geom, n_workers);
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_decode_workspace_bytes(const kvq_geom* geom, int32_t max_seq_len, size_t* bytes) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
    if ((st = check_max_len(geom, max_seq_len)) != KVQ_OK) return st;
    int32_t nw = 0;
    if ((st = workers_for(geom, &nw)) != KVQ_OK) return st;
    *bytes = workspace_need(geom, nw);
    return KVQ_OK;
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_quantize_keys_perchannel(const kvq_geom* geom, const uint16_t* k, int32_t pos0,
                                 int32_t n_tok, uint32_t* k_codes, uint16_t* k_meta,
                                 void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_ptr(k, "k")) != KVQ_OK) return st;
    if ((st = check_ptr(k_codes, "k_codes")) != KVQ_OK) return st;
    if ((st = check_ptr(k_meta, "k_meta")) != KVQ_OK) return st;
    if (pos0 < 0 || n_tok < 0 || pos0 % geom->group || n_tok % geom->group ||
        (int64_t)pos0 + n_tok > geom->capacity)
      return fail(KVQ_ERR_RANGE, "pos0=%d n_tok=%d: need multiples of group=%d within capacity=%d",
                  pos0, n_tok, geom->group, geom->capacity);
    const kvq::Geom g = kvq::to_geom(*geom);
    hipError_t e = kvq::launch_quantize_keys(g, k, (int64_t)n_tok * g.D, pos0, n_tok, k_codes,
                                             k_meta, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "quantize_keys launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_quantize_values_pertoken(const kvq_geom* geom, const uint16_t* v, int32_t pos0,
                                 int32_t n_tok, uint32_t* v_codes, uint16_t* v_meta,
                                 void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_ptr(v, "v")) != KVQ_OK) return st;
    if ((st = check_ptr(v_codes, "v_codes")) != KVQ_OK) return st;
    if ((st = check_ptr(v_meta, "v_meta")) != KVQ_OK) return st;
    if (pos0 < 0 || n_tok < 0 || pos0 % geom->group || n_tok % geom->group ||
        pos0 % KVQ_VBLOCK || n_tok % KVQ_VBLOCK || (int64_t)pos0 + n_tok > geom->capacity)
      return fail(KVQ_ERR_RANGE, "pos0=%d n_tok=%d: need multiples of group=%d and 32 within capacity=%d",
                  pos0, n_tok, geom->group, geom->capacity);
    const kvq::Geom g = kvq::to_geom(*geom);
    hipError_t e = kvq::launch_quantize_values(g, v, (int64_t)n_tok * g.D, pos0, n_tok,
                                               v_codes, v_meta, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "quantize_values launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_prefill(const kvq_geom* geom, const uint16_t* k, const uint16_t* v, int32_t n,
                const kvq_cache* cache, void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(cache)) != KVQ_OK) return st;
    if (n < 0 || n > geom->capacity)
      return fail(KVQ_ERR_RANGE, "n=%d must be in [0, capacity=%d]", n, geom->capacity);
    if (n == 0) return KVQ_OK;
    if ((st = check_ptr(k, "k")) != KVQ_OK) return st;
    if ((st = check_ptr(v, "v")) != KVQ_OK) return st;
    const kvq::Geom g = kvq::to_geom(*geom);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int lqk = packed_len(n, g.R), lqv = packed_len(n, g.Rv);
    const int64_t stride = (int64_t)n * g.D;
    hipError_t e =
        kvq::launch_quantize_keys(g, k, stride, 0, lqk, cache->k_codes, cache->k_meta, s);
    if (e != hipSuccess) return hip_fail(e, "prefill quantize_keys launch");
    e = kvq::launch_quantize_values(g, v, stride, 0, lqv, cache->v_codes, cache->v_meta, s);
    if (e != hipSuccess) return hip_fail(e, "prefill quantize_values launch");
    e = kvq::launch_residual_copy(g, k + (int64_t)lqk * g.D, stride, lqk, n - lqk,
                                  cache->k_res, false, s);
    if (e != hipSuccess) return hip_fail(e, "prefill residual copy launch");
    e = kvq::launch_residual_copy(g, v + (int64_t)lqv * g.D, stride, lqv, n - lqv,
                                  cache->v_res, true, s);
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "prefill residual copy launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_append(const kvq_geom* geom, const uint16_t* k_new, const uint16_t* v_new,
               const int32_t* seq_lens, const kvq_cache* cache, void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(cache)) != KVQ_OK) return st;
    if ((st = check_ptr(k_new, "k_new")) != KVQ_OK) return st;
    if ((st = check_ptr(v_new, "v_new")) != KVQ_OK) return st;
    if ((st = check_lens(seq_lens)) != KVQ_OK) return st;
    hipError_t e = kvq::launch_append(kvq::to_geom(*geom), k_new, v_new, seq_lens, *cache,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "append launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_append_tokens(const kvq_geom* geom, int32_t T, const uint16_t* k_new,
                      const uint16_t* v_new, const int32_t* seq_lens, const kvq_cache* cache,
                      void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_cache(cache)) != KVQ_OK) return st;
    if (T < 1) return fail(KVQ_ERR_RANGE, "T must be >= 1 (got %d)", T);
    if ((st = check_ptr(k_new, "k_new")) != KVQ_OK) return st;
    if ((st = check_ptr(v_new, "v_new")) != KVQ_OK) return st;
    if ((st = check_lens(seq_lens)) != KVQ_OK) return st;
    hipError_t e = kvq::launch_append_tokens(kvq::to_geom(*geom), T, k_new, v_new, seq_lens,
                                             *cache, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "append_tokens launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_decode_partial(const kvq_geom* geom, const uint16_t* q, const kvq_cache* cache,
                       const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                       void* workspace, size_t workspace_bytes, uint16_t* out, void* stream) {
  try {
    kvq::DecodeLaunch L;
    int st = decode_setup(geom, q, cache, seq_lens, max_seq_len, sm_scale, workspace,
                          workspace_bytes, out, &L);
    if (st != KVQ_OK) return st;
    hipError_t e = kvq::launch_decode_partial(L, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "decode_partial launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_decode_combine(const kvq_geom* geom, const uint16_t* q, const kvq_cache* cache,
                       const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                       const void* workspace, size_t workspace_bytes, uint16_t* out,
                       void* stream) {
  try {
    kvq::DecodeLaunch L;
    int st = decode_setup(geom, q, cache, seq_lens, max_seq_len, sm_scale,
                          const_cast<void*>(workspace), workspace_bytes, out, &L);
    if (st != KVQ_OK) return st;
    hipError_t e = kvq::launch_decode_combine(L, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "decode_combine launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_decode_multi_workspace_bytes(const kvq_geom* geom, int32_t T, int32_t max_seq_len,
                                     size_t* bytes) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
    if ((st = check_tokens(geom, T)) != KVQ_OK) return st;
    if ((st = check_max_len(geom, max_seq_len)) != KVQ_OK) return st;
    int32_t nw = 0;
    if ((st = workers_for(geom, &nw, T)) != KVQ_OK) return st;
    *bytes = workspace_need(geom, nw, T);
    return KVQ_OK;
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_decode_attn_multi(const kvq_geom* geom, const uint16_t* q, const kvq_cache* cache,
                          const int32_t* seq_lens, int32_t T, int32_t max_seq_len,
                          float sm_scale, void* workspace, size_t workspace_bytes,
                          uint16_t* out, void* stream) {
  try {
    kvq::DecodeLaunch L;
    int st = decode_setup(geom, q, cache, seq_lens, max_seq_len, sm_scale, workspace,
                          workspace_bytes, out, &L, T);
    if (st != KVQ_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = kvq::launch_decode_partial(L, s);
    if (e != hipSuccess) return hip_fail(e, "decode_partial launch");
    e = kvq::launch_decode_combine(L, s);
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "decode_combine launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_decode_attn(const kvq_geom* geom, const uint16_t* q, const kvq_cache* cache,
                    const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                    void* workspace, size_t workspace_bytes, uint16_t* out, void* stream) {
  int st = kvq_decode_partial(geom, q, cache, seq_lens, max_seq_len, sm_scale, workspace,
                              workspace_bytes, out, stream);
  if (st != KVQ_OK) return st;
  return kvq_decode_combine(geom, q, cache, seq_lens, max_seq_len, sm_scale, workspace,
                            workspace_bytes, out, stream);
}

int kvq_decode_attn_noalloc(const kvq_geom* geom, const uint16_t* q, const kvq_cache* cache,
                            const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                            uint16_t* out, void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    hipError_t e = kvq::noalloc_scratch(&ws, &ws_bytes);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    int32_t n_workers = 0;
    if ((st = workers_for(geom, &n_workers)) != KVQ_OK) return st;
    const size_t need = workspace_need(geom, n_workers);
    if (need > ws_bytes)
      return fail(KVQ_ERR_WORKSPACE,
                  "kvq_decode_attn_noalloc: this geometry's partials need %zu bytes, beyond "
                  "the library's %zu-byte static buffer (use kvq_decode_attn with a workspace)",
                  need, ws_bytes);
    kvq::DecodeLaunch L;
    st = decode_setup(geom, q, cache, seq_lens, max_seq_len, sm_scale, ws, ws_bytes, out, &L);
    if (st != KVQ_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    e = kvq::launch_decode_partial(L, s);
    if (e != hipSuccess) return hip_fail(e, "decode_partial launch");
    e = kvq::launch_decode_combine(L, s);
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "decode_combine launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_bq2_validate_geom(const kvq_bq2_geom* geom) {
  try {
    return check_bq2_geom(geom);
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_bq2_cache_bytes(const kvq_bq2_geom* geom, size_t out[6]) {
  int st = check_bq2_geom(geom);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_ERR_NULL, "out is NULL");
  const size_t units = (size_t)geom->batch * geom->n_kv_heads, C = geom->capacity;
  out[0] = units * (C / 32) * 64 * 2 * 4;         // k_codes
  out[1] = units * (C / 32) * 64 * 2 * 4;         // v_codes
  out[2] = units * C * 2 * 2;                     // k_meta
  out[3] = units * C * 2 * 2;                     // v_meta
  out[4] = units * KVQ_BQ2_SINKS * KVQ_BQ2_HEAD_DIM * 2;  // k_sink
  out[5] = units * KVQ_BQ2_SINKS * KVQ_BQ2_HEAD_DIM * 2;  // v_sink
  return KVQ_OK;
}

int kvq_bq2_decode_workers(const kvq_bq2_geom* geom, int32_t* n_workers) {
  try {
    int st = check_bq2_geom(geom);
    if (st != KVQ_OK) return st;
    if (!n_workers) return fail(KVQ_ERR_NULL, "n_workers is NULL");
    return bq2_workers_for(geom, n_workers);
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_bq2_decode_workspace_bytes(const kvq_bq2_geom* geom, int32_t max_seq_len,
                                   size_t* bytes) {
  try {
    int st = check_bq2_geom(geom);
    if (st != KVQ_OK) return st;
    if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
    if ((st = check_bq2_max_len(geom, max_seq_len)) != KVQ_OK) return st;
    int32_t nw = 0;
    if ((st = bq2_workers_for(geom, &nw)) != KVQ_OK) return st;
    *bytes = bq2_workspace_need(geom, nw);
    return KVQ_OK;
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_bq2_prefill(const kvq_bq2_geom* geom, const uint16_t* k, const uint16_t* v, int32_t n,
                    const kvq_bq2_cache* cache, void* stream) {
  try {
    int st = check_bq2_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_bq2_cache(cache)) != KVQ_OK) return st;
    if (n < 0 || n > geom->capacity)
      return fail(KVQ_ERR_RANGE, "n=%d must be in [0, capacity=%d]", n, geom->capacity);
    if (n == 0) return KVQ_OK;
    if ((st = check_ptr(k, "k")) != KVQ_OK) return st;
    if ((st = check_ptr(v, "v")) != KVQ_OK) return st;
    hipError_t e = kvq::launch_bq2_prefill(kvq::to_geom(*geom), k, v, n, *cache,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "bq2 prefill launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_bq2_append(const kvq_bq2_geom* geom, const uint16_t* k_new, const uint16_t* v_new,
                   const int32_t* seq_lens, const kvq_bq2_cache* cache, void* stream) {
  try {
    int st = check_bq2_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_bq2_cache(cache)) != KVQ_OK) return st;
    if ((st = check_ptr(k_new, "k_new")) != KVQ_OK) return st;
    if ((st = check_ptr(v_new, "v_new")) != KVQ_OK) return st;
    if ((st = check_lens(seq_lens)) != KVQ_OK) return st;
    hipError_t e = kvq::launch_bq2_append(kvq::to_geom(*geom), k_new, v_new, seq_lens, *cache,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "bq2 append launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_bq2_decode_partial(const kvq_bq2_geom* geom, const uint16_t* q,
                           const kvq_bq2_cache* cache, const int32_t* seq_lens,
                           int32_t max_seq_len, float sm_scale, void* workspace,
                           size_t workspace_bytes, uint16_t* out, void* stream) {
  try {
    kvq::Bq2Launch L;
    int st = bq2_decode_setup(geom, q, cache, seq_lens, max_seq_len, sm_scale, workspace,
                              workspace_bytes, out, &L);
    if (st != KVQ_OK) return st;
    hipError_t e = kvq::launch_bq2_decode_partial(L, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "bq2 decode_partial launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_bq2_decode_combine(const kvq_bq2_geom* geom, const uint16_t* q,
                           const kvq_bq2_cache* cache, const int32_t* seq_lens,
                           int32_t max_seq_len, float sm_scale, const void* workspace,
                           size_t workspace_bytes, uint16_t* out, void* stream) {
  try {
    kvq::Bq2Launch L;
    int st = bq2_decode_setup(geom, q, cache, seq_lens, max_seq_len, sm_scale,
                              const_cast<void*>(workspace), workspace_bytes, out, &L);
    if (st != KVQ_OK) return st;
    hipError_t e = kvq::launch_bq2_decode_combine(L, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "bq2 decode_combine launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_bq2_decode_attn(const kvq_bq2_geom* geom, const uint16_t* q,
                        const kvq_bq2_cache* cache, const int32_t* seq_lens,
                        int32_t max_seq_len, float sm_scale, void* workspace,
                        size_t workspace_bytes, uint16_t* out, void* stream) {
  int st = kvq_bq2_decode_partial(geom, q, cache, seq_lens, max_seq_len, sm_scale, workspace,
                                  workspace_bytes, out, stream);
  if (st != KVQ_OK) return st;
  return kvq_bq2_decode_combine(geom, q, cache, seq_lens, max_seq_len, sm_scale, workspace,
                                workspace_bytes, out, stream);
}

// ---- paged cache (kvq_paged.h) --------------------------------------------

int kvq_paged_validate(const kvq_geom* geom, const kvq_paged_cache* cache) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    return check_paged(geom, cache, false);
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_cache_bytes(const kvq_geom* geom, int32_t page_size, int32_t num_pages,
                          size_t out[6]) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if (!out) return fail(KVQ_ERR_NULL, "out is NULL");
    kvq_paged_cache c{};
    c.page_size = page_size;
    c.num_pages = num_pages;
    c.max_pages = page_size > 0 ? (geom->capacity + page_size - 1) / page_size : 0;
    if ((st = check_paged(geom, &c, false)) != KVQ_OK) return st;
    // a pool page is a dense unit of P positions for each of the Hkv heads
    const size_t H = geom->n_kv_heads, D = geom->head_dim, G = geom->group,
                 P = page_size, R = geom->residual, N = num_pages;
    out[0] = N * H * P * (D * geom->k_bits / 32) * 4;          // k_codes
    out[1] = N * H * (P / KVQ_VBLOCK) * D * geom->v_bits * 4;  // v_codes
    out[2] = N * H * (P / G) * D * 2 * 2;                      // k_meta
    out[3] = N * H * P * (D / G) * 2 * 2;                      // v_meta
    const size_t Rv = geom->residual_v > 0 ? geom->residual_v : R;
    out[4] = (size_t)geom->batch * H * R * D * 2;              // k_res
    out[5] = (size_t)geom->batch * H * Rv * D * 2;             // v_res
    return KVQ_OK;
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_decode_workspace_bytes(const kvq_geom* geom, int32_t T, int32_t max_seq_len,
                                     size_t* bytes) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if (!bytes) return fail(KVQ_ERR_NULL, "bytes is NULL");
    if ((st = check_tokens(geom, T)) != KVQ_OK) return st;
    if ((st = check_max_len(geom, max_seq_len)) != KVQ_OK) return st;
    int32_t nw = 0;
    if ((st = workers_for(geom, &nw, T, true)) != KVQ_OK) return st;
    *bytes = workspace_need(geom, nw, T);
    return KVQ_OK;
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_prefill(const kvq_geom* geom, const uint16_t* k, const uint16_t* v, int32_t n,
                      const kvq_paged_cache* cache, void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_paged(geom, cache, true)) != KVQ_OK) return st;
    if (n < 0 || n > geom->capacity)
      return fail(KVQ_ERR_RANGE, "n=%d must be in [0, capacity=%d]", n, geom->capacity);
    if (n == 0) return KVQ_OK;
    if ((st = check_ptr(k, "k")) != KVQ_OK) return st;
    if ((st = check_ptr(v, "v")) != KVQ_OK) return st;
    const kvq::Geom g = kvq::to_geom(*geom, *cache);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int lqk = packed_len(n, g.R), lqv = packed_len(n, g.Rv);
    const int64_t stride = (int64_t)n * g.D;
    hipError_t e =
        kvq::launch_quantize_keys(g, k, stride, 0, lqk, cache->k_codes, cache->k_meta, s);
    if (e != hipSuccess) return hip_fail(e, "prefill quantize_keys launch");
    e = kvq::launch_quantize_values(g, v, stride, 0, lqv, cache->v_codes, cache->v_meta, s);
    if (e != hipSuccess) return hip_fail(e, "prefill quantize_values launch");
    e = kvq::launch_residual_copy(g, k + (int64_t)lqk * g.D, stride, lqk, n - lqk,
                                  cache->k_res, false, s);
    if (e != hipSuccess) return hip_fail(e, "prefill residual copy launch");
    e = kvq::launch_residual_copy(g, v + (int64_t)lqv * g.D, stride, lqv, n - lqv,
                                  cache->v_res, true, s);
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "prefill residual copy launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_append(const kvq_geom* geom, const uint16_t* k_new, const uint16_t* v_new,
                     const int32_t* seq_lens, const kvq_paged_cache* cache, void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_paged(geom, cache, true)) != KVQ_OK) return st;
    if ((st = check_ptr(k_new, "k_new")) != KVQ_OK) return st;
    if ((st = check_ptr(v_new, "v_new")) != KVQ_OK) return st;
    if ((st = check_lens(seq_lens)) != KVQ_OK) return st;
    hipError_t e = kvq::launch_append(kvq::to_geom(*geom, *cache), k_new, v_new, seq_lens,
                                      kvq::pool_view(*cache), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "append launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_append_tokens(const kvq_geom* geom, int32_t T, const uint16_t* k_new,
                            const uint16_t* v_new, const int32_t* seq_lens,
                            const kvq_paged_cache* cache, void* stream) {
  try {
    int st = check_geom(geom);
    if (st != KVQ_OK) return st;
    if ((st = check_paged(geom, cache, true)) != KVQ_OK) return st;
    if (T < 1) return fail(KVQ_ERR_RANGE, "T must be >= 1 (got %d)", T);
    if ((st = check_ptr(k_new, "k_new")) != KVQ_OK) return st;
    if ((st = check_ptr(v_new, "v_new")) != KVQ_OK) return st;
    if ((st = check_lens(seq_lens)) != KVQ_OK) return st;
    hipError_t e =
        kvq::launch_append_tokens(kvq::to_geom(*geom, *cache), T, k_new, v_new, seq_lens,
                                  kvq::pool_view(*cache), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "append_tokens launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_decode_attn_multi(const kvq_geom* geom, const uint16_t* q,
                                const kvq_paged_cache* cache, const int32_t* seq_lens,
                                int32_t T, int32_t max_seq_len, float sm_scale, void* workspace,
                                size_t workspace_bytes, uint16_t* out, void* stream) {
  try {
    if (!cache) return fail(KVQ_ERR_NULL, "cache is NULL");
    const kvq_cache view = kvq::pool_view(*cache);
    kvq::DecodeLaunch L;
    int st = decode_setup(geom, q, &view, seq_lens, max_seq_len, sm_scale, workspace,
                          workspace_bytes, out, &L, T, cache);
    if (st != KVQ_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = kvq::launch_decode_partial(L, s);
    if (e != hipSuccess) return hip_fail(e, "decode_partial launch");
    e = kvq::launch_decode_combine(L, s);
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "decode_combine launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_decode_partial(const kvq_geom* geom, const uint16_t* q,
                             const kvq_paged_cache* cache, const int32_t* seq_lens,
                             int32_t max_seq_len, float sm_scale, void* workspace,
                             size_t workspace_bytes, uint16_t* out, void* stream) {
  try {
    if (!cache) return fail(KVQ_ERR_NULL, "cache is NULL");
    const kvq_cache view = kvq::pool_view(*cache);
    kvq::DecodeLaunch L;
    int st = decode_setup(geom, q, &view, seq_lens, max_seq_len, sm_scale, workspace,
                          workspace_bytes, out, &L, 1, cache);
    if (st != KVQ_OK) return st;
    hipError_t e = kvq::launch_decode_partial(L, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "decode_partial launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_decode_combine(const kvq_geom* geom, const uint16_t* q,
                             const kvq_paged_cache* cache, const int32_t* seq_lens,
                             int32_t max_seq_len, float sm_scale, const void* workspace,
                             size_t workspace_bytes, uint16_t* out, void* stream) {
  try {
    if (!cache) return fail(KVQ_ERR_NULL, "cache is NULL");
    const kvq_cache view = kvq::pool_view(*cache);
    kvq::DecodeLaunch L;
    int st = decode_setup(geom, q, &view, seq_lens, max_seq_len, sm_scale,
                          const_cast<void*>(workspace), workspace_bytes, out, &L, 1, cache);
    if (st != KVQ_OK) return st;
    hipError_t e = kvq::launch_decode_combine(L, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "decode_combine launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_paged_decode_attn(const kvq_geom* geom, const uint16_t* q, const kvq_paged_cache* cache,
                          const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                          void* workspace, size_t workspace_bytes, uint16_t* out,
                          void* stream) {
  return kvq_paged_decode_attn_multi(geom, q, cache, seq_lens, 1, max_seq_len, sm_scale,
                                     workspace, workspace_bytes, out, stream);
}

// ---- measurement aid (kvq_probe.h) ----------------------------------------

int kvq_probe_sink_words(int32_t* words) {
  if (!words) return fail(KVQ_ERR_NULL, "words is NULL");
  *words = kvq::probe_sink_words();
  return KVQ_OK;
}

extern "C++" {
namespace kvq {
// The chunk-stream probe's launcher (kvq_probe.hip).
hipError_t launch_chunk_stream(const void* const (&bufs)[4], int64_t n_chunks,
                               const int32_t (&bytes)[4], int spin, int waves, uint32_t* sink,
                               hipStream_t st);
}  // namespace kvq
}

int kvq_probe_chunk_stream(const void* buf_a, const void* buf_b, const void* buf_c,
                           const void* buf_d, int64_t n_chunks, int32_t bytes_a,
                           int32_t bytes_b, int32_t bytes_c, int32_t bytes_d, int32_t spin,
                           uint32_t* sink, void* stream) {
  try {
    const void* const bufs[4] = {buf_a, buf_b, buf_c, buf_d};
    const int32_t bytes[4] = {bytes_a, bytes_b, bytes_c, bytes_d};
    static const char* const names[4] = {"buf_a", "buf_b", "buf_c", "buf_d"};
    int st = KVQ_OK;
    int64_t total = 0;
    for (int p = 0; p < 4; ++p) {
      if ((st = check_ptr(bufs[p], names[p])) != KVQ_OK) return st;
      if (bytes[p] < 0 || bytes[p] % 512 != 0)
        return fail(KVQ_ERR_RANGE, "piece %d bytes (%d) must be a multiple of 512", p, bytes[p]);
      total += bytes[p];
    }
    if ((st = check_ptr(sink, "sink")) != KVQ_OK) return st;
    if (total <= 0 || total > 4096)
      return fail(KVQ_ERR_RANGE, "a chunk's pieces (%lld bytes) must sum to 1..4096 bytes",
                  (long long)total);
    if (n_chunks <= 0) return fail(KVQ_ERR_RANGE, "n_chunks (%lld) must be positive",
                                   (long long)n_chunks);
    if (spin < 0 || spin > 4096) return fail(KVQ_ERR_RANGE, "spin (%d) must be in [0, 4096]", spin);
    int cus = 0;
    if ((st = cu_count(&cus)) != KVQ_OK) return st;
    const int waves = 2 * 4 * cus;
    if (waves > kvq::probe_sink_words())
      return fail(KVQ_ERR_RANGE, "%d waves exceed the sink's %d words", waves,
                  kvq::probe_sink_words());
    hipError_t e = kvq::launch_chunk_stream(bufs, n_chunks, bytes, spin, waves, sink,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "chunk stream launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  try {
    int st = check_ptr(buf, "buf");
    if (st != KVQ_OK) return st;
    if ((st = check_ptr(sink, "sink")) != KVQ_OK) return st;
    if (bytes == 0 || bytes % 16 != 0)
      return fail(KVQ_ERR_RANGE, "bytes (%zu) must be a positive multiple of 16", bytes);
    hipError_t e = kvq::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "stream read launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

int kvq_probe_stream_read_sweep(const void* buf, size_t bytes, uint32_t* sink,
                                int32_t waves_per_simd, int32_t loads_per_lane,
                                int32_t nontemporal, void* stream) {
  try {
    int st = check_ptr(buf, "buf");
    if (st != KVQ_OK) return st;
    if ((st = check_ptr(sink, "sink")) != KVQ_OK) return st;
    if (bytes == 0 || bytes % 16 != 0)
      return fail(KVQ_ERR_RANGE, "bytes (%zu) must be a positive multiple of 16", bytes);
    if (waves_per_simd < 1 || waves_per_simd > 8)
      return fail(KVQ_ERR_RANGE, "waves_per_simd (%d) must be in [1, 8]", waves_per_simd);
    const int L = loads_per_lane;
    if (L != 1 && L != 2 && L != 4 && L != 8 && L != 16)
      return fail(KVQ_ERR_RANGE, "loads_per_lane (%d) must be 1, 2, 4, 8 or 16", L);
    int cus = 0;
    if ((st = cu_count(&cus)) != KVQ_OK) return st;
    const int waves = waves_per_simd * 4 * cus;
    if (waves > kvq::probe_sink_words())
      return fail(KVQ_ERR_RANGE, "%d waves exceed the sink's %d words", waves,
                  kvq::probe_sink_words());
    if (nontemporal < 0 || nontemporal > 3)
      return fail(KVQ_ERR_RANGE, "nontemporal (%d) must be in [0, 3]", nontemporal);
    if (nontemporal >= 2 && bytes % 1024 != 0)  // whole 1 KB direct loads
      return fail(KVQ_ERR_RANGE, "bytes (%zu) must be a multiple of 1024 for direct loads",
                  bytes);
    hipError_t e = kvq::launch_stream_read_sweep(buf, bytes, sink, waves, L, nontemporal,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "stream read sweep launch");
  } catch (...) {
    return fail(KVQ_ERR_INTERNAL, "unexpected exception");
  }
}

}  // extern "C"
