/*
 * kvq_paged.h — C ABI of libkvq for the asymmetric low-bit KV cache of kvq.h
 * held in fixed-size pages of a shared pool and addressed through a block
 * table, the form in which a serving engine hands out cache memory, on AMD
 * Instinct MI355X (gfx950).  Status codes, streams, ownership, alignment and
 * error conventions are those of kvq.h.
 *
 * Source: [REC] "KIVI asymmetric 2-bit KV ... on Llama-2-class GQA models",
 * Methodology and notes (the quantized cache is carried into engines, vLLM
 * among them, whose caches are paged); what is computed is exactly that of
 * kvq.h ([KIVI] core capabilities and Overview).  The pages give no page
 * layout: the one below is this library's.
 *
 * ---------------------------------------------------------------------------
 * LAYOUT
 * ---------------------------------------------------------------------------
 * Page size P (tokens): a power of two, P >= 32, P a multiple of G.  Logical
 * page j of sequence b holds positions [j P, (j + 1) P) of every KV head of
 * the sequence; block_table[b][j] names the pool page that stores it.  A pool
 * page holds, for each KV head h in [0, Hkv) one after the other, that head's
 * P/32 packed 32-position chunks exactly as kvq.h lays out a dense unit's
 * chunks (same words, same order, same meta entries):
 *   k_codes  uint32 [num_pages][Hkv][P/32][64][2][KW]
 *   v_codes  uint32 [num_pages][Hkv][P/32][64][NW]
 *   k_meta   uint16 [num_pages][Hkv][P/G][D/8][8][2]
 *   v_meta   uint16 [num_pages][Hkv][P/32][4][D/G][8][2]
 * (KW, NW and the entry order inside a chunk as in kvq.h).  The fp16 residual
 * windows are not paged (they are a fixed R positions per sequence):
 *   k_res, v_res  exactly as in kvq.h, [B][Hkv][...] per sequence.
 * So a dense kvq.h cache is this layout with P = capacity, num_pages = B and
 * block_table[b][0] = b.
 *
 * A sequence of n tokens needs valid entries [0, ceil(Lq(n) / P)) of its
 * row (Lq(n) as in kvq.h; with a separate value window, the larger of the key
 * and value packed lengths): only the pages they name are used.  Decode may
 * read any entry of the row, [0, max_pages) (it loads windows of 64 entries,
 * and its first chunk is requested before the lengths are known), so every
 * entry must be readable memory; entries past the needed ones need not hold
 * valid page numbers, and their values do not affect any result.  A needed
 * entry outside [0, num_pages) makes decode give NaN for that sequence and
 * makes the writers skip that page (nothing outside the pools is read or
 * written).  Pages may be shared by several sequences for reading (a
 * common prefix); a call that writes a page (the flush of an append, a
 * prefill) must be the only one using it.
 *
 * Constraints (KVQ_ERR_GEOM otherwise): the geometry as in kvq.h;
 * page_size as above; max_pages >= 1 and max_pages * page_size >= capacity;
 * num_pages >= 1.
 */
#ifndef KVQ_PAGED_H_
#define KVQ_PAGED_H_

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One layer's paged cache: the four page pools, the per-sequence residual
 * windows, and the block table (device memory, caller-owned). */
typedef struct kvq_paged_cache {
  uint32_t *k_codes;           /* pool, layout above */
  uint32_t *v_codes;           /* pool */
  uint16_t *k_meta;            /* pool */
  uint16_t *v_meta;            /* pool */
  uint16_t *k_res;             /* [B][Hkv][R][D], as kvq.h */
  uint16_t *v_res;             /* [B][Hkv][R/32][D/16][64][8], as kvq.h */
  const int32_t *block_table;  /* device int32 [B][max_pages], 4-byte aligned */
  int32_t page_size;           /* P */
  int32_t max_pages;           /* table entries per sequence */
  int32_t num_pages;           /* pages in each pool */
} kvq_paged_cache;

/* Checks the geometry and the cache's page parameters (pointers are not
 * looked at). */
int kvq_paged_validate(const kvq_geom *geom, const kvq_paged_cache *cache);

/* Byte sizes of the six buffers for the given page size and pool pages, in the
 * order k_codes, v_codes, k_meta, v_meta (whole pools), k_res, v_res.  out
 * must hold 6 entries. */
int kvq_paged_cache_bytes(const kvq_geom *geom, int32_t page_size, int32_t num_pages,
                          size_t out[6]);

/* Workspace bytes of kvq_paged_decode_attn (T = 1) and
 * kvq_paged_decode_attn_multi (T query tokens per sequence). */
int kvq_paged_decode_workspace_bytes(const kvq_geom *geom, int32_t T, int32_t max_seq_len,
                                     size_t *bytes);

/* kvq_prefill into the paged cache: every sequence becomes a prefix of n
 * tokens (positions below Lq(n) packed into their pages, the rest in the
 * residual window).  k, v device fp16 [B][Hkv][n][D]; 0 <= n <= capacity. */
int kvq_paged_prefill(const kvq_geom *geom, const uint16_t *k, const uint16_t *v,
                      int32_t n, const kvq_paged_cache *cache, void *stream);

/* kvq_append into the paged cache (same arguments and rules); a flush writes
 * the packed positions [n - R, n) into their pages. */
int kvq_paged_append(const kvq_geom *geom, const uint16_t *k_new, const uint16_t *v_new,
                     const int32_t *seq_lens, const kvq_paged_cache *cache, void *stream);

/* kvq_append_tokens into the paged cache (same arguments and rules). */
int kvq_paged_append_tokens(const kvq_geom *geom, int32_t T, const uint16_t *k_new,
                            const uint16_t *v_new, const int32_t *seq_lens,
                            const kvq_paged_cache *cache, void *stream);

/* kvq_decode_attn over the paged cache: same arguments, rules and results
 * as over a dense cache holding the same positions (the split of the work may
 * differ, and with it the rounding of the partial sums). */
int kvq_paged_decode_attn(const kvq_geom *geom, const uint16_t *q,
                          const kvq_paged_cache *cache, const int32_t *seq_lens,
                          int32_t max_seq_len, float sm_scale, void *workspace,
                          size_t workspace_bytes, uint16_t *out, void *stream);

/* The two phases of kvq_paged_decode_attn (as kvq_decode_partial and
 * kvq_decode_combine are those of kvq_decode_attn). */
int kvq_paged_decode_partial(const kvq_geom *geom, const uint16_t *q,
                             const kvq_paged_cache *cache, const int32_t *seq_lens,
                             int32_t max_seq_len, float sm_scale, void *workspace,
                             size_t workspace_bytes, uint16_t *out, void *stream);
int kvq_paged_decode_combine(const kvq_geom *geom, const uint16_t *q,
                             const kvq_paged_cache *cache, const int32_t *seq_lens,
                             int32_t max_seq_len, float sm_scale, const void *workspace,
                             size_t workspace_bytes, uint16_t *out, void *stream);

/* kvq_decode_attn_multi over the paged cache (T query tokens per sequence,
 * causal over the last T positions; same arguments and rules). */
int kvq_paged_decode_attn_multi(const kvq_geom *geom, const uint16_t *q,
                                const kvq_paged_cache *cache, const int32_t *seq_lens,
                                int32_t T, int32_t max_seq_len, float sm_scale,
                                void *workspace, size_t workspace_bytes, uint16_t *out,
                                void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KVQ_PAGED_H_ */
