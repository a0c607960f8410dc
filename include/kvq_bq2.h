/*
 * kvq_bq2.h — C ABI of libkvq for the rotated per-token 2-bit KV cache format
 * (KV1's BQ2_0) and single-token decode attention over it, on AMD Instinct
 * MI355X (gfx950).  Status codes, streams, ownership, alignment and error
 * conventions are those of kvq.h.
 *
 * Source: [KV1] "KV1-1.2B-Instruct" model card (klein-ml/KV1-1.2B), sections
 * "Quantization Format: KV1.cpp BQ2_0", "Model Overview", "Memory".
 *
 * ---------------------------------------------------------------------------
 * THE FORMAT
 * ---------------------------------------------------------------------------
 * Head dim 64.  Every key and value head vector is first rotated by the
 * normalized 64x64 Sylvester Hadamard matrix H (H[r][c] = (-1)^popcount(r&c)/8,
 * H H = I); scores are unchanged by the rotation, and the attention output is
 * rotated back by H per head ([KV1] Quantization Format, Hadamard rotation).
 * The rotated vector x is formed exactly and rounded once to fp32.
 * Positions 0..3 of a sequence (attention sinks) keep x rounded to fp16.
 * Every other position becomes one block of 64 values, a single time, at its
 * append (in fp32, [KV1] Quantization Format):
 *   mn = min x_c (a zero min taken as +0), mx = max x_c
 *   d = fp16(max((mx - mn) / 3, 1e-6))     (IEEE fp32 ops, round to nearest even)
 *   m = fp16(mn)
 *   code_c = clamp(rne(fp32(fp32(x_c - m) / d)), 0, 3)   (fp16-rounded d, m)
 *   dequantized x_c = code_c * d + m
 * There is no fp16 window: a sequence of n tokens has min(n, 4) sinks and
 * n - min(n, 4) quantized positions.  Precondition (not checked): the inputs
 * are finite and small enough that the rotated entries and (max - min) / 3 fit
 * fp16 (|input| < 8188 suffices).
 *
 * Decode attention for query head h (KV head h / (Hq / Hkv)):
 *   qH = H q,  s_t = sm_scale * qH . x^K_t,  o = sum_t softmax(s)_t x^V_t,
 *   out = H o   (fp32 accumulation, fp16 result)
 * over all n positions, with x_t the dequantized or sink vectors.
 *
 * ---------------------------------------------------------------------------
 * LAYOUT  (tau = t % 32; lane l = 16 g + i, g in [0, 4), i in [0, 16))
 * ---------------------------------------------------------------------------
 *   k_codes uint32 [B][Hkv][C/32][64][2]: entry [k][l][u] holds the codes of
 *           token 32k + 8 (i/4) + 4u + (i%4), channels 16g .. 16g + 15,
 *           channel 16g + f in bits 2f, 2f + 1: word g (little-endian) of the
 *           16 code bytes of that token's BQ2_0 block.
 *   v_codes uint32 [B][Hkv][C/32][64][2]: entry [k][l][m] holds channels
 *           16 (2m + h) + i, h in {0, 1}; token 32k + 8g + j of channel
 *           16 (2m + h) + i in bits 8h + 2 (j/2) + 16 (j%2) .. +1.
 *   k_meta, v_meta uint16 [B][Hkv][C][2]: fp16 (d, m) of position t.
 *   k_sink  uint16 [B][Hkv][4][64]: fp16 rotated key of position s < 4.
 *   v_sink  uint16 [B][Hkv][64][4]: fp16 rotated value of position s < 4,
 *           channel-major (entry [c][s]).
 * Positions 0..3 of k_codes, v_codes, k_meta and v_meta are never written
 * nor read.
 *
 * Constraints (KVQ_ERR_GEOM otherwise): batch >= 1, n_kv_heads >= 1,
 * n_q_heads / n_kv_heads in {1, 2, 4} (the decode kernel gives every query
 * head four matrix-core columns), capacity a positive multiple of 32,
 * capacity <= 2^24.
 */
#ifndef KVQ_BQ2_H_
#define KVQ_BQ2_H_

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_BQ2_HEAD_DIM 64
#define KVQ_BQ2_SINKS 4

/* Geometry of one attention layer's cache in this format. */
typedef struct kvq_bq2_geom {
  int32_t batch;      /* B */
  int32_t n_q_heads;  /* Hq */
  int32_t n_kv_heads; /* Hkv */
  int32_t capacity;   /* C: positions per sequence, multiple of 32 */
} kvq_bq2_geom;

/* The six device buffers of one layer's cache (layout above). */
typedef struct kvq_bq2_cache {
  uint32_t *k_codes;
  uint32_t *v_codes;
  uint16_t *k_meta;
  uint16_t *v_meta;
  uint16_t *k_sink;
  uint16_t *v_sink;
} kvq_bq2_cache;

/* Checks a geometry against the constraints above. */
int kvq_bq2_validate_geom(const kvq_bq2_geom *geom);

/* Byte sizes of the six buffers in the order k_codes, v_codes, k_meta, v_meta,
 * k_sink, v_sink.  out must hold 6 entries. */
int kvq_bq2_cache_bytes(const kvq_bq2_geom *geom, size_t out[6]);

/* Worker waves of the decode partial kernel on the current device (resident
 * waves per compute unit times compute units; queried once per device). */
int kvq_bq2_decode_workers(const kvq_bq2_geom *geom, int32_t *n_workers);

/* Workspace bytes kvq_bq2_decode_attn needs: fp32 partials, at most
 * kvq_bq2_decode_workers() + B * Hkv of them, each [Hq/Hkv][68].
 * max_seq_len is range-checked only. */
int kvq_bq2_decode_workspace_bytes(const kvq_bq2_geom *geom, int32_t max_seq_len,
                                   size_t *bytes);

/* Stores positions [0, n) of every sequence: rotation, then sinks or one
 * quantized block per position, exactly as n single-token appends would.
 *   k, v  device fp16 [B][Hkv][n][64]: the (unrotated) keys and values.
 *   0 <= n <= capacity (KVQ_ERR_RANGE otherwise).
 * Nothing past the 32-position chunk holding position n - 1 is written; value
 * code words of that chunk are written whole (fields of positions >= n set to
 * 0, which is harmless: those positions are unspecified until appended). */
int kvq_bq2_prefill(const kvq_bq2_geom *geom, const uint16_t *k, const uint16_t *v,
                    int32_t n, const kvq_bq2_cache *cache, void *stream);

/* Appends one token per sequence at position seq_lens[b] (the count held
 * BEFORE it; seq_lens is device int32 [B] and is not modified).
 *   k_new, v_new  device fp16 [B][Hkv][64] (unrotated).
 * A sequence with seq_lens[b] < 0 or >= capacity is left untouched. */
int kvq_bq2_append(const kvq_bq2_geom *geom, const uint16_t *k_new,
                   const uint16_t *v_new, const int32_t *seq_lens,
                   const kvq_bq2_cache *cache, void *stream);

/* Single-token decode attention ([KV1] Quantization Format: rotation of the
 * query, attention over the rotated cache, output rotated back).
 *   q           device fp16 [B][Hq][64] (unrotated).
 *   seq_lens    device int32 [B]: positions INCLUDING the current one.
 *   max_seq_len host int32, 1 <= max_seq_len <= capacity, >= every length.
 *   workspace   at least kvq_bq2_decode_workspace_bytes() bytes, 16-byte
 *               aligned; overwritten.
 *   out         device fp16 [B][Hq][64].
 * seq_lens[b] == 0 gives out = 0; a negative length or one above max_seq_len
 * or capacity gives out = NaN (nothing outside the buffers is read). */
int kvq_bq2_decode_attn(const kvq_bq2_geom *geom, const uint16_t *q,
                        const kvq_bq2_cache *cache, const int32_t *seq_lens,
                        int32_t max_seq_len, float sm_scale, void *workspace,
                        size_t workspace_bytes, uint16_t *out, void *stream);

/* The two phases of kvq_bq2_decode_attn (same arguments, same stream): the
 * partial kernel writes (max, sum, weighted value sum) partials into the
 * workspace; the combine merges them, rotates the result back and writes
 * out. */
int kvq_bq2_decode_partial(const kvq_bq2_geom *geom, const uint16_t *q,
                           const kvq_bq2_cache *cache, const int32_t *seq_lens,
                           int32_t max_seq_len, float sm_scale, void *workspace,
                           size_t workspace_bytes, uint16_t *out, void *stream);
int kvq_bq2_decode_combine(const kvq_bq2_geom *geom, const uint16_t *q,
                           const kvq_bq2_cache *cache, const int32_t *seq_lens,
                           int32_t max_seq_len, float sm_scale,
                           const void *workspace, size_t workspace_bytes,
                           uint16_t *out, void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KVQ_BQ2_H_ */
