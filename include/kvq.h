/*
 * kvq.h — C ABI of libkvq: KIVI-style asymmetric low-bit KV-cache quantization
 * fused into single-token decode attention, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [KIVI]  "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 *           (repository digest of jy-yuan/KIVI): sections "核心能力" (core
 *           capabilities), "Overview", "Example".
 *   [KV1]   "KV1-1.2B-Instruct" model card (klein-ml/KV1-1.2B): sections
 *           "Quantization Format: KV1.cpp BQ2_0", "Memory", "Quickstart".
 *   [REC]   "KIVI asymmetric 2-bit KV (2-bit keys / 4-bit values) on
 *           Llama-2-class GQA models" (inference-research record): "Methodology",
 *           "notes".
 *   [KVQ]   "KV Cache Quantization" (mohsenhariri/spectral-kv): "Quantize What
 *           Counts", "Usage".
 *
 * ---------------------------------------------------------------------------
 * THE METHOD
 * ---------------------------------------------------------------------------
 * Keys are quantized per channel: for every channel, a group of G consecutive
 * tokens shares one (scale, min) pair.  Values are quantized per token: every
 * token's head vector is cut into D/G groups of G consecutive channels, each
 * with its own (scale, min).  Codes have b = 2, 4 or 8 bits, chosen separately
 * for keys and values ([KVQ] Usage: the bit range of a budget goes up to 8).
 * The most recent tokens stay in an fp16 residual window of R tokens until the
 * window is full; then it is quantized into packed groups.  ([KIVI] core
 * capabilities, Overview, Example: k_bits, v_bits, group_size,
 * residual_length; [REC] notes: per-channel keys group outlier channels.)
 * Keys and values may have windows of their own length ([KVQ] Usage: a
 * residual length per tensor): R for keys, Rv for values; everything below
 * then holds for each tensor with its own window.
 *
 * Group quantizer (affine, asymmetric; [KV1] Quantization Format gives the
 * formula for b = 2 and states that the fp16-rounded scale and min are used for
 * the codes; the general b form replaces 3 by 2^b - 1):
 *   mn = min x_i, mx = max x_i            (x_i: the fp16 inputs widened to fp32;
 *                                         a zero min or max is taken as +0)
 *   d32 = (mx - mn) / (2^b - 1)           (IEEE fp32 subtract, then IEEE fp32
 *                                          divide, round to nearest even)
 *   scale = fp16(d32), min = fp16(mn)     (round to nearest even; min is exact;
 *                                          a zero scale is stored as +0)
 *   code_i = 0 if scale == 0, else clamp(rne(fp32(fp32(x_i - min) / scale)),
 *                                        0, 2^b - 1)
 *   dequantized x_i = code_i * scale + min          ([KV1] Dequantize)
 *
 * Flush timing (lazy): a token that arrives when the sequence already holds
 * n_before > 0 tokens with n_before % R == 0 first triggers the quantization of
 * positions [n_before - R, n_before) from the residual window into packed rows;
 * then the new token goes to residual slot n_before % R.  So at attention time
 * a sequence of n >= 1 tokens has
 *   r(n)   = ((n - 1) % R) + 1   residual (fp16) tokens: positions [Lq, n)
 *   Lq(n)  = n - r(n)            packed tokens: positions [0, Lq), Lq % R == 0
 * and the current token is always in the residual window.
 *
 * Decode attention for query head h of sequence b (GQA: the KV head is
 * h / (Hq / Hkv), i.e. consecutive query heads share one KV head):
 *   s_t = sm_scale * q_h . k_t   for the n tokens t < n (dequantized keys for
 *                                t < Lq, fp16 residual keys for t >= Lq; with
 *                                Rv, values use their own Lq)
 *   out_h = sum_t softmax(s)_t * v_t     (fp32 accumulation, fp16 result)
 * The result equals softmax attention over the dequantized cache ([KV1]
 * Quickstart: attention over the cache's dequantized values, each token
 * quantized a single time on its way in, is the low-bit result).
 *
 * ---------------------------------------------------------------------------
 * PACKED LAYOUT  (KVQ_LAYOUT_VERSION 3)
 * ---------------------------------------------------------------------------
 * Shapes use: B = batch, Hkv = KV heads, D = head_dim, G = group, R = residual,
 * C = capacity (tokens per sequence), bK / bV = key / value bits.
 * All arrays are dense, C-order, little-endian, caller-owned device memory.
 *
 * Packed tokens are stored in blocks of 32 consecutive positions
 * [32k, 32k + 32); tau = t - 32k is a token's place in its block.  Inside a
 * block the words are in the order in which a 64-lane wave consumes them, so
 * that every lane reads one contiguous run of words: lane l = 16 g + i with
 * lane group g in [0, 4) and i in [0, 16).  Two fixed token orders are used:
 *   key row i of half u (u in {0, 1}):  tau = 8 (i / 4) + 4 u + (i % 4)
 *   value element j of lane group g:    tau = 8 g + j,   j in [0, 8)
 * (the two agree: lane group g's rows 4g..4g+3 of halves 0 and 1 are the
 * tokens 8g + j).  Inside a field, the code order is the one of the 2-bit
 * BQ2_0 block in [KV1] Quantization Format: the first code of a byte takes
 * its lowest bits (extended here to 4-bit fields).
 *
 *   k_codes  uint32 [B][Hkv][C/32][64][2][KW],  KW = D*bK/128.
 *            Entry [k][l][u][w] holds key row i of half u (token tau above) of
 *            block k, restricted to channel slice g = channels
 *            [g*D/4, (g+1)*D/4): its word w holds the 32/bK channels
 *            g*D/4 + w*32/bK + f, channel f of the word in bits f*bK .. +bK-1
 *            (bK = 2, 4).  bK = 8: word w = 2 kc + s holds channels
 *            g*D/4 + 8 kc + 2 s + (0, 1, 4, 5)[f] in byte f.
 *            (A token's natural row of D*bK/32 words is the concatenation of
 *            its 4 slices, word w of slice g being row word g*KW + w.)
 *   k_meta   uint16 [B][Hkv][C/G][D/8][8][2]  fp16 (scale, min) of key group
 *            q = tokens [qG, qG+G); scale first, as the scale field precedes
 *            the min field in the [KV1] BQ2_0 block.  Entry [q][r][e] is the
 *            channel that element e of k-chunk r feeds:
 *              r = g*(D/32) + kc (g in [0,4), kc in [0, D/32)),
 *              channel = g*D/4 + base + (e / 2) + off * (e % 2)
 *            with base = 16*(kc/2) + 4*(kc%2), off = 8 for bK = 2 and
 *                 base = 8*kc,                  off = 4 for bK = 4, 8
 *            (the channels of key word fields: bits 0..15 of a word hold the
 *            even elements, bits 16..31 the odd ones).
 *   v_codes  uint32 [B][Hkv][C/32][64][NW],  NW = D*bV/64.
 *            bV = 4: entry [k][l][n] (n in [0, D/16)) holds channel 16n + i;
 *              token tau = 8g + j sits in bits 4*(j/2) + 16*(j%2) .. +3.
 *            bV = 2: entry [k][l][m] (m in [0, D/32)) holds channels
 *              16(2m + h) + i for h in {0, 1}; token tau = 8g + j of channel
 *              16(2m + h) + i sits in bits 8h + 2*(j/2) + 16*(j%2) .. +1.
 *            bV = 8: entries [k][l][2n], [k][l][2n + 1] (n in [0, D/16)) hold
 *              channel 16n + i; token tau = 8g + j sits in entry 2n + j/4,
 *              bits 8*((j%4)/2) + 16*(j%2) .. +7.
 *   v_meta   uint16 [B][Hkv][C/32][4][D/G][8][2]  fp16 (scale, min) of token
 *            32k + 8g + j and channel group gamma = channels
 *            [gamma*G, gamma*G + G) at entry [k][g][gamma][j].
 *   k_res    uint16 [B][Hkv][R][D]     fp16 residual keys; position p lives
 *            in slot p % R, one row of D channels per slot.
 *   v_res    uint16 [B][Hkv][Rv/32][D/16][64][8]  fp16 residual values in the
 *            value consumer order: entry [k][n][l][j] (l = 16g + i) is slot
 *            32k + 8g + j, channel 16n + i; position p lives in slot p % Rv
 *            (Rv = residual_v, or R when residual_v is 0).
 *
 * Earlier versions are retired: version 1 (token-major key rows,
 * channel-major value blocks) had scattered per-lane addresses and its loads
 * took about 1.2x as long as contiguous ones; version 2 kept v_res in token
 * rows, which the decode kernel had to transpose through LDS.
 *
 * Constraints (checked, KVQ_ERR_GEOM / KVQ_ERR_BITS otherwise):
 *   batch >= 1; n_kv_heads >= 1; n_q_heads % n_kv_heads == 0 and
 *   n_q_heads / n_kv_heads in {1, 2, 4, 8, 16}; head_dim in {64, 128};
 *   k_bits, v_bits in {2, 4, 8}; group in {32, 64, 128}, group <= head_dim,
 *   head_dim % group == 0; residual % group == 0; capacity % residual == 0;
 *   capacity <= 2^24; residual_v == 0, or residual_v % group == 0 and
 *   capacity % residual_v == 0.
 *
 * ---------------------------------------------------------------------------
 * CONVENTIONS
 * ---------------------------------------------------------------------------
 * Ownership: the caller allocates and frees every buffer.  libkvq never
 *   allocates device memory, never frees, and keeps no pointer after a call
 *   returns.  Its only state is a thread-local error string and a per-device
 *   cache of the compute-unit count.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Every call only enqueues work on that stream and returns; nothing
 *   synchronizes.  Faults inside kernels surface at the caller's next sync.
 * Errors: every call returns an int status (KVQ_OK = 0, negative on error).
 *   All checks are done on the host before anything is enqueued, so a failing
 *   call has no effect.  kvq_last_error() gives the text of the last failure on
 *   the calling thread.  Device data (seq_lens values) cannot be checked on the
 *   host: out-of-range lengths are clamped inside the kernels so that no access
 *   leaves the buffers, and the affected outputs are documented per call.
 * Alignment: every device pointer must be 16-byte aligned, except seq_lens
 *   (4-byte aligned) (KVQ_ERR_ALIGN).
 * Thread safety: calls may be made from several host threads; calls whose
 *   device work overlaps on the same buffers race, as any kernels would.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 2
#define KVQ_LAYOUT_VERSION 3
#define KVQ_VBLOCK 32 /* tokens per v_codes block */

enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = -1,      /* a required pointer is NULL */
  KVQ_ERR_GEOM = -2,      /* geometry violates the constraints above */
  KVQ_ERR_BITS = -3,      /* k_bits / v_bits not in {2, 4, 8} */
  KVQ_ERR_ALIGN = -4,     /* a device pointer is not 16-byte aligned */
  KVQ_ERR_WORKSPACE = -5, /* workspace missing or too small */
  KVQ_ERR_RANGE = -6,     /* a token range / length argument is out of range */
  KVQ_ERR_HIP = -7,       /* a HIP runtime call failed (text in kvq_last_error) */
  KVQ_ERR_INTERNAL = -8   /* unexpected internal failure */
};

/* Geometry of one attention layer's cache. */
typedef struct kvq_geom {
  int32_t batch;      /* B: sequences */
  int32_t n_q_heads;  /* Hq: query heads */
  int32_t n_kv_heads; /* Hkv: KV heads; Hq / Hkv query heads share one */
  int32_t head_dim;   /* D: 64 or 128 */
  int32_t k_bits;     /* bK: 2, 4 or 8 */
  int32_t v_bits;     /* bV: 2, 4 or 8 */
  int32_t group;      /* G: tokens per key group = channels per value group */
  int32_t residual;   /* R: fp16 residual window length, multiple of G (the key
                         window's when residual_v is set) */
  int32_t capacity;   /* C: max tokens per sequence, multiple of R (and Rv) */
  int32_t residual_v; /* Rv: value window length, multiple of G; 0: R */
} kvq_geom;

/* The six device buffers of one layer's cache (layout above). */
typedef struct kvq_cache {
  uint32_t *k_codes;
  uint32_t *v_codes;
  uint16_t *k_meta;
  uint16_t *v_meta;
  uint16_t *k_res;
  uint16_t *v_res;
} kvq_cache;

/* ----- version, errors, sizes (host only, no device work) ----------------- */

int kvq_abi_version(void);    /* returns KVQ_ABI_VERSION */
int kvq_layout_version(void); /* returns KVQ_LAYOUT_VERSION */

/* Static text for a status code (never NULL). */
const char *kvq_status_str(int status);

/* Text describing the last failing call on this thread ("" if none). */
const char *kvq_last_error(void);

/* Checks a geometry against the constraints above. */
int kvq_validate_geom(const kvq_geom *geom);

/* Byte sizes of the six cache buffers, in the order k_codes, v_codes, k_meta,
 * v_meta, k_res, v_res.  out must hold 6 entries. */
int kvq_cache_bytes(const kvq_geom *geom, size_t out[6]);

/* Worker waves of the decode partial kernel on the current device: the
 * waves the GPU keeps resident at once for this geometry (from the kernel's
 * register and LDS use, times the compute-unit count; queried once per device).
 * The packed 32-token chunks of all (sequence, KV head) units are split into
 * that many equal contiguous shares, one per wave (split-context attention with
 * balanced splits for any mix of sequence lengths). */
int kvq_decode_workers(const kvq_geom *geom, int32_t *n_workers);

/* Workspace bytes kvq_decode_attn needs: fp32 partials, one per (worker wave,
 * unit) pair a launch produces, at most kvq_decode_workers() + B * Hkv of them,
 * each [Hq/Hkv][head_dim + 4].  max_seq_len is range-checked only. */
int kvq_decode_workspace_bytes(const kvq_geom *geom, int32_t max_seq_len,
                               size_t *bytes);

/* ----- quantization of a packed prefix ------------------------------------ */

/* Per-channel key quantization of positions [pos0, pos0 + n_tok) of every
 * sequence ([KIVI] core capabilities and Overview: keys per channel; [KV1]
 * Quantization Format: the group quantizer).
 *   k       device fp16 [B][Hkv][n_tok][D]: the keys of those positions.
 *   pos0    first position; multiple of G.   n_tok: multiple of G, >= 0.
 *   pos0 + n_tok <= capacity (KVQ_ERR_RANGE otherwise).
 *   k_codes, k_meta: the cache buffers; rows [pos0, pos0+n_tok) of k_codes and
 *   key groups [pos0/G, (pos0+n_tok)/G) of k_meta are written, nothing else. */
int kvq_quantize_keys_perchannel(const kvq_geom *geom, const uint16_t *k,
                                 int32_t pos0, int32_t n_tok,
                                 uint32_t *k_codes, uint16_t *k_meta,
                                 void *stream);

/* Per-token value quantization of positions [pos0, pos0 + n_tok) ([KIVI] core
 * capabilities and Overview: values per token).
 *   v       device fp16 [B][Hkv][n_tok][D].
 *   pos0, n_tok: multiples of KVQ_VBLOCK (32) and of G; pos0+n_tok <= capacity.
 *   v_codes and v_meta blocks [pos0/32, (pos0+n_tok)/32) are written, nothing
 *   else. */
int kvq_quantize_values_pertoken(const kvq_geom *geom, const uint16_t *v,
                                 int32_t pos0, int32_t n_tok,
                                 uint32_t *v_codes, uint16_t *v_meta,
                                 void *stream);

/* Sets up every sequence of the cache as a prefix of n tokens, with the state
 * the lazy flush rule gives after n single-token appends: positions [0, Lq(n))
 * quantized (both calls above), positions [Lq(n), n) copied to residual slots
 * p % R.  Lq(0) = 0.
 *   k, v    device fp16 [B][Hkv][n][D].   0 <= n <= capacity. */
int kvq_prefill(const kvq_geom *geom, const uint16_t *k, const uint16_t *v,
                int32_t n, const kvq_cache *cache, void *stream);

/* ----- decode step --------------------------------------------------------- */

/* Appends one token per sequence ([KIVI] core capabilities: the recent tokens
 * stay fp16; the window is flushed into packed groups when it is full).
 *   k_new, v_new  device fp16 [B][Hkv][D]: the new token's key and value.
 *   seq_lens      device int32 [B]: tokens each sequence holds BEFORE this
 *                 token.  Not modified: the caller advances it (once per step,
 *                 after every layer has appended).
 * For every sequence with n = seq_lens[b]: if n > 0 and n % R == 0, positions
 * [n - R, n) are quantized from the residual window into packed rows
 * (bit-identical to kvq_quantize_* on the same tokens); then the new token is
 * written to slot n % R.  A sequence with n < 0 or n >= capacity is left
 * untouched (no write), which is the caller's error. */
int kvq_append(const kvq_geom *geom, const uint16_t *k_new,
               const uint16_t *v_new, const int32_t *seq_lens,
               const kvq_cache *cache, void *stream);

/* Appends T tokens per sequence in one call: the new tokens of a multi-token
 * decode step, before kvq_decode_attn_multi ([KIVI] core capabilities, as
 * kvq_append).  The cache ends bit-identical to T kvq_append calls, token t
 * with k_new[:, t], v_new[:, t] and lengths seq_lens + t (a window that fills
 * part-way is flushed before the token that finds it full).
 *   T             host int32, >= 1.
 *   k_new, v_new  device fp16 [B][T][Hkv][D]: the new tokens, oldest first.
 *   seq_lens      device int32 [B]: tokens each sequence holds BEFORE the
 *                 first of them.  Not modified.
 * A sequence with n = seq_lens[b] < 0 or n + T > capacity is left untouched
 * (no write), which is the caller's error.  One workgroup per (sequence, KV
 * head) does its tokens in order, so a call that flushes takes longer than
 * one that does not. */
int kvq_append_tokens(const kvq_geom *geom, int32_t T, const uint16_t *k_new,
                      const uint16_t *v_new, const int32_t *seq_lens,
                      const kvq_cache *cache, void *stream);

/* Single-token decode attention over the packed cache plus the residual window
 * (split-context partial softmax over the packed tokens, then a combine that
 * also covers the fp16 residual window; GQA heads of one KV head are processed
 * together).
 *   q           device fp16 [B][Hq][D]: the current token's queries.
 *   seq_lens    device int32 [B]: tokens per sequence INCLUDING the current one
 *               (the current token must already be appended).
 *   max_seq_len host int32: an upper bound of every seq_lens[b];
 *               1 <= max_seq_len <= capacity.
 *   sm_scale    softmax scale (1/sqrt(D) for standard attention).
 *   workspace   device memory of at least kvq_decode_workspace_bytes(geom,
 *               max_seq_len) bytes, 16-byte aligned; contents on entry do not
 *               matter; overwritten.
 *   out         device fp16 [B][Hq][D].
 * A sequence with seq_lens[b] == 0 gets out = 0.  A sequence whose length is
 * negative or above max_seq_len or capacity gets out = NaN (no memory outside
 * the buffers is read). */
int kvq_decode_attn(const kvq_geom *geom, const uint16_t *q,
                    const kvq_cache *cache, const int32_t *seq_lens,
                    int32_t max_seq_len, float sm_scale, void *workspace,
                    size_t workspace_bytes, uint16_t *out, void *stream);

/* The two phases of kvq_decode_attn, for callers that time or schedule them
 * apart.  kvq_decode_attn(...) == kvq_decode_partial(...) followed by
 * kvq_decode_combine(...) on the same stream with the same arguments.
 * kvq_decode_partial covers every token (packed and residual window), writing
 * (max, sum, weighted value sum) partials into the workspace, and does not
 * touch out; kvq_decode_combine merges a unit's partials and writes out. */
int kvq_decode_partial(const kvq_geom *geom, const uint16_t *q,
                       const kvq_cache *cache, const int32_t *seq_lens,
                       int32_t max_seq_len, float sm_scale, void *workspace,
                       size_t workspace_bytes, uint16_t *out, void *stream);
int kvq_decode_combine(const kvq_geom *geom, const uint16_t *q,
                       const kvq_cache *cache, const int32_t *seq_lens,
                       int32_t max_seq_len, float sm_scale,
                       const void *workspace, size_t workspace_bytes,
                       uint16_t *out, void *stream);

/* kvq_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results as kvq_decode_attn (the same kernels, bit for
 * bit), but the split partials go to a static device array of the library,
 * KVQ_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the first call on a
 * device until the process ends.  The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine.
 *   A geometry whose partials need more than KVQ_NOALLOC_SCRATCH_BYTES
 *   (kvq_decode_workspace_bytes) fails with KVQ_ERR_WORKSPACE before any
 *   launch; use kvq_decode_attn with a workspace for it.
 *   Nothing in the array needs to start at zero: every partial the combine
 *   reads is written by the same call's partial kernel first, and the array
 *   keeps the last call's contents.
 *   Every call on one GPU shares that GPU's array: calls on one stream are
 *   ordered, but calls that overlap on one GPU (two streams, two threads, two
 *   captured graphs replayed concurrently) race and give wrong results. */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int kvq_decode_attn_noalloc(const kvq_geom *geom, const uint16_t *q,
                            const kvq_cache *cache, const int32_t *seq_lens,
                            int32_t max_seq_len, float sm_scale, uint16_t *out,
                            void *stream);

/* ----- several query tokens per sequence ----------------------------------- */

/* Attention of the last T positions of every sequence at once (verification
 * of T drafted tokens, or a prefill chunk, over the packed cache; [KIVI] core
 * capabilities: prefill works alongside the quantized cache).  The T tokens
 * must already be appended.  Query token i (0 <= i < T) sits at position
 * n - T + i and attends causally: to positions [0, n - T + i] of the cache as
 * it stands at length n (packed below Lq(n), residual window above),
 *   out_i = sum_{t <= n-T+i} softmax(s)_t v_t,  s_t = sm_scale * q_i . k_t.
 * Every cache byte is read once for all T tokens (the T * Hq/Hkv rows of a KV
 * head are one matrix-core tile).
 *   q        device fp16 [B][T][Hq][D];  out: device fp16 [B][T][Hq][D].
 *   seq_lens device int32 [B]: positions per sequence INCLUDING the T tokens.
 *   T        >= 1, T * Hq/Hkv in {1, 2, 4, 8, 16}, T <= max_seq_len
 *            (KVQ_ERR_RANGE otherwise).
 *   workspace at least kvq_decode_multi_workspace_bytes(geom, T, max_seq_len).
 * T = 1 is kvq_decode_attn.  A row whose query token sees no position (n < T)
 * gets 0; lengths outside [0, max_seq_len] give NaN as in kvq_decode_attn. */
int kvq_decode_multi_workspace_bytes(const kvq_geom *geom, int32_t T,
                                     int32_t max_seq_len, size_t *bytes);
int kvq_decode_attn_multi(const kvq_geom *geom, const uint16_t *q,
                          const kvq_cache *cache, const int32_t *seq_lens,
                          int32_t T, int32_t max_seq_len, float sm_scale,
                          void *workspace, size_t workspace_bytes,
                          uint16_t *out, void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KVQ_H_ */
