/*
 * bq2_oracle.c — plain, slow CPU oracle for the rotated per-token 2-bit KV
 * cache format (KV1's BQ2_0) and single-token decode attention over it.
 *
 * TEST INFRASTRUCTURE ONLY, like kvq_oracle.c (whose software fp16 conversion
 * it uses).  It shares nothing with the GPU library: the packed layout is
 * restated below from its written specification.
 *
 * Source: [KV1] "KV1-1.2B-Instruct" model card, sections "Quantization Format:
 * KV1.cpp BQ2_0" (one block for each position and KV head, covering its 64 channels:
 * fp16 scale d, fp16 min m, sixteen bytes of 2-bit codes with code i of a byte
 * at bit 2i; quantize in fp32 with d = fp16(max((max - min)/3, 1e-6)),
 * m = fp16(min), code = clamp(round half to even((x - m)/d), 0, 3) using the
 * fp16-rounded d and m; dequantize as code * d + m; Q, K and V multiplied by
 * the normalized 64x64 Sylvester Hadamard matrix H (H H = I) after RoPE, so
 * the stored K and V are rotated while q.k is not changed, and each head's
 * attention output rotated back by H; positions 0-3 keep full-precision K/V), and "Model
 * Overview" (32 query heads, 8 KV heads, head dim 64, 4 fp16 sink tokens).
 *
 * Readings where the page is silent (each listed in the design notes):
 *   - the rotated vector is formed exactly (fp64: 64 fp16 terms scaled by 1/8
 *     need at most 47 significant bits) and rounded once to fp32, the
 *     precision the format quantizes in;
 *   - sink positions 0-3 store the fp16 rounding of that fp32 rotated vector;
 *   - every other position is quantized a single time, at its append (no
 *     fp16 window);
 *   - a zero min is stored as +0 (as in the group quantizer of kvq_oracle.c);
 *   - the query is rotated exactly in fp64 here, and attention runs in fp64
 *     over all n positions, including the current one.
 *
 * Layout (restated from its specification; tau = t % 32, lane l = 16 g + i):
 *   k_codes u32 [B][Hkv][C/32][64][2]: word [k][l][u] holds token
 *           32 k + 8 (i/4) + 4 u + i % 4, channels 16 g .. 16 g + 15, channel
 *           16 g + f at bit 2 f (word g of that token's BQ2_0 code bytes).
 *   v_codes u32 [B][Hkv][C/32][64][2]: word [k][l][m] holds channels
 *           16 (2 m + h) + i (h = 0, 1); token 32 k + 8 g + j at bit
 *           8 h + 2 (j / 2) + 16 (j % 2).
 *   k_meta, v_meta u16 [B][Hkv][C][2]: (d, m) of position t.
 *   k_sink u16 [B][Hkv][4][64]: fp16 rotated key of position s < 4.
 *   v_sink u16 [B][Hkv][64][4]: fp16 rotated value, channel-major.
 *   Positions 0-3 of the packed arrays are never written nor read.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

float orc_half_to_float(uint16_t h);
uint16_t orc_float_to_half(float f);

#define BQ2_D 64
#define BQ2_SINKS 4

/* ------------------------------------------------------------------------ */
/* Hadamard rotation                                                         */
/* ------------------------------------------------------------------------ */

/* Entry (r, c) of the normalized Sylvester Hadamard matrix of order 64:
 * (-1)^(number of bits set in r AND c) / 8. */
double orc_bq2_hadamard(int r, int c) {
  int bits = __builtin_popcount((unsigned)(r & c));
  return (bits & 1) ? -0.125 : 0.125;
}

/* y = H x for one 64-vector, as a plain matrix-vector product in fp64. */
static void hadamard64(const double *x, double *y) {
  for (int r = 0; r < BQ2_D; ++r) {
    double s = 0.0;
    for (int c = 0; c < BQ2_D; ++c) s += orc_bq2_hadamard(r, c) * x[c];
    y[r] = s;
  }
}

/* The rotated vector of 64 fp16 values, rounded once to fp32 (exact fp64 sum
 * first: every term is a multiple of 2^-27 below 2^13, so the sum needs fewer
 * than 53 bits). */
void orc_bq2_rotate(const uint16_t *x, float *out) {
  double xd[BQ2_D], yd[BQ2_D];
  for (int c = 0; c < BQ2_D; ++c) xd[c] = orc_half_to_float(x[c]);
  hadamard64(xd, yd);
  for (int c = 0; c < BQ2_D; ++c) out[c] = (float)yd[c];
}

/* ------------------------------------------------------------------------ */
/* Quantizer ([KV1] Quantization Format, in fp32)                            */
/* ------------------------------------------------------------------------ */

static float rne(float y) {
  float fl = floorf(y);
  float frac = y - fl;
  if (frac > 0.5f || (frac == 0.5f && fmodf(fl, 2.0f) != 0.0f)) fl += 1.0f;
  return fl;
}

/* One block: 64 fp32 values -> fp16 bits of d and m, one code per value. */
void orc_bq2_quantize(const float *x, uint16_t *d_out, uint16_t *m_out, uint8_t *codes) {
  float mn = x[0], mx = x[0];
  for (int c = 1; c < BQ2_D; ++c) {
    if (x[c] < mn) mn = x[c];
    if (x[c] > mx) mx = x[c];
  }
  if (mn == 0.0f) mn = 0.0f; /* -0 -> +0 */
  float range = mx - mn;     /* fp32 subtract */
  float d32 = range / 3.0f;  /* fp32 divide */
  const float floor_d = 1e-6f;
  if (!(d32 > floor_d)) d32 = floor_d; /* max(d32, 1e-6) */
  uint16_t d16 = orc_float_to_half(d32);
  uint16_t m16 = orc_float_to_half(mn);
  float d = orc_half_to_float(d16), m = orc_half_to_float(m16);
  for (int c = 0; c < BQ2_D; ++c) {
    float y = (x[c] - m) / d; /* fp32 subtract, fp32 divide */
    float q = rne(y);
    if (q < 0.0f) q = 0.0f;
    if (q > 3.0f) q = 3.0f;
    codes[c] = (uint8_t)q;
  }
  *d_out = d16;
  *m_out = m16;
}

/* The page's 20-byte block: d, m (little-endian fp16), then code bytes with
 * codes 4j .. 4j + 3 in byte j at bits 0, 2, 4, 6. */
void orc_bq2_block(uint16_t d16, uint16_t m16, const uint8_t *codes, uint8_t *block) {
  block[0] = (uint8_t)(d16 & 0xff);
  block[1] = (uint8_t)(d16 >> 8);
  block[2] = (uint8_t)(m16 & 0xff);
  block[3] = (uint8_t)(m16 >> 8);
  for (int j = 0; j < BQ2_D / 4; ++j)
    block[4 + j] = (uint8_t)(codes[4 * j] | (codes[4 * j + 1] << 2) | (codes[4 * j + 2] << 4) |
                             (codes[4 * j + 3] << 6));
}

/* ------------------------------------------------------------------------ */
/* Layout                                                                    */
/* ------------------------------------------------------------------------ */

static int64_t key_word(int64_t unit, int64_t C, int64_t t, int c, int *bit) {
  int64_t k = t / 32;
  int tau = (int)(t % 32);
  int g = c / 16;
  int u = (tau / 4) % 2;
  int i = 4 * (tau / 8) + tau % 4;
  *bit = 2 * (c % 16);
  return ((unit * (C / 32) + k) * 64 + 16 * g + i) * 2 + u;
}

static int64_t value_word(int64_t unit, int64_t C, int64_t t, int c, int *bit) {
  int64_t k = t / 32;
  int tau = (int)(t % 32);
  int g = tau / 8, j = tau % 8;
  int n = c / 16, i = c % 16;
  int m = n / 2, h = n % 2;
  *bit = 8 * h + 2 * (j / 2) + 16 * (j % 2);
  return ((unit * (C / 32) + k) * 64 + 16 * g + i) * 2 + m;
}

static void put2(uint32_t *w, int bit, uint32_t code) {
  *w = (*w & ~(3u << bit)) | ((code & 3u) << bit);
}

/* Stores position t of unit u from its fp16 (unrotated) key and value rows. */
static void store_position(int64_t u, int64_t C, int64_t t, const uint16_t *krow,
                           const uint16_t *vrow, uint32_t *k_codes, uint32_t *v_codes,
                           uint16_t *k_meta, uint16_t *v_meta, uint16_t *k_sink,
                           uint16_t *v_sink) {
  float kx[BQ2_D], vx[BQ2_D];
  orc_bq2_rotate(krow, kx);
  orc_bq2_rotate(vrow, vx);
  if (t < BQ2_SINKS) {
    for (int c = 0; c < BQ2_D; ++c) {
      k_sink[(u * BQ2_SINKS + t) * BQ2_D + c] = orc_float_to_half(kx[c]);
      v_sink[(u * BQ2_D + c) * BQ2_SINKS + t] = orc_float_to_half(vx[c]);
    }
    return;
  }
  uint8_t kc[BQ2_D], vc[BQ2_D];
  uint16_t kd, km, vd, vm;
  orc_bq2_quantize(kx, &kd, &km, kc);
  orc_bq2_quantize(vx, &vd, &vm, vc);
  for (int c = 0; c < BQ2_D; ++c) {
    int bit;
    int64_t w = key_word(u, C, t, c, &bit);
    put2(&k_codes[w], bit, kc[c]);
    w = value_word(u, C, t, c, &bit);
    put2(&v_codes[w], bit, vc[c]);
  }
  k_meta[(u * C + t) * 2] = kd;
  k_meta[(u * C + t) * 2 + 1] = km;
  v_meta[(u * C + t) * 2] = vd;
  v_meta[(u * C + t) * 2 + 1] = vm;
}

/* Positions [0, n) of every unit from fp16 rows k, v [B*Hkv][n][64]. */
void orc_bq2_prefill(int B, int Hkv, int64_t C, const uint16_t *k, const uint16_t *v,
                     int64_t n, uint32_t *k_codes, uint32_t *v_codes, uint16_t *k_meta,
                     uint16_t *v_meta, uint16_t *k_sink, uint16_t *v_sink) {
  int64_t units = (int64_t)B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u)
    for (int64_t t = 0; t < n && t < C; ++t)
      store_position(u, C, t, k + (u * n + t) * BQ2_D, v + (u * n + t) * BQ2_D, k_codes,
                     v_codes, k_meta, v_meta, k_sink, v_sink);
}

/* One token per sequence at position seq_lens[b] (the count held before it);
 * k_new, v_new fp16 [B][Hkv][64]. */
void orc_bq2_append(int B, int Hkv, int64_t C, const uint16_t *k_new, const uint16_t *v_new,
                    const int32_t *seq_lens, uint32_t *k_codes, uint32_t *v_codes,
                    uint16_t *k_meta, uint16_t *v_meta, uint16_t *k_sink, uint16_t *v_sink) {
  int64_t units = (int64_t)B * Hkv;
  for (int64_t u = 0; u < units; ++u) {
    int64_t t = seq_lens[u / Hkv];
    if (t < 0 || t >= C) continue;
    store_position(u, C, t, k_new + u * BQ2_D, v_new + u * BQ2_D, k_codes, v_codes, k_meta,
                   v_meta, k_sink, v_sink);
  }
}

/* Codes and (d, m) of every position in natural order (tests):
 * k_code, v_code u8 [B*Hkv][C][64]. */
void orc_bq2_unpack(int B, int Hkv, int64_t C, const uint32_t *k_codes, const uint32_t *v_codes,
                    uint8_t *k_code, uint8_t *v_code) {
  int64_t units = (int64_t)B * Hkv;
  for (int64_t u = 0; u < units; ++u)
    for (int64_t t = 0; t < C; ++t)
      for (int c = 0; c < BQ2_D; ++c) {
        int bit;
        int64_t w = key_word(u, C, t, c, &bit);
        k_code[(u * C + t) * BQ2_D + c] = (uint8_t)((k_codes[w] >> bit) & 3u);
        w = value_word(u, C, t, c, &bit);
        v_code[(u * C + t) * BQ2_D + c] = (uint8_t)((v_codes[w] >> bit) & 3u);
      }
}

/* Rotated key and value of position t as the cache represents it (fp64). */
static void cached_kv(int64_t u, int64_t C, int64_t t, const uint32_t *k_codes,
                      const uint32_t *v_codes, const uint16_t *k_meta, const uint16_t *v_meta,
                      const uint16_t *k_sink, const uint16_t *v_sink, double *kk, double *vv) {
  if (t < BQ2_SINKS) {
    for (int c = 0; c < BQ2_D; ++c) {
      kk[c] = orc_half_to_float(k_sink[(u * BQ2_SINKS + t) * BQ2_D + c]);
      vv[c] = orc_half_to_float(v_sink[(u * BQ2_D + c) * BQ2_SINKS + t]);
    }
    return;
  }
  double kd = orc_half_to_float(k_meta[(u * C + t) * 2]);
  double km = orc_half_to_float(k_meta[(u * C + t) * 2 + 1]);
  double vd = orc_half_to_float(v_meta[(u * C + t) * 2]);
  double vm = orc_half_to_float(v_meta[(u * C + t) * 2 + 1]);
  for (int c = 0; c < BQ2_D; ++c) {
    int bit;
    int64_t w = key_word(u, C, t, c, &bit);
    kk[c] = (double)((k_codes[w] >> bit) & 3u) * kd + km; /* [KV1] Dequantize */
    w = value_word(u, C, t, c, &bit);
    vv[c] = (double)((v_codes[w] >> bit) & 3u) * vd + vm;
  }
}

/* Rotated keys and values of positions [0, n) of every unit (fp64, tests):
 * out_k, out_v [B*Hkv][n][64]. */
void orc_bq2_cache_kv(int B, int Hkv, int64_t C, const uint32_t *k_codes,
                      const uint32_t *v_codes, const uint16_t *k_meta, const uint16_t *v_meta,
                      const uint16_t *k_sink, const uint16_t *v_sink, int64_t n, double *out_k,
                      double *out_v) {
  int64_t units = (int64_t)B * Hkv;
  for (int64_t u = 0; u < units; ++u)
    for (int64_t t = 0; t < n; ++t)
      cached_kv(u, C, t, k_codes, v_codes, k_meta, v_meta, k_sink, v_sink,
                out_k + (u * n + t) * BQ2_D, out_v + (u * n + t) * BQ2_D);
}

/*
 * For every sequence b and query head h, with n = seq_lens[b] and KV head
 * h / (Hq/Hkv): qH = H q (exact), s_t = sm_scale * qH . k_t over the cached
 * rotated keys, p = softmax(s), o = sum_t p_t v_t over the cached rotated
 * values, out = H o ([KV1] Hadamard rotation), all in fp64.  q fp16
 * [B][Hq][64]; out fp64 [B][Hq][64]; n == 0 gives 0.
 */
void orc_bq2_decode_attn(int B, int Hq, int Hkv, int64_t C, const uint16_t *q,
                         const uint32_t *k_codes, const uint32_t *v_codes,
                         const uint16_t *k_meta, const uint16_t *v_meta,
                         const uint16_t *k_sink, const uint16_t *v_sink,
                         const int32_t *seq_lens, double sm_scale, double *out) {
  int64_t units = (int64_t)B * Hkv;
  int g = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int b = (int)(u / Hkv);
    int hkv = (int)(u % Hkv);
    int64_t n = seq_lens[b];
    if (n > C) n = C;
    int64_t nn = n > 0 ? n : 1;
    double *kk = (double *)malloc((size_t)nn * BQ2_D * sizeof(double));
    double *vv = (double *)malloc((size_t)nn * BQ2_D * sizeof(double));
    double *s = (double *)malloc((size_t)nn * sizeof(double));
    for (int64_t t = 0; t < n; ++t)
      cached_kv(u, C, t, k_codes, v_codes, k_meta, v_meta, k_sink, v_sink, kk + t * BQ2_D,
                vv + t * BQ2_D);
    for (int hh = 0; hh < g; ++hh) {
      int h = hkv * g + hh;
      double *oh = out + ((int64_t)b * Hq + h) * BQ2_D;
      for (int c = 0; c < BQ2_D; ++c) oh[c] = 0.0;
      if (n <= 0) continue;
      double qd[BQ2_D], qr[BQ2_D], o[BQ2_D];
      for (int c = 0; c < BQ2_D; ++c) qd[c] = orc_half_to_float(q[((int64_t)b * Hq + h) * BQ2_D + c]);
      hadamard64(qd, qr);
      double smax = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int c = 0; c < BQ2_D; ++c) dot += qr[c] * kk[t * BQ2_D + c];
        s[t] = sm_scale * dot;
        if (s[t] > smax) smax = s[t];
      }
      double denom = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        s[t] = exp(s[t] - smax);
        denom += s[t];
      }
      for (int c = 0; c < BQ2_D; ++c) o[c] = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        double p = s[t] / denom;
        for (int c = 0; c < BQ2_D; ++c) o[c] += p * vv[t * BQ2_D + c];
      }
      hadamard64(o, oh);
    }
    free(kk);
    free(vv);
    free(s);
  }
}
