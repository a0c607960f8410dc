/*
 * kvq_oracle.c — plain, slow CPU oracle for KIVI-style quantized KV caches and
 * single-token decode attention over them.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library: the packed layout is restated
 * here from its written specification, and fp16 conversion is done in software.
 *
 * Sources (web pages, cited by title and section):
 *   [KIVI] "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 *          (repository digest): core capabilities (keys per channel, values per
 *          token, fp16 residual window, 2/4 bits, group size), Overview,
 *          Example (k_bits, v_bits, group_size, residual_length).
 *   [KV1]  "KV1-1.2B-Instruct" model card: "Quantization Format: KV1.cpp BQ2_0"
 *          (quantize in fp32, scale = (max-min)/(2^b-1), fp16-rounded scale and
 *          min used for the codes, round half to even, clamp, dequantize as
 *          code*scale+min, code order inside a byte), "Quickstart" (attending
 *          over the once-quantized cache gives the exact low-bit result).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - the code divides by the stored fp16 scale (KV1 states the fp16-rounded
 *     scale and min are the ones used for the codes);
 *   - a zero fp16 scale gives code 0 for every element (KV1's 1e-6 floor belongs
 *     to its own format and is not applied);
 *   - zero min / max are taken as +0 so that stored bits do not depend on order;
 *   - lazy flush: a full residual window is quantized when the next token
 *     arrives, so 1..R residual tokens are present at attention time;
 *   - query head h uses KV head h / (Hq/Hkv);
 *   - attention covers all n tokens, including the current one, no mask.
 *
 * Floating point: the quantizer runs in IEEE fp32 (the precision KV1 fixes for
 * quantizing); dequantization and attention run in fp64.  Build with
 * -O2 -fno-fast-math -ffp-contract=off so that gcc neither contracts nor
 * reorders the fp32 steps.  OpenMP splits independent (sequence, KV head)
 * units across threads; every unit's arithmetic is serial and deterministic.
 *
 * Parity pins (tests): exhaustive fp32->fp16 rounding against numpy; worked
 * examples derived by hand; brute-force nearest-grid-point code selection in
 * exact rational arithmetic; reconstruction bound; constant groups; KV1 BQ2_0
 * byte order; byte accounting against the KV1 memory table; attention against
 * torch float64 scaled_dot_product_attention and a naive loop; closed forms
 * (q = 0, n = 1, identical rows, all-residual); incremental flushes equal to a
 * bulk quantization.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif


/* ------------------------------------------------------------------------ */
/* fp16 <-> fp32 in software                                                 */
/* ------------------------------------------------------------------------ */

/* Widens IEEE binary16 bits to a float (exact). */
float orc_half_to_float(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int mant = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)mant, -24); /* subnormal: mant * 2^-24 */
  } else if (expo == 31) {
    v = mant ? NAN : INFINITY;
  } else {
    v = ldexp((double)(mant + 1024), expo - 25); /* (1.mant) * 2^(expo-15) */
  }
  return (float)(sign ? -v : v);
}

/* Rounds a float to the nearest binary16, ties to even; returns the bits. */
uint16_t orc_float_to_half(float f) {
  uint32_t fbits;
  memcpy(&fbits, &f, sizeof fbits);
  uint16_t sign = (uint16_t)((fbits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  /* 65504 is the largest finite half; its successor would be 65536, and the
   * midpoint 65520 rounds to the even one (65536), i.e. overflows. */
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);

  int e2; /* a = fr * 2^e2, 0.5 <= fr < 1, so 2^(e2-1) <= a < 2^e2 */
  (void)frexp(a, &e2);
  int e = e2 - 1; /* unbiased exponent of a */
  double quantum = (e < -14) ? ldexp(1.0, -24) : ldexp(1.0, e - 10);

  double n = a / quantum; /* exact: quantum is a power of two */
  double fl = floor(n);
  double frac = n - fl;
  if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  /* fl * quantum is the rounded magnitude */
  if (e < -14) {
    /* subnormal range; fl == 1024 is the smallest normal, whose bits are 0x400 */
    return (uint16_t)(sign | (uint16_t)fl);
  }
  long m = (long)fl; /* in [1024, 2048] */
  int expo = e + 15;
  if (m == 2048) {
    m = 1024;
    expo += 1;
  }
  if (expo >= 31) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)(expo << 10) | (uint16_t)(m - 1024));
}

/* Vector helpers for the tests. */
void orc_float_to_half_array(const float *x, uint16_t *y, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) y[i] = orc_float_to_half(x[i]);
}
void orc_half_to_float_array(const uint16_t *x, float *y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_half_to_float(x[i]);
}

/* ------------------------------------------------------------------------ */
/* The group quantizer                                                      */
/* ------------------------------------------------------------------------ */

/* Round half to even of a non-negative-or-any float, written out. */
static float round_half_even(float y) {
  float fl = floorf(y);
  float frac = y - fl; /* exact for |y| < 2^23 */
  if (frac > 0.5f || (frac == 0.5f && fmodf(fl, 2.0f) != 0.0f)) fl += 1.0f;
  return fl;
}

/*
 * Quantizes n fp16 values x[0], x[stride], ... with b bits.
 * Writes the fp16 bits of (scale, min) and one code per element
 * (codes[i*code_stride]).  [KV1] Quantization Format, in fp32:
 *   scale = fp16((max - min) / (2^b - 1)), min = fp16(min),
 *   code = clamp(round_half_even((x - min) / scale), 0, 2^b - 1)
 * with the fp16-rounded scale and min used for the codes; a zero scale gives
 * code 0.
 */
void orc_quantize_group(const uint16_t *x, int64_t n, int64_t stride, int bits,
                        uint16_t *scale_out, uint16_t *min_out, uint8_t *codes,
                        int64_t code_stride) {
  float mn = orc_half_to_float(x[0]);
  float mx = mn;
  for (int64_t i = 1; i < n; ++i) {
    float v = orc_half_to_float(x[i * stride]);
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  if (mn == 0.0f) mn = 0.0f; /* -0 -> +0 */
  if (mx == 0.0f) mx = 0.0f;

  const float levels = (float)((1 << bits) - 1);
  float range = mx - mn;     /* fp32 subtract */
  float d32 = range / levels; /* fp32 divide */
  uint16_t d16 = orc_float_to_half(d32);
  if ((d16 & 0x7fffu) == 0) d16 = 0; /* zero scale stored as +0 */
  uint16_t m16 = orc_float_to_half(mn);

  float scale = orc_half_to_float(d16);
  float minv = orc_half_to_float(m16);
  for (int64_t i = 0; i < n; ++i) {
    float code = 0.0f;
    if (scale != 0.0f) {
      float v = orc_half_to_float(x[i * stride]);
      float y = (v - minv) / scale; /* fp32 subtract, fp32 divide */
      code = round_half_even(y);
      if (code < 0.0f) code = 0.0f;
      if (code > levels) code = levels;
    }
    codes[i * code_stride] = (uint8_t)code;
  }
  *scale_out = d16;
  *min_out = m16;
}

/* ------------------------------------------------------------------------ */
/* Packed layout, version 3 (restated from its specification)               */
/*                                                                           */
/* Packed tokens live in blocks of 32 positions; tau = t % 32.  Inside a     */
/* block, words follow a 64-lane consumer order, lane l = 16 g + i.          */
/*   key row i of half u holds    tau = 8 (i/4) + 4 u + i % 4                */
/*   value element j of group g:  tau = 8 g + j                              */
/* k_codes  u32 [B][Hkv][C/32][64][2][KW], KW = D*bK/128: [k][l][u][w] is    */
/*          slice g (channels g*D/4 ..) of key row i of half u; its word w   */
/*          holds channels g*D/4 + w*32/bK + f in bits f*bK (2, 4 bits);     */
/*          8 bits: word 2kc + s holds g*D/4 + 8kc + 2s + (0,1,4,5)[f] in    */
/*          byte f.                                                          */
/* k_meta   u16 [B][Hkv][C/G][D/8][8][2]: entry [q][r][e] is the channel     */
/*          key_meta_channel(r, e) of key group q.                           */
/* v_codes  u32 [B][Hkv][C/32][64][NW], NW = D*bV/64: 4 bits: word n of lane */
/*          l is channel 16n + i, token 8g + j at bit 4(j/2) + 16(j%2);      */
/*          2 bits: word m of lane l holds channels 16(2m+h) + i, token      */
/*          8g + j at bit 8h + 2(j/2) + 16(j%2).  8 bits: words 2n, 2n+1 of  */
/*          lane l are channel 16n + i, token 8g + j in word 2n + j/4 at bit */
/*          8((j%4)/2) + 16(j%2).                                            */
/* v_meta   u16 [B][Hkv][C/32][4][D/G][8][2]: entry [k][g][gamma][j] is      */
/*          token 32k + 8g + j, channel group gamma.                         */
/* k_res    u16 [B][Hkv][Rk][D]: position p in slot p % Rk, one row per     */
/*          slot (Rk: the key window).                                      */
/* v_res    u16 [B][Hkv][Rv/32][D/16][64][8]: entry [k][n][16g + i][j] is    */
/*          slot 32k + 8g + j, channel 16n + i; position p in slot p % Rv   */
/*          (Rv: the value window).                                         */
/* ------------------------------------------------------------------------ */

static void put_field(uint32_t *word, int bit, int bits, uint32_t code) {
  uint32_t mask = ((1u << bits) - 1u) << bit;
  *word = (*word & ~mask) | ((code << bit) & mask);
}

static uint32_t get_field(uint32_t word, int bit, int bits) {
  return (word >> bit) & ((1u << bits) - 1u);
}

/* Index into k_codes of the word holding token t, channel c of a unit, and
 * the bit at which its code starts. */
static int64_t key_word(int64_t unit, int64_t C, int D, int bK, int64_t t,
                        int c, int *bit) {
  int64_t k = t / 32;
  int tau = (int)(t % 32);
  int slice = D / 4; /* channels of a lane group's slice */
  int g = c / slice, cs = c % slice;
  int kw = D * bK / 128; /* words per slice */
  int w, byte;
  if (bK == 8) {
    /* within the 8 channels 8kc .. 8kc+7: p = 2s + (0,1,4,5)[f] */
    int kc = cs / 8, p = cs % 8;
    int s = (p % 4) / 2;
    int f = (p % 2) + 2 * (p / 4);
    w = 2 * kc + s;
    byte = f;
    *bit = 8 * byte;
  } else {
    w = cs * bK / 32;
    *bit = cs * bK % 32;
  }
  /* the key row i of half u that holds tau = 8 (i/4) + 4 u + i % 4 */
  int u = (tau / 4) % 2;
  int i = 4 * (tau / 8) + tau % 4;
  int l = 16 * g + i;
  return (unit * (C / 32) + k) * (int64_t)D * bK + ((int64_t)l * 2 + u) * kw + w;
}

/* Channel of key-meta entry e (0..7) of k-chunk r (0..D/8-1). */
static int key_meta_channel(int D, int bK, int r, int e) {
  int kcs = D / 32; /* k-chunks per slice */
  int g = r / kcs, kc = r % kcs;
  int base, off;
  if (bK == 2) {
    base = 16 * (kc / 2) + 4 * (kc % 2);
    off = 8;
  } else {
    base = 8 * kc;
    off = 4;
  }
  return g * (D / 4) + base + e / 2 + off * (e % 2);
}

/* entry_of[c] = position (r*8 + e) of channel c inside a key group's meta. */
static void key_meta_entries(int D, int bK, int *entry_of) {
  for (int r = 0; r < D / 8; ++r)
    for (int e = 0; e < 8; ++e) entry_of[key_meta_channel(D, bK, r, e)] = r * 8 + e;
}

static uint32_t key_code(const uint32_t *k_codes, int64_t unit, int64_t C,
                         int D, int bK, int64_t t, int c) {
  int bit;
  int64_t w = key_word(unit, C, D, bK, t, c, &bit);
  return get_field(k_codes[w], bit, bK);
}

/* Index into v_codes of the word holding token t, channel c, and its bit. */
static int64_t value_word(int64_t unit, int64_t C, int D, int bV, int64_t t,
                          int c, int *bit) {
  int64_t k = t / 32;
  int tau = (int)(t % 32);
  int g = tau / 8, j = tau % 8;
  int i = c % 16, n = c / 16;
  int l = 16 * g + i;
  int nw = D * bV / 64; /* words per lane */
  int w;
  if (bV == 8) {
    w = 2 * n + j / 4;
    *bit = 8 * ((j % 4) / 2) + 16 * (j % 2);
  } else if (bV == 4) {
    w = n;
    *bit = 4 * (j / 2) + 16 * (j % 2);
  } else {
    w = n / 2;
    *bit = 8 * (n % 2) + 2 * (j / 2) + 16 * (j % 2);
  }
  return (unit * (C / 32) + k) * (int64_t)D * bV + (int64_t)l * nw + w;
}

static uint32_t value_code(const uint32_t *v_codes, int64_t unit, int64_t C,
                           int D, int bV, int64_t t, int c) {
  int bit;
  int64_t w = value_word(unit, C, D, bV, t, c, &bit);
  return get_field(v_codes[w], bit, bV);
}

/* Entry of (scale, min) for token t, channel group gm in v_meta. */
static int64_t value_meta_index(int64_t unit, int64_t C, int D, int G,
                                int64_t t, int gm) {
  int64_t k = t / 32;
  int tau = (int)(t % 32);
  return ((unit * (C / 32) + k) * 4 + tau / 8) * (D / G) * 8 + gm * 8 + tau % 8;
}

/* Index inside one unit's v_res of slot s, channel c. */
static int64_t value_res_index(int D, int s, int c) {
  int k = s / 32, tau = s % 32;
  int g = tau / 8, j = tau % 8;
  int n = c / 16, i = c % 16;
  return (((int64_t)k * (D / 16) + n) * 64 + 16 * g + i) * 8 + j;
}

/* Quantizes key groups of one unit from a source of token rows src[t*D + c]
 * (fp16) whose first row is position pos0; n_tok tokens, multiples of G. */
static void quantize_keys_unit(const uint16_t *src, int64_t pos0, int64_t n_tok,
                               int D, int bK, int G, int64_t C, int64_t unit,
                               uint32_t *k_codes, uint16_t *k_meta) {
  uint8_t *codes = (uint8_t *)malloc((size_t)G);
  int entry_of[128];
  key_meta_entries(D, bK, entry_of);
  for (int64_t j0 = 0; j0 < n_tok; j0 += G) {
    int64_t j = (pos0 + j0) / G; /* key group index */
    for (int c = 0; c < D; ++c) {
      uint16_t d16, m16;
      /* per channel: the G tokens of the group ([KIVI] keys per channel) */
      orc_quantize_group(src + j0 * D + c, G, D, bK, &d16, &m16, codes, 1);
      uint16_t *meta = k_meta + ((unit * (C / G) + j) * D + entry_of[c]) * 2;
      meta[0] = d16;
      meta[1] = m16;
      for (int i = 0; i < G; ++i) {
        int bit;
        int64_t w = key_word(unit, C, D, bK, pos0 + j0 + i, c, &bit);
        put_field(&k_codes[w], bit, bK, codes[i]);
      }
    }
  }
  free(codes);
}

/* Quantizes value tokens of one unit; src[t*D + c] fp16, position pos0 first. */
static void quantize_values_unit(const uint16_t *src, int64_t pos0,
                                 int64_t n_tok, int D, int bV, int G, int64_t C,
                                 int64_t unit, uint32_t *v_codes,
                                 uint16_t *v_meta) {
  uint8_t *codes = (uint8_t *)malloc((size_t)G);
  int ngroups = D / G;
  for (int64_t i = 0; i < n_tok; ++i) {
    int64_t t = pos0 + i;
    for (int gm = 0; gm < ngroups; ++gm) {
      uint16_t d16, m16;
      /* per token: G consecutive channels ([KIVI] values per token) */
      orc_quantize_group(src + i * D + (int64_t)gm * G, G, 1, bV, &d16, &m16,
                         codes, 1);
      uint16_t *meta = v_meta + value_meta_index(unit, C, D, G, t, gm) * 2;
      meta[0] = d16;
      meta[1] = m16;
      for (int cc = 0; cc < G; ++cc) {
        int bit;
        int64_t w = value_word(unit, C, D, bV, t, gm * G + cc, &bit);
        put_field(&v_codes[w], bit, bV, codes[cc]);
      }
    }
  }
  free(codes);
}

/* Bulk per-channel key quantization of positions [pos0, pos0+n_tok) of every
 * unit; k is fp16 [B*Hkv][n_tok][D]. */
void orc_quantize_keys(int B, int Hkv, int D, int bK, int G, int64_t C,
                       const uint16_t *k, int64_t pos0, int64_t n_tok,
                       uint32_t *k_codes, uint16_t *k_meta) {
  int64_t units = (int64_t)B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u)
    quantize_keys_unit(k + u * n_tok * D, pos0, n_tok, D, bK, G, C, u, k_codes,
                       k_meta);
}

/* Bulk per-token value quantization; v is fp16 [B*Hkv][n_tok][D]. */
void orc_quantize_values(int B, int Hkv, int D, int bV, int G, int64_t C,
                         const uint16_t *v, int64_t pos0, int64_t n_tok,
                         uint32_t *v_codes, uint16_t *v_meta) {
  int64_t units = (int64_t)B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u)
    quantize_values_unit(v + u * n_tok * D, pos0, n_tok, D, bV, G, C, u,
                         v_codes, v_meta);
}

/* ------------------------------------------------------------------------ */
/* Residual window and lazy flush                                            */
/* ------------------------------------------------------------------------ */

/* Number of packed tokens of a sequence holding n tokens (lazy flush): the
 * residual keeps ((n-1) % R) + 1 tokens when n >= 1. */
int64_t orc_packed_len(int64_t n, int R) {
  if (n <= 0) return 0;
  return n - (((n - 1) % R) + 1);
}

/* Appends one token per sequence.  seq_lens[b] = tokens held BEFORE the new
 * one.  Keys and values each have their own window (Rk, Rv positions; [KVQ]
 * Usage: a residual length per tensor).  If that count n is positive and a
 * multiple of Rk, key positions [n-Rk, n) are quantized from the key window
 * first, and likewise for values with Rv; then the new token goes to key slot
 * n % Rk and value slot n % Rv.  ([KIVI] core capabilities: recent tokens
 * kept in fp16.)  k_new, v_new fp16 [B][Hkv][D]. */
void orc_append(int B, int Hkv, int D, int bK, int bV, int G, int Rk, int Rv, int64_t C,
                const uint16_t *k_new, const uint16_t *v_new,
                const int32_t *seq_lens, uint32_t *k_codes, uint32_t *v_codes,
                uint16_t *k_meta, uint16_t *v_meta, uint16_t *k_res,
                uint16_t *v_res) {
  int64_t units = (int64_t)B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int b = (int)(u / Hkv);
    int64_t n = seq_lens[b];
    if (n < 0 || n >= C) continue;
    uint16_t *kr = k_res + u * Rk * D;
    uint16_t *vr = v_res + u * Rv * D;
    if (n > 0 && n % Rk == 0) /* key slots 0..Rk-1 hold positions n-Rk .. n-1 */
      quantize_keys_unit(kr, n - Rk, Rk, D, bK, G, C, u, k_codes, k_meta);
    if (n > 0 && n % Rv == 0) {
      uint16_t *rows = (uint16_t *)malloc((size_t)Rv * D * sizeof(uint16_t));
      for (int s = 0; s < Rv; ++s)
        for (int c = 0; c < D; ++c) rows[s * D + c] = vr[value_res_index(D, s, c)];
      quantize_values_unit(rows, n - Rv, Rv, D, bV, G, C, u, v_codes, v_meta);
      free(rows);
    }
    memcpy(kr + (n % Rk) * D, k_new + u * D, (size_t)D * sizeof(uint16_t));
    for (int c = 0; c < D; ++c) vr[value_res_index(D, (int)(n % Rv), c)] = v_new[u * D + c];
  }
}

/* ------------------------------------------------------------------------ */
/* Dequantization (fp64, exact)                                              */
/* ------------------------------------------------------------------------ */

/* Dequantized key of token t < packed length: code * scale + min ([KV1]
 * Dequantize).  The product of a code below 256 and an fp16 scale, plus an
 * fp16 min, is exact in fp64. */
static double dequant_key(const uint32_t *k_codes, const uint16_t *k_meta,
                          const int *entry_of, int64_t unit, int64_t C, int D,
                          int bK, int G, int64_t t, int c) {
  const uint16_t *meta = k_meta + ((unit * (C / G) + t / G) * D + entry_of[c]) * 2;
  double scale = orc_half_to_float(meta[0]);
  double minv = orc_half_to_float(meta[1]);
  return (double)key_code(k_codes, unit, C, D, bK, t, c) * scale + minv;
}

static double dequant_value(const uint32_t *v_codes, const uint16_t *v_meta,
                            int64_t unit, int64_t C, int D, int bV, int G,
                            int64_t t, int c) {
  const uint16_t *meta = v_meta + value_meta_index(unit, C, D, G, t, c / G) * 2;
  double scale = orc_half_to_float(meta[0]);
  double minv = orc_half_to_float(meta[1]);
  return (double)value_code(v_codes, unit, C, D, bV, t, c) * scale + minv;
}

/* Keys and values of positions t < n of unit u as the cache represents them:
 * a key is dequantized below the key packed length Lq(n, Rk) and the key
 * window's fp16 above it; a value likewise with Rv.  kk, vv fp64 [n][D]. */
static void unit_kv(int D, int bK, int bV, int G, int Rk, int Rv, int64_t C,
                    const int *entry_of, const uint32_t *k_codes, const uint32_t *v_codes,
                    const uint16_t *k_meta, const uint16_t *v_meta, const uint16_t *k_res,
                    const uint16_t *v_res, int64_t u, int64_t n, double *kk, double *vv) {
  int64_t lqk = orc_packed_len(n, Rk), lqv = orc_packed_len(n, Rv);
  for (int64_t t = 0; t < n; ++t)
    for (int c = 0; c < D; ++c) {
      kk[t * D + c] = t < lqk
                          ? dequant_key(k_codes, k_meta, entry_of, u, C, D, bK, G, t, c)
                          : orc_half_to_float(k_res[(u * Rk + t % Rk) * D + c]);
      vv[t * D + c] =
          t < lqv ? dequant_value(v_codes, v_meta, u, C, D, bV, G, t, c)
                  : orc_half_to_float(v_res[u * Rv * D + value_res_index(D, (int)(t % Rv), c)]);
    }
}

/* Full-precision key/value of every position t < n of every unit as the cache
 * represents it (unit_kv).  out_k, out_v: fp64 [B*Hkv][n][D]. */
void orc_cache_kv(int B, int Hkv, int D, int bK, int bV, int G, int Rk, int Rv,
                  int64_t C, const uint32_t *k_codes, const uint32_t *v_codes,
                  const uint16_t *k_meta, const uint16_t *v_meta,
                  const uint16_t *k_res, const uint16_t *v_res, int64_t n,
                  double *out_k, double *out_v) {
  int64_t units = (int64_t)B * Hkv;
  int entry_of[128];
  key_meta_entries(D, bK, entry_of);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u)
    unit_kv(D, bK, bV, G, Rk, Rv, C, entry_of, k_codes, v_codes, k_meta, v_meta, k_res, v_res,
            u, n, out_k + u * n * D, out_v + u * n * D);
}

/* ------------------------------------------------------------------------ */
/* Decode attention (fp64)                                                   */
/* ------------------------------------------------------------------------ */

/*
 * For every sequence b and query head h: with n = seq_lens[b] (tokens including
 * the current one) and KV head h / (Hq/Hkv),
 *   s_t = sm_scale * sum_c q[c] * k_t[c],  p = softmax(s),  out = sum_t p_t v_t
 * over all n tokens (dequantized for t < packed length, fp16 residual for the
 * rest), in fp64.  q fp16 [B][Hq][D]; out fp64 [B][Hq][D].  n == 0 gives 0.
 */
void orc_decode_attn(int B, int Hq, int Hkv, int D, int bK, int bV, int G,
                     int Rk, int Rv, int64_t C, const uint16_t *q,
                     const uint32_t *k_codes, const uint32_t *v_codes,
                     const uint16_t *k_meta, const uint16_t *v_meta,
                     const uint16_t *k_res, const uint16_t *v_res,
                     const int32_t *seq_lens, double sm_scale, double *out) {
  int64_t units = (int64_t)B * Hkv;
  int g = Hq / Hkv;
  int entry_of[128];
  key_meta_entries(D, bK, entry_of);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int b = (int)(u / Hkv);
    int hkv = (int)(u % Hkv);
    int64_t n = seq_lens[b];
    if (n > C) n = C;
    /* this unit's keys and values, as the cache represents them */
    double *kk = (double *)malloc((size_t)(n > 0 ? n : 1) * D * sizeof(double));
    double *vv = (double *)malloc((size_t)(n > 0 ? n : 1) * D * sizeof(double));
    double *s = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    unit_kv(D, bK, bV, G, Rk, Rv, C, entry_of, k_codes, v_codes, k_meta, v_meta, k_res, v_res,
            u, n, kk, vv);
    for (int hh = 0; hh < g; ++hh) {
      int h = hkv * g + hh;
      const uint16_t *qh = q + ((int64_t)b * Hq + h) * D;
      double *oh = out + ((int64_t)b * Hq + h) * D;
      for (int c = 0; c < D; ++c) oh[c] = 0.0;
      if (n <= 0) continue;
      double smax = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int c = 0; c < D; ++c)
          dot += (double)orc_half_to_float(qh[c]) * kk[t * D + c];
        s[t] = sm_scale * dot;
        if (s[t] > smax) smax = s[t];
      }
      double denom = 0.0;
      for (int64_t t = 0; t < n; ++t) {
        s[t] = exp(s[t] - smax);
        denom += s[t];
      }
      for (int64_t t = 0; t < n; ++t) {
        double p = s[t] / denom;
        for (int c = 0; c < D; ++c) oh[c] += p * vv[t * D + c];
      }
    }
    free(kk);
    free(vv);
    free(s);
  }
}

/*
 * Attention of the last T positions of each sequence at once ([KIVI] core
 * capabilities: prefill alongside the quantized cache; the plainest reading is
 * causal attention of T new tokens).  With n = seq_lens[b] (the T tokens
 * included), query token i (0 <= i < T) sits at position n - T + i and
 * attends to positions [0, n - T + i] of the cache at length n: dequantized
 * below the packed length Lq(n), the fp16 window above, in fp64.
 * q fp16 [B][T][Hq][D]; out fp64 [B][T][Hq][D]; a token that sees no position
 * gets 0.
 */
void orc_decode_attn_multi(int B, int Hq, int Hkv, int D, int bK, int bV, int G,
                           int Rk, int Rv, int64_t C, int T, const uint16_t *q,
                           const uint32_t *k_codes, const uint32_t *v_codes,
                           const uint16_t *k_meta, const uint16_t *v_meta,
                           const uint16_t *k_res, const uint16_t *v_res,
                           const int32_t *seq_lens, double sm_scale, double *out) {
  int64_t units = (int64_t)B * Hkv;
  int g = Hq / Hkv;
  int entry_of[128];
  key_meta_entries(D, bK, entry_of);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int b = (int)(u / Hkv);
    int hkv = (int)(u % Hkv);
    int64_t n = seq_lens[b];
    if (n > C) n = C;
    int64_t nn = n > 0 ? n : 1;
    double *kk = (double *)malloc((size_t)nn * D * sizeof(double));
    double *vv = (double *)malloc((size_t)nn * D * sizeof(double));
    double *s = (double *)malloc((size_t)nn * sizeof(double));
    unit_kv(D, bK, bV, G, Rk, Rv, C, entry_of, k_codes, v_codes, k_meta, v_meta, k_res, v_res,
            u, n, kk, vv);
    for (int i = 0; i < T; ++i) {
      int64_t vis = n - T + i + 1; /* positions this token sees */
      for (int hh = 0; hh < g; ++hh) {
        int h = hkv * g + hh;
        const uint16_t *qh = q + (((int64_t)b * T + i) * Hq + h) * D;
        double *oh = out + (((int64_t)b * T + i) * Hq + h) * D;
        for (int c = 0; c < D; ++c) oh[c] = 0.0;
        if (vis <= 0) continue;
        double smax = -INFINITY;
        for (int64_t t = 0; t < vis; ++t) {
          double dot = 0.0;
          for (int c = 0; c < D; ++c) dot += (double)orc_half_to_float(qh[c]) * kk[t * D + c];
          s[t] = sm_scale * dot;
          if (s[t] > smax) smax = s[t];
        }
        double denom = 0.0;
        for (int64_t t = 0; t < vis; ++t) {
          s[t] = exp(s[t] - smax);
          denom += s[t];
        }
        for (int64_t t = 0; t < vis; ++t) {
          double p = s[t] / denom;
          for (int c = 0; c < D; ++c) oh[c] += p * vv[t * D + c];
        }
      }
    }
    free(kk);
    free(vv);
    free(s);
  }
}

/* Writes positions [pos0, pos0 + n_tok) of fp16 key rows k [B*Hkv][n_tok][D]
 * into their key-window slots p % Rk. */
void orc_key_residual_store(int B, int Hkv, int D, int Rk, const uint16_t *k, int64_t pos0,
                            int64_t n_tok, uint16_t *k_res) {
  int64_t units = (int64_t)B * Hkv;
  for (int64_t u = 0; u < units; ++u)
    for (int64_t t = 0; t < n_tok; ++t) {
      int slot = (int)((pos0 + t) % Rk);
      for (int c = 0; c < D; ++c) k_res[(u * Rk + slot) * D + c] = k[(u * n_tok + t) * D + c];
    }
}

/* Likewise for value rows v into the value window (slots p % Rv, layout
 * above). */
void orc_value_residual_store(int B, int Hkv, int D, int Rv, const uint16_t *v, int64_t pos0,
                              int64_t n_tok, uint16_t *v_res) {
  int64_t units = (int64_t)B * Hkv;
  for (int64_t u = 0; u < units; ++u)
    for (int64_t t = 0; t < n_tok; ++t) {
      int slot = (int)((pos0 + t) % Rv);
      for (int c = 0; c < D; ++c)
        v_res[u * Rv * D + value_res_index(D, slot, c)] = v[(u * n_tok + t) * D + c];
    }
}

/* The residual window in natural order, for tests: out [B*Hkv][R][D]. */
void orc_value_res_rows(int B, int Hkv, int D, int R, const uint16_t *v_res,
                        uint16_t *out) {
  int64_t units = (int64_t)B * Hkv;
  for (int64_t u = 0; u < units; ++u)
    for (int s = 0; s < R; ++s)
      for (int c = 0; c < D; ++c)
        out[(u * R + s) * D + c] = v_res[u * R * D + value_res_index(D, s, c)];
}

/* The cache's codes and (scale, min) pairs in natural order, for tests:
 * k_code, v_code u8 [B*Hkv][C][D]; k_sm u16 [B*Hkv][C/G][D][2];
 * v_sm u16 [B*Hkv][C][D/G][2]. */
void orc_unpack(int B, int Hkv, int D, int bK, int bV, int G, int64_t C,
                const uint32_t *k_codes, const uint32_t *v_codes,
                const uint16_t *k_meta, const uint16_t *v_meta, uint8_t *k_code,
                uint8_t *v_code, uint16_t *k_sm, uint16_t *v_sm) {
  int64_t units = (int64_t)B * Hkv;
  int entry_of[128];
  key_meta_entries(D, bK, entry_of);
  for (int64_t u = 0; u < units; ++u) {
    for (int64_t t = 0; t < C; ++t)
      for (int c = 0; c < D; ++c) {
        k_code[(u * C + t) * D + c] = (uint8_t)key_code(k_codes, u, C, D, bK, t, c);
        v_code[(u * C + t) * D + c] = (uint8_t)value_code(v_codes, u, C, D, bV, t, c);
      }
    for (int64_t q = 0; q < C / G; ++q)
      for (int c = 0; c < D; ++c)
        for (int x = 0; x < 2; ++x)
          k_sm[((u * (C / G) + q) * D + c) * 2 + x] =
              k_meta[((u * (C / G) + q) * D + entry_of[c]) * 2 + x];
    for (int64_t t = 0; t < C; ++t)
      for (int gm = 0; gm < D / G; ++gm)
        for (int x = 0; x < 2; ++x)
          v_sm[((u * C + t) * (D / G) + gm) * 2 + x] =
              v_meta[value_meta_index(u, C, D, G, t, gm) * 2 + x];
  }
}

/* Threads the OpenMP runtime will use for the parallel loops above. */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
