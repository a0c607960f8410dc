// Drives the host code of libkvq (kvq_api.cpp, built with the launchers of
// host_stubs.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer: every
// entry point's argument checks on a sweep of valid and invalid geometries,
// the error text, the HIP-failure path (no device is present where this runs,
// or the stub launchers fail), and the per-thread error text from several
// threads at once.  Any sanitizer report aborts; a broken expectation exits 1.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>
#include <thread>
#include <vector>

#include "kvq.h"
#include "kvq_bq2.h"
#include "kvq_paged.h"
#include "kvq_probe.h"

static int failures = 0;
#define EXPECT(c)                                                      \
  do {                                                                 \
    if (!(c)) {                                                        \
      fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #c); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)(z ^ (z >> 31));
}
static const int32_t kVals[] = {-2147483647 - 1, -65, -1, 0, 1, 2, 3, 4, 8, 16, 32, 48, 64,
                                96, 128, 256, 4096, 65536, 1 << 24, 2147483647};
static int32_t pick() { return kVals[rnd() % (sizeof(kVals) / sizeof(kVals[0]))]; }

alignas(16) static uint32_t w32[4096];
alignas(16) static uint16_t w16[4096];
alignas(16) static int32_t lens[64];

static kvq_geom small_geom() {
  kvq_geom g;
  g.batch = 2; g.n_q_heads = 8; g.n_kv_heads = 2; g.head_dim = 128; g.k_bits = 2;
  g.v_bits = 4; g.group = 32; g.residual = 128; g.capacity = 256; g.residual_v = 0;
  return g;
}

int main() {
  EXPECT(kvq_abi_version() == KVQ_ABI_VERSION);
  EXPECT(kvq_layout_version() == KVQ_LAYOUT_VERSION);
  for (int s = -20; s <= 5; ++s) EXPECT(kvq_status_str(s) != NULL);
  EXPECT(kvq_validate_geom(NULL) == KVQ_ERR_NULL);
  EXPECT(strlen(kvq_last_error()) > 0);

  // geometry sweep: every field from a list of ordinary and extreme values
  size_t bytes[6];
  int valid = 0;
  for (int i = 0; i < 200000; ++i) {
    kvq_geom g;
    g.batch = pick(); g.n_q_heads = pick(); g.n_kv_heads = pick(); g.head_dim = pick();
    g.k_bits = pick(); g.v_bits = pick(); g.group = pick(); g.residual = pick();
    g.capacity = pick(); g.residual_v = (rnd() & 1) ? 0 : pick();
    const int st = kvq_validate_geom(&g);
    EXPECT(st == KVQ_OK || st == KVQ_ERR_GEOM || st == KVQ_ERR_BITS);
    EXPECT(kvq_cache_bytes(&g, bytes) == st);
    if (st == KVQ_OK) {
      ++valid;
      for (int b = 0; b < 6; ++b) EXPECT(bytes[b] > 0);
      size_t pb[6];
      const int P = 1 << (5 + rnd() % 4), np = pick();
      const int ps = kvq_paged_cache_bytes(&g, P, np, pb);
      EXPECT(ps == KVQ_OK || ps == KVQ_ERR_GEOM || ps == KVQ_ERR_RANGE);
      kvq_paged_cache pc;
      memset(&pc, 0, sizeof pc);
      pc.page_size = pick(); pc.max_pages = pick(); pc.num_pages = pick();
      const int vs = kvq_paged_validate(&g, &pc);
      EXPECT(vs != KVQ_OK || pc.page_size > 0);
    } else {
      EXPECT(strlen(kvq_last_error()) > 0);
    }
  }
  // valid geometries, each also with one field replaced by an extreme value
  static const int kBits[] = {2, 4, 8};
  for (int D = 64; D <= 128; D *= 2)
    for (int bk : kBits)
      for (int bv : kBits)
        for (int G = 32; G <= D; G *= 2)
          for (int gq = 1; gq <= 16; gq *= 2)
            for (int rm = 1; rm <= 4; rm *= 2) {
              kvq_geom g0;
              g0.batch = 3; g0.n_kv_heads = 2; g0.n_q_heads = 2 * gq; g0.head_dim = D;
              g0.k_bits = bk; g0.v_bits = bv; g0.group = G; g0.residual = G * rm;
              g0.capacity = G * rm * 5; g0.residual_v = (rm & 2) ? G : 0;
              if (g0.residual_v && g0.capacity % g0.residual_v) g0.residual_v = 0;
              const int st = kvq_validate_geom(&g0);
              EXPECT(st == KVQ_OK);
              if (st != KVQ_OK) fprintf(stderr, "  %s\n", kvq_last_error());
              EXPECT(kvq_cache_bytes(&g0, bytes) == KVQ_OK);
              valid += st == KVQ_OK;
              for (int f = 0; f < 10; ++f)
                for (int32_t v : kVals) {
                  kvq_geom gm = g0;
                  int32_t* fields[10] = {&gm.batch, &gm.n_q_heads, &gm.n_kv_heads, &gm.head_dim,
                                         &gm.k_bits, &gm.v_bits, &gm.group, &gm.residual,
                                         &gm.capacity, &gm.residual_v};
                  *fields[f] = v;
                  const int sm = kvq_validate_geom(&gm);
                  EXPECT(kvq_cache_bytes(&gm, bytes) == sm);
                  size_t pb[6];
                  (void)kvq_paged_cache_bytes(&gm, 64, v, pb);
                }
            }
  EXPECT(valid > 0);
  for (int i = 0; i < 100000; ++i) {
    kvq_bq2_geom g;
    g.batch = pick(); g.n_q_heads = pick(); g.n_kv_heads = pick(); g.capacity = pick();
    const int st = kvq_bq2_validate_geom(&g);
    EXPECT(kvq_bq2_cache_bytes(&g, bytes) == st);
  }

  // null arguments are refused before anything else happens
  kvq_geom g = small_geom();
  EXPECT(kvq_validate_geom(&g) == KVQ_OK);
  kvq_cache c;
  c.k_codes = w32; c.v_codes = w32; c.k_meta = w16; c.v_meta = w16; c.k_res = w16;
  c.v_res = w16;
  EXPECT(kvq_append(&g, NULL, w16, lens, &c, NULL) == KVQ_ERR_NULL);
  EXPECT(kvq_append(&g, w16, w16, lens, NULL, NULL) == KVQ_ERR_NULL);
  EXPECT(kvq_decode_attn(&g, NULL, &c, lens, 256, 0.1f, w32, sizeof w32, w16, NULL) ==
         KVQ_ERR_NULL);
  EXPECT(kvq_quantize_keys_perchannel(&g, w16, 7, 32, w32, w16, NULL) == KVQ_ERR_RANGE);
  EXPECT(kvq_prefill(&g, w16, w16, 257, &c, NULL) == KVQ_ERR_RANGE);
  EXPECT(kvq_decode_attn(&g, w16, &c, lens, 0, 0.1f, w32, sizeof w32, w16, NULL) ==
         KVQ_ERR_RANGE);
  EXPECT(kvq_decode_attn_multi(&g, w16, &c, lens, 3, 256, 0.1f, w32, sizeof w32, w16, NULL) ==
         KVQ_ERR_RANGE);

  // the HIP-failure path: a call that reaches the runtime or a launcher gets
  // KVQ_ERR_HIP and the runtime's text
  EXPECT(kvq_append(&g, w16, w16, lens, &c, NULL) == KVQ_ERR_HIP);
  EXPECT(strstr(kvq_last_error(), "append") != NULL);
  int32_t nw = 0;
  EXPECT(kvq_decode_workers(&g, &nw) == KVQ_ERR_HIP);
  EXPECT(kvq_decode_attn(&g, w16, &c, lens, 256, 0.1f, w32, sizeof w32, w16, NULL) ==
         KVQ_ERR_HIP);
  EXPECT(kvq_decode_attn_noalloc(&g, w16, &c, lens, 256, 0.1f, w16, NULL) == KVQ_ERR_HIP);
  EXPECT(strlen(kvq_last_error()) > 0);

  // per-thread error text: each thread fails with its own value and must read
  // back its own text, never another thread's
  std::atomic<int> bad{0};
  std::vector<std::thread> th;
  for (int t = 0; t < 8; ++t)
    th.emplace_back([t, &bad] {
      kvq_geom gt = small_geom();
      gt.head_dim = 1000 + t;  // "head_dim must be 64 or 128 (got 100t)"
      char want[64];
      snprintf(want, sizeof want, "(got %d)", 1000 + t);
      for (int i = 0; i < 20000; ++i) {
        if (kvq_validate_geom(&gt) != KVQ_ERR_GEOM) ++bad;
        if (strstr(kvq_last_error(), want) == NULL) ++bad;
        if (i % 97 == 0) {  // a success leaves the text of the last failure alone
          kvq_geom ok = small_geom();
          if (kvq_validate_geom(&ok) != KVQ_OK) ++bad;
        }
      }
    });
  for (auto& x : th) x.join();
  EXPECT(bad.load() == 0);

  if (failures) {
    fprintf(stderr, "%d expectations failed\n", failures);
    return 1;
  }
  printf("host api under sanitizers: ok (%d valid geometries)\n", valid);
  return 0;
}
