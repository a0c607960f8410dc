// kvq_device.h — device helpers shared by the decode kernels of both cache
// formats: MFMA operand helpers (codes as fp16 subnormals, hi/lo fp16 splits),
// lane reductions, the persistent work decomposition over (sequence, KV head)
// units and the partial-merging combine kernel.  Included by the .hip files
// only; everything is in an unnamed namespace.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32;  // tokens per chunk (= value block)
constexpr int kWaves = kThreads / 64;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int packed_len(int n, int R) {
  return n <= 0 ? 0 : n - (((n - 1) % R) + 1);
}

__device__ __forceinline__ f4 mfma(const uint32_t (&a)[4], const uint32_t (&b)[4], f4 c) {
  const u4 av = {a[0], a[1], a[2], a[3]};
  const u4 bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, av),
                                                __builtin_bit_cast(h8, bv), c, 0, 0, 0);
}

// Two floats -> packed fp16 pair, rounded to nearest even (v_cvt_pk_f16_f32,
// the same rate as the round-toward-zero form).  Both parts of a hi/lo split
// are rounded to nearest: the lo part's rounding errors are then half an ulp
// of it, of either sign, so a weighted sum over many tokens carries no
// systematic bias (with truncation every weight came out up to 2^-22 low,
// which over a long context of large values exceeded the tolerance).
__device__ __forceinline__ uint32_t pk_rne(float a, float b) {
  const h2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_half(uint32_t v) {
  return (float)__builtin_bit_cast(h2, v)[0];
}
__device__ __forceinline__ float hi_half(uint32_t v) {
  return (float)__builtin_bit_cast(h2, v)[1];
}
// -1.0f that the compiler cannot see as a constant (kept in a register), so
// that hi * m1 + a stays one mixed-precision fma instead of a conversion and
// a subtraction.
__device__ __forceinline__ float opaque_m1() {
  float x = -1.0f;
  asm volatile("" : "+v"(x));
  return x;
}
// hi/lo fp16 split of (a, b): a ~= hi.x + lo.x to ~2^-23 relative.  The
// remainders a - hi.x are exact fp32 operations, each one v_fma_mix_f32 of
// the fp16 half (m1 = -1).
__device__ __forceinline__ void split2(float a, float b, float m1, uint32_t& hi,
                                       uint32_t& lo) {
  hi = pk_rne(a, b);
  const h2 hh = __builtin_bit_cast(h2, hi);
  lo = pk_rne(__builtin_fmaf((float)hh[0], m1, a), __builtin_fmaf((float)hh[1], m1, b));
}
// 2^x on the hardware unit (no range fix-up: results below the fp32 normal
// range only arise for weights that are negligible next to the running max).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// x * fp16 field of a packed (scale, min) word (+ acc), converted inside the
// fma (v_fma_mix_f32).  The +0 addend keeps the fma from being folded into a
// plain multiply that would need a separate conversion.
__device__ __forceinline__ float mul_lo(float x, uint32_t w, float acc = 0.0f) {
  return __builtin_fmaf(x, (float)__builtin_bit_cast(h2, w)[0], acc);
}
__device__ __forceinline__ float mul_hi(float x, uint32_t w, float acc = 0.0f) {
  return __builtin_fmaf(x, (float)__builtin_bit_cast(h2, w)[1], acc);
}

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m, 64)); }
__device__ __forceinline__ float xor_sum(float x, int m) { return x + __shfl_xor(x, m, 64); }

// DPP lane moves inside a row of 16 lanes (no LDS traffic).
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                           kCtrl, 0xF, 0xF, true));
}
// a where mask bits are set, else b (a bitwise merge: one VALU op; a select
// between two elements of one array could otherwise become an indexed private
// array)
__device__ __forceinline__ float bit_sel(uint32_t mask, float a, float b) {
  const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
  return __builtin_bit_cast(float, ub ^ ((ua ^ ub) & mask));
}

// Quad sharing of a lane group's 8 positions j = 4 u + q (two score tiles u,
// rows q) when the four lanes of a quad hold the same 8 values: quad lane i
// (masks m1, m2: all ones where bit 0 / bit 1 of i is set) takes positions
// 2 i and 2 i + 1, and gets all 8 results back from the quad.
__device__ __forceinline__ void quad_pick2(uint32_t m1, uint32_t m2, const float (&s)[2][4],
                                           float (&x)[2]) {
#pragma unroll
  for (int k = 0; k < 2; ++k)
    x[k] = bit_sel(m2, bit_sel(m1, s[1][2 + k], s[1][k]), bit_sel(m1, s[0][2 + k], s[0][k]));
}
__device__ __forceinline__ void quad_gather2(const float (&x)[2], float (&p)[2][4]) {
  // position j from quad lane j / 2 (quad_perm control: the source of quad
  // positions 0..3, 2 bits each)
  p[0][0] = dpp<0x00>(x[0]);
  p[0][1] = dpp<0x00>(x[1]);
  p[0][2] = dpp<0x55>(x[0]);
  p[0][3] = dpp<0x55>(x[1]);
  p[1][0] = dpp<0xAA>(x[0]);
  p[1][1] = dpp<0xAA>(x[1]);
  p[1][2] = dpp<0xFF>(x[0]);
  p[1][3] = dpp<0xFF>(x[1]);
}

// Sum over aligned groups of n lanes (n = 8 or 16).  Rotations act on whole
// 16-lane rows, so they serve n = 16; for n = 8 the 4-apart step is a lane
// shuffle.
template <int kN>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (kN >= 16) {
    x += dpp<0x128>(x);  // row_ror:8  -> lanes i, i+8
    x += dpp<0x124>(x);  // row_ror:4  -> lanes i, i+4, i+8, i+12
  } else {
    x = xor_sum(x, 4);
  }
  x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
  return x;
}

// ---------------------------------------------------------------------------
// Token order inside a 32-token chunk (the packed layout stores every chunk in
// this consumer order, so each lane's share is one contiguous run of words).
//
// Value side: the A operand of lane (channel c, lane group g) holds 8 codes of
// channel c; element j is token 8g + j.  A 4-bit word holds them with element
// 2e in nibble e and element 2e+1 in nibble 4 + e of the word, i.e. nibble e
// of its two halves form the fp16 pair (2e, 2e+1); a 2-bit word holds two
// channel tiles, tile parity h in bits 8h.. of each half (unpack_value_tile).
// Key side: score tile u row r is token 8 (r/4) + 4u + r%4, so the score
// tile's output registers (lane group g, register q of tile u) hold tokens
// 8g + 4u + q: exactly element 4u + q of the value side's B operand, and the
// scores never leave their lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ constexpr int key_row_token(int u, int r) {
  return 8 * (r >> 2) + 4 * u + (r & 3);
}

// First channel of the two 4-channel runs a key-side B fragment (lane group g,
// k-chunk kc) covers; element 2e is channel run0 + e, element 2e+1 is channel
// run0 + kOff + e.  Matches the unpack in unpack_keys().
template <int D, int BK>
__device__ __forceinline__ constexpr int key_run0(int g, int kc) {
  return BK == 2 ? g * (D / 4) + 16 * (kc >> 1) + 4 * (kc & 1) : g * (D / 4) + 8 * kc;
}
template <int BK>
constexpr int kKeyOff = BK == 2 ? 8 : 4;

// Lane's slice of a key row: channels [g*D/4, (g+1)*D/4) -> KW words.
template <int D, int BK>
constexpr int kKW = (D / 4) * BK / 32;

// Where a code sits inside its fp16 operand.  The matrix core aligns the 32
// products of an instruction by their operands' nominal exponents before it
// sums them, and keeps about 27 bits below the largest (measured on gfx950:
// one wave, exact fp64 sums; C is added with fp32 rounding).  A subnormal's
// nominal exponent is that of the smallest normal number, 2^-14, whatever its
// value, so a code at the bottom of the mantissa (c * 2^-24) wastes nearly ten
// of those bits: products about 18 binades below an instruction's largest
// already lose bits, which a cache whose scales differ by 2^15 between the
// tokens (values) or channels (keys) of one chunk reaches.  So every field is
// moved to the top of the mantissa: a pair comes out as code * 2^(L - 24) *
// (its class factor below), L = kCodeLift (2-bit fields at bits 6 and 8,
// 4-bit ones all at bits 6..9, 8-bit ones at bits 2..9), and the 2^L is
// taken back out by the power-of-two scale applied to the finished sums.
// (A 4-bit field at bits 2..5 would still sit 2^4 below the nominal exponent,
// and up to 32 products truncated one way against the largest cost about
// 2^-18 of it: measured on caches with large value scales.)
template <int B> constexpr int kCodeLift = B == 8 ? 2 : 6;

// Key codes to A-operand pairs with one AND per pair: a 2-bit odd pair
// (VGPR v odd) sits two bits above its even neighbour (the two share one
// shift), so it comes out as code * 4 * 2^(L - 24); 4-bit and 8-bit pairs all
// come out as code * 2^(L - 24).  The query fragments carry the inverse and a
// headroom factor: q' of an even channel is scaled by kKeyEvenQ and of an odd
// channel by kKeyOddQ (channel parity = pair parity, the runs start at
// multiples of 4), and every pair then contributes kKeyAcc * 2^L * code * q'.
// The factors keep q' inside fp16 for any fp16 keys (a scale is at most
// 43669 at 2 bits, 8734 at 4 and 514 at 8) and as large as that allows, so
// that the lo fp16 part of q' stays out of the subnormals for small key
// scales (a lo part in the subnormals has an absolute step that large codes
// magnify).
template <int BK> constexpr float kKeyEvenQ = BK == 4 ? 4.0f : BK == 8 ? 64.0f : 1.0f;
template <int BK> constexpr float kKeyOddQ = BK == 4 ? 4.0f : BK == 8 ? 64.0f : 0.25f;
template <int BK> constexpr int kKeyAccLog2 = BK == 4 ? 2 : BK == 8 ? 6 : 0;

// Value side, likewise: at 2 bits the odd pairs of a value word (VGPR e odd:
// tokens 8g + 2e, 8g + 2e + 1 with e odd, i.e. score registers q = 2, 3) come
// out of their mask as code * 4 * 2^(L - 24); their softmax weights are taken
// 4x smaller (2^(s - m - 2)), so every pair contributes 2^L * p * code * dV.
// 4-bit and 8-bit pairs all come out as code * 2^(L - 24) and both classes'
// weights carry a headroom factor (4 at 4 bits, 64 at 8: 4 * 8734 and
// 64 * 514 stay inside fp16), which keeps the lo parts of p dV normal.
template <int BV> constexpr float kValEven = BV == 4 ? 4.0f : BV == 8 ? 64.0f : 1.0f;
template <int BV> constexpr float kValOdd = BV == 4 ? 4.0f : BV == 8 ? 64.0f : 0.25f;
template <int BV> constexpr float kValEvenLog2 = BV == 4 ? 2.0f : BV == 8 ? 6.0f : 0.0f;
template <int BV> constexpr float kValOddLog2 = BV == 4 ? 2.0f : BV == 8 ? 6.0f : -2.0f;

// A word shifted left (k > 0) or right (k < 0) by |k| bits.
template <int K>
__device__ __forceinline__ uint32_t shl(uint32_t w) {
  if constexpr (K >= 0)
    return w << K;
  else
    return w >> (-K);
}
// Masks of the lifted fields in both halves of a word: even and odd pairs.
template <int B> constexpr uint32_t kMaskEven = B == 2 ? 0x00C000C0u : B == 4 ? 0x03C003C0u
                                                                               : 0x03FC03FCu;
template <int B> constexpr uint32_t kMaskOdd = B == 2 ? 0x03000300u : B == 4 ? 0x03C003C0u
                                                                              : 0x03FC03FCu;

// Two words shifted left (K > 0) or right (K < 0) by |K| <= 6 bits as one
// 64-bit shift (which issues at the rate of a 32-bit one).  The bits that
// cross between the two words land in bits [0, K) of the high word or
// [32 - |K|, 32) of the low one, which the 2-bit field masks clear (they
// cover bits 6..9 and 22..25).  Written as the instruction itself: seeing the
// masks, the compiler would otherwise split it back into 32-bit shifts.
template <int K>
__device__ __forceinline__ void shl_pair(uint32_t lo, uint32_t hi, uint32_t& out_lo,
                                         uint32_t& out_hi) {
  static_assert(K >= -6 && K <= 6, "fields stay clear of the crossing bits");
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  uint64_t r;
  if constexpr (K >= 0)
    asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "i"(K), "v"(v));
  else
    asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "i"(-K), "v"(v));
  out_lo = (uint32_t)r;
  out_hi = (uint32_t)(r >> 32);
}

// 2-bit codes of a 64-channel head: the two score tiles' A operands from a
// lane's two key words (tile u: word u) and the four value tiles' from its two
// value words (tiles 2w, 2w + 1 share word w), each pair of words shifted
// together: the results of unpack_keys<64, 2> per word and unpack_value_tile<2>
// per tile with half the shifts.
__device__ __forceinline__ void unpack_keys_2x64(const uint32_t (&w)[2],
                                                 uint32_t (&a)[2][2][4]) {
  uint32_t x[4][2];
  shl_pair<6>(w[0], w[1], x[0][0], x[0][1]);
  shl_pair<2>(w[0], w[1], x[1][0], x[1][1]);
  shl_pair<-2>(w[0], w[1], x[2][0], x[2][1]);
  shl_pair<-6>(w[0], w[1], x[3][0], x[3][1]);
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int f = 0; f < 8; ++f)
      a[u][f >> 2][f & 3] = x[f >> 1][u] & ((f & 1) ? kMaskOdd<2> : kMaskEven<2>);
}
__device__ __forceinline__ void unpack_values_2x64(const uint32_t (&vw)[2],
                                                   uint32_t (&a)[4][4]) {
  uint32_t l6[2], l2[2], r2[2], r6[2];
  shl_pair<6>(vw[0], vw[1], l6[0], l6[1]);
  shl_pair<2>(vw[0], vw[1], l2[0], l2[1]);
  shl_pair<-2>(vw[0], vw[1], r2[0], r2[1]);
  shl_pair<-6>(vw[0], vw[1], r6[0], r6[1]);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int wi = n >> 1;
    const uint32_t x0 = (n & 1) ? r2[wi] : l6[wi];
    const uint32_t x1 = (n & 1) ? r6[wi] : l2[wi];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a[n][e] = (e < 2 ? x0 : x1) & ((e & 1) ? kMaskOdd<2> : kMaskEven<2>);
  }
}

template <int D, int BK>
__device__ __forceinline__ void unpack_keys(const uint32_t (&w)[kKW<D, BK>],
                                            uint32_t (&a)[D / 32][4]) {
  constexpr int KW = kKW<D, BK>;
  if constexpr (BK == 2 || BK == 4) {
    // 2 bits: field s of a half (bits 2s) to bit 6 (even s) or 8 (odd s):
    // fields 2j, 2j + 1 share the shift 6 - 4j.  4 bits: nibble s of a half
    // (bits 4s) to bits 6..9.  Words are shifted in pairs (one 64-bit shift
    // for two words) where there are two.
#pragma unroll
    for (int wp = 0; wp < KW; wp += 2) {
      constexpr int NP = KW >= 2 ? 2 : 1;
      uint32_t x[4][NP];
      if constexpr (NP == 2) {
        shl_pair<6>(w[wp], w[wp + 1], x[0][0], x[0][1]);
        shl_pair<2>(w[wp], w[wp + 1], x[1][0], x[1][1]);
        shl_pair<-2>(w[wp], w[wp + 1], x[2][0], x[2][1]);
        shl_pair<-6>(w[wp], w[wp + 1], x[3][0], x[3][1]);
      } else {
        x[0][0] = shl<6>(w[wp]);
        x[1][0] = shl<2>(w[wp]);
        x[2][0] = shl<-2>(w[wp]);
        x[3][0] = shl<-6>(w[wp]);
      }
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const int wi = wp + k;
        if constexpr (BK == 2) {
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int ri = 8 * wi + s;
            a[ri >> 2][ri & 3] = x[s >> 1][k] & ((s & 1) ? kMaskOdd<2> : kMaskEven<2>);
          }
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) a[wi][s] = x[s][k] & kMaskEven<4>;
        }
      }
    }
  } else {
    // k-chunk kc from words 2kc + (s/2): pair s is bytes 0, 2 (s even) or
    // 1, 3 (s odd) of that word, moved to bits 2..9 of each half (the two
    // words of a k-chunk shifted together)
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      uint32_t l2[2], r6[2];
      shl_pair<2>(w[2 * kc], w[2 * kc + 1], l2[0], l2[1]);
      shl_pair<-6>(w[2 * kc], w[2 * kc + 1], r6[0], r6[1]);
#pragma unroll
      for (int s = 0; s < 4; ++s) a[kc][s] = ((s & 1) ? r6[s >> 1] : l2[s >> 1]) & kMaskEven<8>;
    }
  }
}

// The A operand of value channel tile n (pairs e = 0..3: tokens 2e, 2e + 1 of
// the lane group) from a lane's value code words vw (layout 3):
//   bV = 4: word n, token pair e in nibble e of each half -> bits 6..9;
//   bV = 2: word n/2, tile parity h = n % 2, pair e at bits 8h + 2e -> bit 6
//           (even e) or 8 (odd e); pairs 2j, 2j + 1 share the shift 6 - 4j - 8h;
//   bV = 8: words 2n + e/2, pair e in bytes (0, 2) or (1, 3) -> bits 2..9.
template <int BV, int NW>
__device__ __forceinline__ void unpack_value_tile(const uint32_t (&vw)[NW], int n,
                                                  uint32_t (&a)[4]) {
  if constexpr (BV == 4) {
    const uint32_t x[4] = {shl<6>(vw[n]), shl<2>(vw[n]), shl<-2>(vw[n]), shl<-6>(vw[n])};
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = x[e] & kMaskEven<4>;
  } else if constexpr (BV == 2) {
    const uint32_t w = vw[n >> 1];
    const uint32_t x0 = (n & 1) ? shl<-2>(w) : shl<6>(w);
    const uint32_t x1 = (n & 1) ? shl<-6>(w) : shl<2>(w);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = (e < 2 ? x0 : x1) & ((e & 1) ? kMaskOdd<2> : kMaskEven<2>);
  } else {
    // the tile's two words shifted together
    uint32_t l2[2], r6[2];
    shl_pair<2>(vw[2 * n], vw[2 * n + 1], l2[0], l2[1]);
    shl_pair<-6>(vw[2 * n], vw[2 * n + 1], r6[0], r6[1]);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = ((e & 1) ? r6[e >> 1] : l2[e >> 1]) & kMaskEven<8>;
  }
}

// 4-bit value tiles n and n + 1 (n even) at once, their code words shifted in
// pairs (one 64-bit shift for two words); the same operands as
// unpack_value_tile.
template <int BV, int NW>
__device__ __forceinline__ void unpack_value_tiles2(const uint32_t (&vw)[NW], int n,
                                                    uint32_t (&a0)[4], uint32_t (&a1)[4]) {
  static_assert(BV == 4, "4-bit tiles (2-bit tiles share one word, 8-bit ones pair inside)");
  uint32_t x[4][2];
  shl_pair<6>(vw[n], vw[n + 1], x[0][0], x[0][1]);
  shl_pair<2>(vw[n], vw[n + 1], x[1][0], x[1][1]);
  shl_pair<-2>(vw[n], vw[n + 1], x[2][0], x[2][1]);
  shl_pair<-6>(vw[n], vw[n + 1], x[3][0], x[3][1]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a0[e] = x[e][0] & kMaskEven<4>;
    a1[e] = x[e][1] & kMaskEven<4>;
  }
}

// N consecutive words (N = 1, 2, 4 or 8; 4 N-byte aligned up to 16) as wide
// nontemporal loads: the packed cache streams through once per step, and loads
// that do not allocate in the caches read HBM about a sixth faster than plain
// ones on this GPU (a plain 16-byte stream levels off near 6.0 TB/s, a
// nontemporal one near 7.0 TB/s).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int N>
__device__ __forceinline__ void load_run(const uint32_t* p, uint32_t (&w)[N]) {
  if constexpr (N == 1) {
    w[0] = __builtin_nontemporal_load(p);
  } else if constexpr (N == 2) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + k);
      w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
  }
}


// Direct loads from global memory into LDS (global_load_lds_dwordx4): lane l
// of an instruction reads the 16 bytes at g + 16 l and the LDS takes them at
// byte address lds + 16 l; lanes with exec off neither read nor write.  g and
// lds are wave-uniform.  No data passes through registers, so a chunk in
// flight costs no VGPRs.  The compiler does not see these loads: the caller
// waits for them with wait_vm<n>() before reading the LDS bytes (loads finish
// in issue order, so vmcnt(n) means all but the last n issued are done), and
// lds_dma_begin() before the first load that overwrites bytes the wave read.
__device__ __forceinline__ void lds_dma_begin() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
template <bool NT>
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds, uint32_t lane16) {
  // (readfirstlane returns int: each half goes through uint32_t, so the low
  // half is zero-extended, not sign-extended, into the 64-bit address)
  const uint64_t g64 = reinterpret_cast<uint64_t>(g);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane((uint32_t)(g64 >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane((uint32_t)g64));
  const uint64_t ga = ((uint64_t)hi << 32) | (uint64_t)lo;
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :: "s"(lds), "v"(lane16), "s"(ga) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds), "v"(lane16), "s"(ga) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// The LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}
// Copies `bytes` (a multiple of 16) from g to LDS address lds, 1 KB per
// instruction; the last one with lanes past the end switched off.  Returns
// nothing; issues (bytes + 1023) / 1024 loads.
template <int BYTES, bool NT>
__device__ __forceinline__ void lds_copy(const char* g, uint32_t lds, uint32_t lane16, int lane) {
  static_assert(BYTES % 16 == 0, "16-byte pieces");
#pragma unroll
  for (int i = 0; i < (BYTES + 1023) / 1024; ++i) {
    constexpr int kFull = BYTES / 1024;
    if (i < kFull) {
      lds_dma16<NT>(g + 1024 * i, lds + 1024 * i, lane16);
    } else if (lane < (BYTES - 1024 * kFull) / 16) {
      lds_dma16<NT>(g + 1024 * i, lds + 1024 * i, lane16);
    }
  }
}


// ---------------------------------------------------------------------------
// Persistent decomposition.  The work of one (sequence, KV head) unit is its
// packed 32-token chunks (one work unit each) followed by the 32-token chunks
// of its fp16 residual window (rw work units each: rw ~ fp16 bytes / packed
// bytes per token, so that work units stand for equal HBM traffic).  The units
// in order u = b * Hkv + hkv form one flat work list of `total` units.  Worker
// wave w of the W launched takes [w * cpw, min((w + 1) * cpw, total)),
// cpw = ceil(total / W): every wave moves the same number of bytes whatever
// the mix of lengths.  A packed chunk belongs to the wave whose range holds
// it; a residual chunk to the wave whose range holds its first work unit.  A
// wave writes one partial per unit its range meets, at index w + u (distinct
// over all (w, u) pairs that occur, at most W + units of them); a partial with
// no tokens has max -inf and sum 0.
// ---------------------------------------------------------------------------
// A cache format supplies a policy Fmt: Fmt::Launch (its launch record, with
// g.B, g.Hq, g.Hkv, g.C, seq_lens, max_seq_len, n_workers, rw, ws, out),
// Fmt::work_of(L, n), the work of one KV head of a sequence of n tokens, and
// Fmt::row(L, b, hkv, j), the query / output row of row j of unit (b, hkv).
// ---------------------------------------------------------------------------
constexpr int kPartPad = 4;  // partial row = D values, max, sum, 2 pad floats

struct SeqWork {
  int n;   // tokens (0 for an invalid length)
  int nq;  // packed chunks per KV head
  int nr;  // residual chunks per KV head (rw work units each; the first nm of
           // them are mixed chunks, packed for one tensor only)
  int w;   // work units per KV head
  int nm = 0;          // mixed chunks (separate key and value windows)
  bool keys_packed = false;  // in the mixed chunks: keys packed (else values)
};
// Inclusive prefix sum over the wave's 64 lanes: DPP shifts inside each row
// of 16 lanes, then row broadcasts (lane 15 into the next row, lane 31 into
// rows 2 and 3); lanes a DPP move does not reach add 0.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// The batch's work layout as one wave sees it: for the first 64 sequences,
// lane b holds sequence b's work over all its KV heads (c) and the inclusive
// prefix (inc); total covers the whole batch.
struct BatchWork {
  int c, inc, head_total, total;
  int n;  // lane b < 64: length of sequence b
};

template <class Fmt>
__device__ __forceinline__ BatchWork batch_work(const typename Fmt::Launch& L, int lane) {
  BatchWork bw;
  const int n = lane < L.g.B ? L.seq_lens[lane] : L.max_seq_len;
  bw.n = n;
  bw.c = lane < L.g.B ? Fmt::work_of(L, n).w * L.g.Hkv : 0;
  bw.inc = wave_scan_incl(bw.c);
  bw.head_total = __builtin_amdgcn_readlane(bw.inc, 63);
  bw.total = bw.head_total;
  for (int b0 = 64; b0 < L.g.B; b0 += 64) {  // batches beyond 64 sequences
    const int nb = b0 + lane < L.g.B ? L.seq_lens[b0 + lane] : L.max_seq_len;
    int s = b0 + lane < L.g.B ? Fmt::work_of(L, nb).w * L.g.Hkv : 0;
    s = wave_scan_incl(s);
    bw.total += __builtin_amdgcn_readlane(s, 63);
  }
  return bw;
}

// Sequence b holding flat work unit x < total, and base = Hkv * (work of
// sequences < b).
template <class Fmt>
__device__ __forceinline__ void wave_find_seq(const typename Fmt::Launch& L, const BatchWork& bw,
                                              int lane, int x, int& b_out, int& base_out) {
  if (x < bw.head_total) {
    const uint64_t m = __ballot(bw.inc > x);
    const int l = __ffsll((unsigned long long)m) - 1;
    b_out = l;
    base_out = __builtin_amdgcn_readlane(bw.inc - bw.c, l);
    return;
  }
  int base = bw.head_total;
  for (int b0 = 64; b0 < L.g.B; b0 += 64) {
    const int b = b0 + lane;
    const int c = (b < L.g.B) ? Fmt::work_of(L, L.seq_lens[b]).w * L.g.Hkv : 0;
    const int inc = wave_scan_incl(c);
    const uint64_t m = __ballot(base + inc > x);
    if (m) {
      const int l = __ffsll((unsigned long long)m) - 1;
      b_out = b0 + l;
      base_out = base + __builtin_amdgcn_readlane(inc - c, l);
      return;
    }
    base += __builtin_amdgcn_readlane(inc, 63);
  }
  b_out = L.g.B;
  base_out = base;
}
// Packed chunks [pc0, pc1) and residual chunks [rk0, rk1) of unit work
// starting at xu that fall in the work range [x0, x1).
struct SegRange {
  int pc0, pc1, rk0, rk1;
};

template <class Launch>
__device__ __forceinline__ SegRange seg_range(const Launch& L, const SeqWork& sw, int xu, int x0,
                                              int x1) {
  SegRange r;
  r.pc0 = max(x0, xu) - xu;
  r.pc1 = min(x1, xu + sw.nq) - xu;
  const int d0 = x0 - xu - sw.nq, d1 = x1 - xu - sw.nq;
  r.rk0 = d0 <= 0 ? 0 : (d0 + L.rw - 1) / L.rw;
  r.rk1 = min(sw.nr, d1 <= 0 ? 0 : (d1 + L.rw - 1) / L.rw);
  return r;
}
// One workgroup per RS rows of a (KV head, sequence) unit (RS = GQ: the whole
// unit; RS = 1: one row, for launches with few units, where a unit's many
// partials would otherwise be streamed by few workgroups; in between for units
// with more outputs than a workgroup has threads); blockIdx.x =
// hkv * (GQ / RS) + row group.  Merges the unit's partials for those rows and
// writes their outputs:
//   M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L.
// The unit's partials are contiguous (indices w + u for consecutive waves w).
// Each thread owns one float4 of the output and a 1/P share of the partials
// and merges them as a stream (running max, rescale when it grows), so the
// (m, l, o) loads of a partial do not wait for any reduction; the P shares are
// then merged through LDS.  Empty partials (m = -inf) carry weight 0.
template <class Fmt, int D, int GQ, int RS = GQ>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(typename Fmt::Launch L) {
  static_assert(GQ % RS == 0, "whole row groups of a unit");
  constexpr int DP = D + kPartPad;
  constexpr int NO = RS * D / 4;                          // float4 outputs of the workgroup
  constexpr int P = NO >= kThreads ? 1 : kThreads / NO;   // partial shares per output
  constexpr int OPT = NO >= kThreads ? NO / kThreads : 1;  // outputs per thread
  constexpr int U = 4;                                     // partials in flight per thread
  static_assert(NO % kThreads == 0 || kThreads % NO == 0, "outputs tile the workgroup");
  constexpr bool kRotate = Fmt::kRotateOut;  // out = H o per head (64 channels)
  static_assert(!kRotate || (D == 64 && OPT == 1), "rotation covers one 64-channel head");
  // (a row's 16 float4 outputs sit in 16 consecutive lanes of the first wave:
  // the rotation's lane exchanges stay inside them)
  static_assert(!kRotate || NO % 16 == 0, "a row's outputs are whole 16-lane groups");
  __shared__ int red[2 * kThreads / 64];
  __shared__ float4 s_o[kThreads];
  __shared__ float2 s_ml[kThreads];
  const auto& g = L.g;
  const int hkv = blockIdx.x / (GQ / RS), row0 = (blockIdx.x % (GQ / RS)) * RS;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int n = L.seq_lens[b];
  if (n < 0 || n > g.C || n > L.max_seq_len) {
    for (int i = tid; i < RS * D; i += kThreads)
      L.out[Fmt::row(L, b, hkv, row0 + i / D) * D + i % D] = 0x7e00;  // NaN
    return;
  }
  if (n == 0) {
    for (int i = tid; i < RS * D; i += kThreads)
      L.out[Fmt::row(L, b, hkv, row0 + i / D) * D + i % D] = 0;
    return;
  }
  // flat position of this unit's work
  int tot = 0, pre = 0;
  for (int bb = tid; bb < g.B; bb += kThreads) {
    const int c = Fmt::work_of(L, L.seq_lens[bb]).w;
    tot += c;
    if (bb < b) pre += c;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    tot += __shfl_xor(tot, off, 64);
    pre += __shfl_xor(pre, off, 64);
  }
  if ((tid & 63) == 0) {
    red[tid >> 6] = tot;
    red[kThreads / 64 + (tid >> 6)] = pre;
  }
  __syncthreads();
  tot = 0;
  pre = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    tot += red[i];
    pre += red[kThreads / 64 + i];
  }
  const int total = tot * g.Hkv;
  const SeqWork sw = Fmt::work_of(L, L.seq_lens[b]);
  const int xu = pre * g.Hkv + hkv * sw.w;
  const int cpw = (total + L.n_workers - 1) / L.n_workers;
  const int w_first = xu / cpw, w_last = (xu + sw.w - 1) / cpw;
  const int S = w_last - w_first + 1;
  const float* base = L.ws + (int64_t)(w_first + b * g.Hkv + hkv) * GQ * DP;
  const int share = (P > 1) ? tid / NO : 0;

#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    const int t = (P > 1) ? tid % NO : tid + j * kThreads;
    const int ol = t / (D / 4), oh = row0 + ol, oc = (t % (D / 4)) * 4;
    const float* pr = base + oh * DP;
    float M = kNegInf, Ls = 0.0f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = share; s0 < S; s0 += U * P) {
      float m[U], l[U];
      float4 o[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        // a partial past the end re-reads this thread's first one with weight 0
        const int sk = s0 + k * P;
        const float* q = pr + (int64_t)(sk < S ? sk : share) * GQ * DP;
        m[k] = q[D];
        l[k] = q[D + 1];
        o[k] = *reinterpret_cast<const float4*>(q + oc);
        if (sk >= S) m[k] = kNegInf;
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if (m[k] == kNegInf) continue;
        const float Mn = fmaxf(M, m[k]);
        const float a = exp2_hw(M - Mn);  // 0 while M is -inf
        const float c = exp2_hw(m[k] - Mn);
        M = Mn;
        Ls = Ls * a + l[k] * c;
        O.x = O.x * a + o[k].x * c;
        O.y = O.y * a + o[k].y * c;
        O.z = O.z * a + o[k].z * c;
        O.w = O.w * a + o[k].w * c;
      }
    }
    if constexpr (P > 1) {
      s_o[tid] = O;
      s_ml[tid] = make_float2(M, Ls);
      __syncthreads();
      if (share == 0) {
#pragma unroll
        for (int q = 1; q < P; ++q) {
          const float2 ml = s_ml[tid + q * NO];
          if (ml.x == kNegInf) continue;
          const float4 oq = s_o[tid + q * NO];
          const float Mn = fmaxf(M, ml.x);
          const float a = exp2_hw(M - Mn), c = exp2_hw(ml.x - Mn);
          M = Mn;
          Ls = Ls * a + ml.y * c;
          O.x = O.x * a + oq.x * c;
          O.y = O.y * a + oq.y * c;
          O.z = O.z * a + oq.z * c;
          O.w = O.w * a + oq.w * c;
        }
      }
    }
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;  // a row that sees no position: 0
    const int64_t o = Fmt::row(L, b, hkv, oh) * D + oc;
    if constexpr (kRotate) {
      // out_c = sum_j H[c][j] o_j / 8, H[c][j] = (-1)^popcount(c & j): the fast
      // Walsh-Hadamard transform, six butterfly stages (a, b) -> (a + b, a - b)
      // over channel bits 0..5.  Lane i of a row's 16 holds channels 4 i .. 4 i
      // + 3, so bits 0 and 1 pair values inside a lane and bits 2..5 pair lanes
      // i and i ^ 2^(bit - 2).
      if (share == 0) {
        float x[4] = {O.x * inv, O.y * inv, O.z * inv, O.w * inv};
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {  // channel bits 0, 1: inside the lane
          const int sp = 1 << sb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (e & sp) continue;
            const float a = x[e], bb = x[e + sp];
            x[e] = a + bb;
            x[e + sp] = a - bb;
          }
        }
        const int i = t % (D / 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {  // channel bits 2..5: across lanes
          const int m = 1 << k;
          const bool upper = (i & m) != 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = __shfl_xor(x[e], m, 64);
            x[e] = upper ? p - x[e] : x[e] + p;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) L.out[o + e] = f2h(x[e] * 0.125f);
      }
    } else if (share == 0) {
      L.out[o + 0] = f2h(O.x * inv);
      L.out[o + 1] = f2h(O.y * inv);
      L.out[o + 2] = f2h(O.z * inv);
      L.out[o + 3] = f2h(O.w * inv);
    }
  }
}
// Units of a launch below which the combine takes one row per workgroup.
constexpr int kCombineRowUnits = 128;

}  // namespace
}  // namespace kvq
