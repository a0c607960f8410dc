// kvq_decode.hip — single-token decode attention over the packed cache plus
// the fp16 residual window: split-context partial softmax and combine (gfx950).
//
// What is computed (KIVI repository page, "Overview": attention with keys
// quantized per channel and values per token, the recent tokens kept in fp16;
// KV1-1.2B model card, "Quickstart": attending over the dequantized cache gives
// the exact low-bit result):
//   s_t = sm_scale * q . k_t,  out = sum_t softmax(s)_t v_t
// with k_t = code * scale + min from the key group's per-channel (scale, min)
// for packed tokens, the fp16 residual for the rest, and v_t likewise from the
// token's per-group (scale, min).
//
// Algebra on the dequantizer (per key group j and value group gamma):
//   q . k_t = sum_c (q_c scale_jc) code_tc + sum_c q_c min_jc
//   sum_t p_t v_tc = sum_t (p_t scale_t,gamma) code_tc + sum_t p_t min_t,gamma
// so both contractions run on the small integer codes.  On gfx950 they are done
// by v_mfma_f32_16x16x32_f16 with the codes fed as fp16 subnormals (a code c
// masked out of a packed word *is* the fp16 number c * 2^-24, which the matrix
// cores multiply exactly) and the fp32 factors (q * scale, p * scale) split into
// a high and a low fp16 part, two MFMAs accumulating into the same fp32 tile.
// The scaled-query and weight operands are computed once per key group / per
// 32-token chunk; everything per code is a shift and a mask.
//
// Work decomposition: a persistent grid of single-wave workgroups, as many
// as the GPU keeps resident at once.  The 32-token chunks of all (sequence,
// KV head) units (packed chunks, then the fp16 residual window's chunks, each
// weighted by its bytes) form one flat list; every wave takes an equal
// contiguous share of it (so any mix of sequence lengths is balanced) and runs
// an online softmax over it, writing one partial (max, sum, weighted values)
// per unit its share touches.  The GQA query heads of a KV head share every
// load.  The combine kernel (one workgroup per unit) merges a unit's partials:
//   M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L.
// Scores are kept in log2 units (sm_scale * log2 e folded into q).
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

// Two floats -> packed fp16 pair, rounded toward zero (hi part of a hi/lo
// split; the lo part carries the remainder, so the rounding mode of the split
// does not matter).
__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
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
// hi/lo fp16 split of (a, b): a ~= hi.x + lo.x to ~2^-21 relative.  The
// remainders a - hi.x are exact fp32 operations, each one v_fma_mix_f32 of
// the fp16 half (m1 = -1).
__device__ __forceinline__ void split2(float a, float b, float m1, uint32_t& hi,
                                       uint32_t& lo) {
  hi = pk_rtz(a, b);
  const h2 hh = __builtin_bit_cast(h2, hi);
  lo = pk_rtz(__builtin_fmaf((float)hh[0], m1, a), __builtin_fmaf((float)hh[1], m1, b));
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
// 2e in nibble e and element 2e+1 in nibble 4 + e, so (w >> 4e) & 0x000F000F
// is the fp16 pair (2e, 2e+1); a 2-bit word holds two channel tiles, tile
// parity h in bits 8h.., and (w >> (8h + 2e)) & 0x00030003 is the pair.
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

// Key codes to A-operand pairs with one AND per pair: an odd pair (VGPR v
// odd) is masked where it sits, two bits (2-bit fields) or four bits (4-bit)
// above its even neighbour, so it comes out as code * 4 (or * 16) * 2^-24.
// The query fragments carry the inverse: q' of an even channel is scaled by
// kKeyEvenQ and of an odd channel by kKeyOddQ (channel parity = pair parity,
// the runs start at multiples of 4), and every pair then contributes
// kKeyAcc * code * q'.  The factors keep q' inside fp16 for any fp16 keys
// (a 4-bit scale is at most 8734, a 2-bit one is not scaled up).
template <int BK> constexpr float kKeyEvenQ = BK == 2 ? 1.0f : 4.0f;
template <int BK> constexpr float kKeyOddQ = 0.25f;
template <int BK> constexpr int kKeyAccLog2 = BK == 2 ? 0 : 2;

// Value side, likewise: the odd pairs of a value word (VGPR e odd: tokens
// 8g + 2e, 8g + 2e + 1 with e odd, i.e. score registers q = 2, 3) come out of
// their mask as code * 16 (4-bit) or * 4 (2-bit) * 2^-24.  Their softmax
// weights are taken 4x smaller (2^(s - m - 2)) and the even pairs' weights
// kValEven times larger, so every pair contributes kValEven * p * code * dV.
// (4 * 8734 and 43669 stay inside fp16.)
template <int BV> constexpr float kValEven = BV == 4 ? 4.0f : 1.0f;
template <int BV> constexpr float kValOdd = 0.25f;
template <int BV> constexpr float kValEvenLog2 = BV == 4 ? 2.0f : 0.0f;
constexpr float kValOddLog2 = -2.0f;

template <int D, int BK>
__device__ __forceinline__ void unpack_keys(const uint32_t (&w)[kKW<D, BK>],
                                            uint32_t (&a)[D / 32][4]) {
  if constexpr (BK == 2) {
    // field s of a half: (w >> 4 (s/2)) masked at bits 2 (s%2)
#pragma unroll
    for (int wi = 0; wi < kKW<D, BK>; ++wi)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int ri = 8 * wi + s;
        a[ri >> 2][ri & 3] = (w[wi] >> (4 * (s >> 1))) & ((s & 1) ? 0x000C000Cu : 0x00030003u);
      }
  } else {
    // field s of a half: (w >> 8 (s/2)) masked at bits 4 (s%2)
#pragma unroll
    for (int wi = 0; wi < kKW<D, BK>; ++wi)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[wi][s] = (w[wi] >> (8 * (s >> 1))) & ((s & 1) ? 0x00F000F0u : 0x000F000Fu);
  }
}

// N consecutive words (N = 2, 4 or 8; 8 N-byte aligned up to 16) as wide loads.
template <int N>
__device__ __forceinline__ void load_run(const uint32_t* p, uint32_t (&w)[N]) {
  if constexpr (N == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[k];
      w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
  }
}

// ---------------------------------------------------------------------------
// Packed tokens of one split: MFMA path.  NG = head_dim / group is a template
// parameter, so the key-group length G = D / NG and the value-tile -> group
// mapping are compile-time constants (no branches around the accumulators).
// ---------------------------------------------------------------------------
template <int D, int BK, int BV, int GQ, int NG>
struct Cfg {
  static constexpr int G = D / NG;
  static constexpr int KC = D / 32;               // k-chunks of a score tile
  static constexpr int NT = D / 16;               // value channel tiles
  static constexpr int NW = D * BV / 64;          // value code words per lane
  static constexpr int KW = kKW<D, BK>;           // key words per lane and row
  static constexpr int WR = D * BK / 32;          // words per key row
  static constexpr int SL = 16 / GQ;              // MFMA columns per head
  static constexpr int NF = (NG + SL - 1) / SL;   // value-side B fragments
  static constexpr int IPH = 4 * KC;              // fold items per head
  static constexpr int ITEMS = GQ * IPH;          // fold items per key group
  static constexpr int IPL = (ITEMS + 63) / 64;   // fold items per lane
  // LDS (bytes) per wave: q' fragments [2][GQ][4][KC] x 16 B, beta [GQ]
  static constexpr int kQB = 2 * GQ * 4 * KC * 16;
  static constexpr int kWaveLds = kQB + 16 * ((GQ * 4 + 4 + 15) / 16);  // + spare beta
  static constexpr int gam(int n) { return (16 * n) / G; }  // group of value tile n
};

// Loads of one 32-token chunk (a lane's share).
template <int D, int BK, int BV, int GQ, int NG>
struct Raw {
  using C = Cfg<D, BK, BV, GQ, NG>;
  uint32_t kw[2][C::KW];              // key code words of score tiles 0, 1
  uint32_t vw[C::NW];                 // value code words (tile n: word n*BV/4)
  uint32_t vmA[C::NF][4], vmB[C::NF][4];  // value (scale, min) of the B elements
  uint4 kmA[C::IPL], kmB[C::IPL];     // key (scale, min) of the chunk's group
};

template <int D, int BK, int BV, int GQ, int NG>
struct PackedWave {
  using C = Cfg<D, BK, BV, GQ, NG>;
  using R = Raw<D, BK, BV, GQ, NG>;
  static constexpr int KC = C::KC, NT = C::NT, KW = C::KW, WR = C::WR, SL = C::SL;
  static constexpr int NF = C::NF, IPH = C::IPH, IPL = C::IPL, G = C::G;
  // With two or more MFMA columns per head, the hi and lo parts of q' go to
  // neighbouring columns (one MFMA per k-chunk, one DPP add to recombine);
  // with one column per head they are two MFMAs into the same accumulator.
  static constexpr bool kColSplit = SL >= 2;
  static constexpr int KP = kColSplit ? 1 : 2;  // q' parts held per lane

  // wave-uniform bases
  const uint32_t* kcodes;
  const uint32_t* kmeta;
  const uint32_t* vcodes;
  const uint32_t* vmeta;
  const float* qfs;
  uint4* qB;
  float* beta_l;
  // lane constants
  int lane, col, lg, hcol, slot;
  int kofs, vofs;      // this lane's key / value words inside a chunk
  int vmofs[NF];       // value meta run of fragment f inside a chunk
  int kmofs[IPL];      // key meta run of fold item i inside a group
  int kmoff[IPL][2];   // channels of fold item i (runs A and B)
  int fitem[IPL];
  float kscale, bscale;
  float m1;  // -1 in a register (split2)
  // state
  f4 oacc[NT];
  float m_run, l_run;
  float m_even, m_odd;  // m_run less the classes' log2 factors (packed chunks)
  float l_odd;          // sum of odd-class weights (scaled by kValOdd)
  float bias[NF];       // value-min term; odd class kept apart in bias_odd
  float bias_odd[NF];
  uint32_t bq[KP][KC][4];
  float beta_c;
  int cur_group;

  __device__ void init(int lane_) {
    lane = lane_;
    m1 = opaque_m1();
    col = lane & 15;
    lg = lane >> 4;
    hcol = col / SL;
    slot = col % SL;
    kofs = lane * 2 * KW;
    vofs = lane * C::NW;
#pragma unroll
    for (int f = 0; f < NF; ++f) vmofs[f] = (lg * NG + (f * SL + slot) % NG) * 8;
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      const int it = lane + 64 * i;
      fitem[i] = it;
      const int r = it % IPH, gg = r / KC, kc = r % KC;
      kmofs[i] = r * 8;
      kmoff[i][0] = key_run0<D, BK>(gg, kc);
      kmoff[i][1] = kmoff[i][0] + kKeyOff<BK>;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) oacc[n] = f4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    m_even = kNegInf;
    m_odd = kNegInf;
    l_run = 0.0f;
    l_odd = 0.0f;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      bias[f] = 0.0f;
      bias_odd[f] = 0.0f;
    }
    beta_c = 0.0f;
    cur_group = -1;
  }

  __device__ __forceinline__ void load(int ch, R& r) const {
    {
      uint32_t w[2 * KW];
      load_run<2 * KW>(kcodes + (int64_t)ch * (D * BK) + kofs, w);
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        r.kw[0][k] = w[k];
        r.kw[1][k] = w[KW + k];
      }
    }
    load_run<C::NW>(vcodes + (int64_t)ch * (D * BV) + vofs, r.vw);
    // value (scale, min) of tokens 8 lg + j: even j feed B elements 2i (run
    // A), odd j elements 2i + 1 (run B)
    const uint32_t* vm = vmeta + (int64_t)ch * (4 * NG * 8);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      uint32_t w[8];
      load_run<8>(vm + vmofs[f], w);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r.vmA[f][i] = w[2 * i];
        r.vmB[f][i] = w[2 * i + 1];
      }
    }
    // key meta of the chunk's group, with the chunk's other loads (one
    // in-order stream, so waiting for a chunk never waits for a later one).
    // Entry e of an item is channel run A + e/2 (even e) or run B + e/2 (odd).
    // Lanes past the fold items load an in-range run too (the run depends on
    // the item modulo a head's items): no load sits under a branch.
    const uint32_t* km = kmeta + (int64_t)((ch * kChunk) / G) * D;
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      uint32_t w[8];
      load_run<8>(km + kmofs[i], w);
      r.kmA[i] = make_uint4(w[0], w[2], w[4], w[6]);
      r.kmB[i] = make_uint4(w[1], w[3], w[5], w[7]);
    }
  }

  // q' = q * 2^-E * key scale (hi/lo fp16 fragments in LDS) and beta' =
  // q * 2^-E . key min, for the key group starting in this chunk.
  __device__ __forceinline__ void fold(const R& r) {
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      const int it = fitem[i];
      float bpart = 0.0f;
      // (when the items fill the wave exactly the test is compile-time true)
      if (C::ITEMS % 64 == 0 || it < C::ITEMS) {
        const int h = it / IPH, rr = it % IPH, gg = rr / KC, kc = rr % KC;
        const float4 qa = *reinterpret_cast<const float4*>(qfs + h * D + kmoff[i][0]);
        const float4 qb = *reinterpret_cast<const float4*>(qfs + h * D + kmoff[i][1]);
        const float qA[4] = {qa.x, qa.y, qa.z, qa.w}, qBv[4] = {qb.x, qb.y, qb.z, qb.w};
        const uint32_t mA[4] = {r.kmA[i].x, r.kmA[i].y, r.kmA[i].z, r.kmA[i].w};
        const uint32_t mB[4] = {r.kmB[i].x, r.kmB[i].y, r.kmB[i].z, r.kmB[i].w};
        uint32_t hp[4], lp[4];
        float bodd = 0.0f;  // odd channels (their q' carries kKeyOddQ)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split2(mul_lo(qA[e], mA[e]), mul_lo(qBv[e], mB[e]), m1, hp[e], lp[e]);
          if (e & 1) {
            bodd = mul_hi(qA[e], mA[e], bodd);
            bodd = mul_hi(qBv[e], mB[e], bodd);
          } else {
            bpart = mul_hi(qA[e], mA[e], bpart);
            bpart = mul_hi(qBv[e], mB[e], bpart);
          }
        }
        // beta = q . min with the channel factors taken back out
        bpart = __builtin_fmaf(bodd, 1.0f / kKeyOddQ<BK>, bpart * (1.0f / kKeyEvenQ<BK>));
        qB[((0 * GQ + h) * 4 + gg) * KC + kc] = make_uint4(hp[0], hp[1], hp[2], hp[3]);
        qB[((1 * GQ + h) * 4 + gg) * KC + kc] = make_uint4(lp[0], lp[1], lp[2], lp[3]);
      }
      bpart = group_sum<IPH>(bpart);
      // every lane stores (no branch): a head's first item lane its beta, the
      // others a spare slot
      const bool lead = (C::ITEMS % 64 == 0 || it < C::ITEMS) && (it % IPH) == 0;
      beta_l[lead ? it / IPH : GQ] = bpart;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int p = 0; p < KP; ++p)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int part = kColSplit ? (slot & 1) : p;
        const uint4 v = qB[((part * GQ + hcol) * 4 + lg) * KC + kc];
        bq[p][kc][0] = v.x; bq[p][kc][1] = v.y; bq[p][kc][2] = v.z; bq[p][kc][3] = v.w;
      }
    beta_c = beta_l[hcol] * bscale;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Online softmax over a chunk's scores (exact running max; rescale only
  // when it grows).  Each lane tests its own 8 scores; the cross-lane maximum
  // is only formed on the (rare) path where some lane sees a larger score.
  // kPacked: weights carry the value classes' factors (q < 2: kValEven,
  // q >= 2: kValOdd) and their sums are kept per class; otherwise plain.
  template <bool kPacked>
  __device__ __forceinline__ void softmax(const float (&s)[2][4], float (&p)[2][4]) {
    float cm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    if (__any(cm > m_run)) {
      cm = xor_max(cm, 16);
      cm = xor_max(cm, 32);
      const float m_new = fmaxf(m_run, cm);
      const float a = exp2_hw(m_run - m_new);
      m_run = m_new;
      m_even = m_new - kValEvenLog2<BV>;
      m_odd = m_new - kValOddLog2;
      l_run *= a;
      l_odd *= a;
#pragma unroll
      for (int n = 0; n < NT; ++n) oacc[n] *= a;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        bias[f] *= a;
        bias_odd[f] *= a;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (kPacked) {
          p[u][q] = exp2_hw(s[u][q] - (q < 2 ? m_even : m_odd));
          if (q < 2)
            l_run += p[u][q];
          else
            l_odd += p[u][q];
        } else {
          p[u][q] = exp2_hw(s[u][q] - m_run);
          l_run += p[u][q];
        }
      }
  }

  // Packed accumulation to real scale (codes were fp16 numbers c * 2^-24,
  // pairs carry kValEven) with its value-min term added; class sums folded.
  // Afterwards the state is plain (as the residual path needs).
  __device__ __forceinline__ void to_real() {
    // the value-min term is summed over the four lane groups (token subsets)
    float btot[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const float bt = __builtin_fmaf(bias_odd[f], 1.0f / kValOdd<BV>,
                                      bias[f] * (1.0f / kValEven<BV>));
      btot[f] = xor_sum(xor_sum(bt, 16), 32);
      bias[f] = 0.0f;
      bias_odd[f] = 0.0f;
    }
    constexpr float oscale = 16777216.0f / kValEven<BV>;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float bsum = btot[C::gam(n) / SL];
#pragma unroll
      for (int q = 0; q < 4; ++q) oacc[n][q] = __builtin_fmaf(oacc[n][q], oscale, bsum);
    }
    l_run = __builtin_fmaf(l_odd, 1.0f / kValOdd<BV>, l_run * (1.0f / kValEven<BV>));
    l_odd = 0.0f;
    m_even = m_run;
    m_odd = m_run;
  }

  // Switch to the residual window: bring the packed accumulation to real scale
  // (codes were fp16 numbers c * 2^-24) with its value-min term added, and set
  // the key-side B fragments to q * 2^-E in natural channel order (element j of
  // lane group g, k-chunk kc = channel 32 kc + 8 g + j), hi or lo part.
  __device__ __forceinline__ void enter_residual() {
    to_real();
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const float4 qa = *reinterpret_cast<const float4*>(qfs + hcol * D + 32 * kc + 8 * lg);
      const float4 qb = *reinterpret_cast<const float4*>(qfs + hcol * D + 32 * kc + 8 * lg + 4);
      // channel 32 kc + 8 lg + j: parity of j; the key-side factors come out
      constexpr float ue = 1.0f / kKeyEvenQ<BK>, uo = 1.0f / kKeyOddQ<BK>;
      const float qv[8] = {qa.x * ue, qa.y * uo, qa.z * ue, qa.w * uo,
                           qb.x * ue, qb.y * uo, qb.z * ue, qb.w * uo};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t hi, lo;
        split2(qv[2 * i], qv[2 * i + 1], m1, hi, lo);
        if constexpr (kColSplit) {
          bq[0][kc][i] = (slot & 1) ? lo : hi;
        } else {
          bq[0][kc][i] = hi;
          bq[1][kc][i] = lo;
        }
      }
    }
    cur_group = -1;
  }

  // Residual chunk: fp16 tokens t0 + [0, 32) of the window (those >= n_tok
  // masked).  Keys come straight from the window's slot rows; values are
  // stored in the value consumer order, so tile n's A operand is one 16-byte
  // load per lane (slots past n_tok are zeroed in registers: their weight is
  // 0, and the window may hold anything there).
  __device__ __forceinline__ void process_residual(int t0, int n_tok, int R,
                                                   const uint16_t* kres,
                                                   const uint16_t* vres) {
    // value operands first: their loads overlap the score MFMAs
    const uint4* vq = reinterpret_cast<const uint4*>(vres) +
                      (int64_t)((t0 % R) / kChunk) * (D / 16) * 64 + lane;
    uint4 va[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) va[n] = vq[n * 64];
    uint32_t vmask[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 8 * lg + 2 * i;
      vmask[i] = (t < n_tok ? 0x0000ffffu : 0u) | (t + 1 < n_tok ? 0xffff0000u : 0u);
    }
    // scores: tile u row r = token key_row_token(u, r)
    const float kscale_r = bscale;  // keys are real fp16 values here
    float s[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tin = t0 + key_row_token(u, col);
      const int slot_in = (tin < n_tok ? tin : n_tok - 1) % R;
      const uint4* krow = reinterpret_cast<const uint4*>(kres + (int64_t)slot_in * D);
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 kv = krow[4 * kc + lg];
        const uint32_t a[4] = {kv.x, kv.y, kv.z, kv.w};
        acc = mfma(a, bq[0][kc], acc);
        if constexpr (!kColSplit) acc = mfma(a, bq[1][kc], acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x = acc[q];
        if constexpr (kColSplit) {
          x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                   __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
        }
        const bool valid = t0 + 8 * lg + 4 * u + q < n_tok;
        s[u][q] = valid ? x * kscale_r : kNegInf;
      }
    }
    float p[2][4];
    softmax<false>(s, p);
    uint32_t bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      split2(p[i >> 1][2 * (i & 1)], p[i >> 1][2 * (i & 1) + 1], m1, bh[i], bl[i]);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint32_t a[4] = {va[n].x & vmask[0], va[n].y & vmask[1], va[n].z & vmask[2],
                             va[n].w & vmask[3]};
      oacc[n] = mfma(a, bh, oacc[n]);
      oacc[n] = mfma(a, bl, oacc[n]);
    }
  }

  __device__ __forceinline__ void process(int ch, const R& r) {
    if constexpr (G == kChunk) {
      fold(r);  // every chunk is a key group: no branch, so the fold can be
                // scheduled against the previous chunk's value products
    } else {
      const int grp = (ch * kChunk) / G;
      if (grp != cur_group) {
        cur_group = grp;
        fold(r);
      }
    }
    // scores: s = 2^(E+24) * (codes x q') + beta
    float s[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t a[KC][4];
      unpack_keys<D, BK>(r.kw[u], a);
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        acc = mfma(a[kc], bq[0][kc], acc);
        if constexpr (!kColSplit) acc = mfma(a[kc], bq[1][kc], acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x = acc[q];
        if constexpr (kColSplit) {
          // hi column + lo column (lanes col and col ^ 1 of a quad)
          x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                   __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
        }
        s[u][q] = __builtin_fmaf(x, kscale, beta_c);
      }
    }
    float p[2][4];
    softmax<true>(s, p);
    // weighted value sum
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // elements 2i (run A) and 2i+1 (run B) = score tile i/2, rows 2(i%2), +1;
        // odd i is the odd class
        const float pa = p[i >> 1][2 * (i & 1)], pb = p[i >> 1][2 * (i & 1) + 1];
        split2(mul_lo(pa, r.vmA[f][i]), mul_lo(pb, r.vmB[f][i]), m1, bh[i], bl[i]);
        float& bacc = (i & 1) ? bias_odd[f] : bias[f];
        bacc = mul_hi(pa, r.vmA[f][i], bacc);
        bacc = mul_hi(pb, r.vmB[f][i], bacc);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (C::gam(n) / SL != f) continue;  // compile-time
        uint32_t a[4];
        if constexpr (BV == 4) {
          // pair e: (w >> 8 (e/2)) masked at bits 4 (e%2)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a[e] = (r.vw[n] >> (8 * (e >> 1))) & ((e & 1) ? 0x00F000F0u : 0x000F000Fu);
        } else {
          // tile parity selects the byte; pair e: (w' >> 4 (e/2)) at bits 2 (e%2)
          const uint32_t x = r.vw[n >> 1] >> (8 * (n & 1));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a[e] = (x >> (4 * (e >> 1))) & ((e & 1) ? 0x000C000Cu : 0x00030003u);
        }
        oacc[n] = mfma(a, bh, oacc[n]);
        oacc[n] = mfma(a, bl, oacc[n]);
      }
    }
  }
};

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
constexpr int kPartPad = 4;  // partial row = D values, max, sum, 2 pad floats

struct SeqWork {
  int n;   // tokens (0 for an invalid length)
  int nq;  // packed chunks per KV head
  int nr;  // residual chunks per KV head
  int w;   // work units per KV head
};

__device__ __forceinline__ SeqWork seq_work_of(const DecodeLaunch& L, int n) {
  SeqWork sw{0, 0, 0, 0};
  if (n <= 0 || n > L.g.C || n > L.max_seq_len) return sw;
  const int lq = packed_len(n, L.g.R);
  sw.n = n;
  sw.nq = lq / kChunk;
  sw.nr = (n - lq + kChunk - 1) / kChunk;
  sw.w = sw.nq + sw.nr * L.rw;
  return sw;
}

__device__ __forceinline__ SeqWork seq_work(const DecodeLaunch& L, int b) {
  return seq_work_of(L, L.seq_lens[b]);
}

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
// uniform: every length equals max_seq_len.
struct BatchWork {
  int c, inc, head_total, total;
  bool uniform;
};

__device__ __forceinline__ BatchWork batch_work(const DecodeLaunch& L, int lane) {
  BatchWork bw;
  const int n = lane < L.g.B ? L.seq_lens[lane] : L.max_seq_len;
  bw.c = lane < L.g.B ? seq_work_of(L, n).w * L.g.Hkv : 0;
  bw.inc = wave_scan_incl(bw.c);
  bw.head_total = __builtin_amdgcn_readlane(bw.inc, 63);
  bw.total = bw.head_total;
  bw.uniform = __ballot(n != L.max_seq_len) == 0;
  for (int b0 = 64; b0 < L.g.B; b0 += 64) {  // batches beyond 64 sequences
    const int nb = b0 + lane < L.g.B ? L.seq_lens[b0 + lane] : L.max_seq_len;
    int s = b0 + lane < L.g.B ? seq_work_of(L, nb).w * L.g.Hkv : 0;
    s = wave_scan_incl(s);
    bw.total += __builtin_amdgcn_readlane(s, 63);
    bw.uniform = bw.uniform && __ballot(nb != L.max_seq_len) == 0;
  }
  return bw;
}

// Sequence b holding flat work unit x < total, and base = Hkv * (work of
// sequences < b).
__device__ __forceinline__ void wave_find_seq(const DecodeLaunch& L, const BatchWork& bw,
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
    const int c = (b < L.g.B) ? seq_work(L, b).w * L.g.Hkv : 0;
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

template <int D, int BK, int BV, int GQ, int NG>
constexpr int kWaveSmem = GQ * D * 4 + Cfg<D, BK, BV, GQ, NG>::kWaveLds;

// Packed chunks [pc0, pc1) and residual chunks [rk0, rk1) of unit work
// starting at xu that fall in the work range [x0, x1).
struct SegRange {
  int pc0, pc1, rk0, rk1;
};

__device__ __forceinline__ SegRange seg_range(const DecodeLaunch& L, const SeqWork& sw, int xu,
                                              int x0, int x1) {
  SegRange r;
  r.pc0 = max(x0, xu) - xu;
  r.pc1 = min(x1, xu + sw.nq) - xu;
  const int d0 = x0 - xu - sw.nq, d1 = x1 - xu - sw.nq;
  r.rk0 = d0 <= 0 ? 0 : (d0 + L.rw - 1) / L.rw;
  r.rk1 = min(sw.nr, d1 <= 0 ? 0 : (d1 + L.rw - 1) / L.rw);
  return r;
}

// Sets up the wave for unit (b, hkv) and issues the loads of the range's first
// packed chunk into ra (before anything else, so that their latency overlaps
// the query's).
template <int D, int BK, int BV, int GQ, int NG>
__device__ __forceinline__ void seg_begin(const DecodeLaunch& L, int64_t unit, const SegRange& r,
                                          char* smem, int lane, PackedWave<D, BK, BV, GQ, NG>& w,
                                          Raw<D, BK, BV, GQ, NG>& ra) {
  using C = Cfg<D, BK, BV, GQ, NG>;
  const Geom& g = L.g;
  char* wl = smem + GQ * D * 4;
  w.kcodes = L.cache.k_codes + unit * g.C * C::WR;
  w.kmeta = reinterpret_cast<const uint32_t*>(L.cache.k_meta) + unit * (g.C / C::G) * D;
  w.vcodes = L.cache.v_codes + unit * (g.C / kVBlock) * D * BV;
  w.vmeta = reinterpret_cast<const uint32_t*>(L.cache.v_meta) +
            unit * (g.C / kVBlock) * NG * kVBlock;
  w.qfs = reinterpret_cast<float*>(smem);
  w.qB = reinterpret_cast<uint4*>(wl);
  w.beta_l = reinterpret_cast<float*>(wl + C::kQB);
  w.init(lane);
  if (r.pc0 < r.pc1) w.load(r.pc0, ra);
}

// Runs the range of unit (b, hkv) -> partial p, seg_begin having been done.
template <int D, int BK, int BV, int GQ, int NG>
__device__ void seg_run(const DecodeLaunch& L, int b, int hkv, const SeqWork& sw,
                        const SegRange& r, int p, char* smem, int lane,
                        PackedWave<D, BK, BV, GQ, NG>& w, Raw<D, BK, BV, GQ, NG>& ra) {
  using C = Cfg<D, BK, BV, GQ, NG>;
  using R = Raw<D, BK, BV, GQ, NG>;
  constexpr int NT = C::NT, SL = C::SL;
  constexpr int QPH = D / 64;  // query values per lane and head
  constexpr int DP = D + kPartPad;
  const Geom& g = L.g;
  const int64_t unit = (int64_t)b * g.Hkv + hkv;
  float* part_base = L.ws + (int64_t)p * GQ * DP;
  float* qfs = reinterpret_cast<float*>(smem);  // [GQ][D] q * 2^-E_h
  const int pc0 = r.pc0, pc1 = r.pc1, rk0 = r.rk0, rk1 = r.rk1;
  R rb;
  // query of the unit's GQ heads; per-head exponent E with max|q| < 2^E so
  // that q * 2^-E * scale fits fp16
  const uint16_t* qg = L.q + ((int64_t)b * g.Hq + hkv * GQ) * D;
  int eh[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float qv[QPH];
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < QPH; ++k) {
      qv[k] = h2f(qg[h * D + lane + 64 * k]) * L.scale_log2;
      mx = fmaxf(mx, fabsf(qv[k]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = xor_max(mx, off);
    int e = 0;
    if (mx > 0.0f) (void)frexpf(mx, &e);
    eh[h] = e;
#pragma unroll
    for (int k = 0; k < QPH; ++k)  // channel lane + 64 k has the parity of lane
      qfs[h * D + lane + 64 * k] =
          ldexpf(qv[k], -e) * ((lane & 1) ? kKeyOddQ<BK> : kKeyEvenQ<BK>);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  int e_mine = 0;
#pragma unroll
  for (int h = 0; h < GQ; ++h)
    if (w.hcol == h) e_mine = eh[h];
  // codes are the fp16 numbers c * 2^-24, pairs carry the key-side factor
  w.kscale = ldexpf(1.0f, e_mine + 24 - kKeyAccLog2<BK>);
  w.bscale = ldexpf(1.0f, e_mine);

  if (pc0 < pc1) {
    // two chunk buffers: the next chunk's loads are in flight while one is
    // used (a deeper ring measured no faster).  Prefetches past the last
    // chunk re-load that chunk (always in bounds) instead of being skipped,
    // so no load sits under a branch.
    const int last = pc1 - 1;
    int ch = pc0;
    for (; ch < last; ch += 2) {  // pairs; ra holds chunk ch on entry
      w.load(ch + 1, rb);
      w.process(ch, ra);
      w.load(min(ch + 2, last), ra);
      w.process(ch + 1, rb);
    }
    if (ch == last) w.process(ch, ra);  // odd count: the last chunk is in ra
  }
  const bool resid = rk0 < rk1;
  if (resid) {
    w.enter_residual();
    const uint16_t* kres = L.cache.k_res + unit * g.R * D;
    const uint16_t* vres = L.cache.v_res + unit * g.R * D;
    const int lq = sw.nq * kChunk;
    for (int k = rk0; k < rk1; ++k) w.process_residual(lq + k * kChunk, sw.n, g.R, kres, vres);
  }

  // partial: O (value-min term included), max, sum of this wave's tokens
  if (!resid) w.to_real();
  float l_run = w.l_run;
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);
  float* part = part_base + w.hcol * DP;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int gm = C::gam(n);
    if (gm % SL != w.slot) continue;
    const float4 v = make_float4(w.oacc[n][0], w.oacc[n][1], w.oacc[n][2], w.oacc[n][3]);
    *reinterpret_cast<float4*>(part + 16 * n + 4 * w.lg) = v;
  }
  if (w.lg == 0 && w.slot == 0) {
    part[D] = w.m_run;
    part[D + 1] = l_run;
  }
  // the next segment of this wave rewrites the LDS buffers
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// The part of unit (b, hkv) in work range [x0, x1) -> partial p.  xu = first
// work unit of the unit.
template <int D, int BK, int BV, int GQ, int NG>
__device__ void unit_segment(const DecodeLaunch& L, int b, int hkv, const SeqWork& sw,
                             int xu, int x0, int x1, int p, char* smem, int lane) {
  constexpr int DP = D + kPartPad;
  const SegRange r = seg_range(L, sw, xu, x0, x1);
  if (r.pc0 >= r.pc1 && r.rk0 >= r.rk1) {  // only part of a residual chunk's weight
    // an empty partial: zero sums, max -inf (weight 0 in the merge)
    float* part_base = L.ws + (int64_t)p * GQ * DP;
    for (int i = lane; i < GQ * DP; i += 64) {
      const int c = i % DP;
      part_base[i] = (c == D) ? kNegInf : 0.0f;
    }
    return;
  }
  PackedWave<D, BK, BV, GQ, NG> w;
  Raw<D, BK, BV, GQ, NG> ra;
  seg_begin<D, BK, BV, GQ, NG>(L, (int64_t)b * L.g.Hkv + hkv, r, smem, lane, w, ra);
  seg_run<D, BK, BV, GQ, NG>(L, b, hkv, sw, r, p, smem, lane, w, ra);
}

// One wave per workgroup; grid = the number of worker waves.
template <int D, int BK, int BV, int GQ, int NG>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeLaunch L) {
  __shared__ __attribute__((aligned(16))) char smem[kWaveSmem<D, BK, BV, GQ, NG>];
  const int lane = threadIdx.x;
  const int w = blockIdx.x, nw = gridDim.x;
  // Speculation: if every length equals max_seq_len (a uniform batch), the
  // work layout is plain arithmetic, so the first segment's first chunk can
  // be requested before the lengths are read.  The loads are in bounds
  // whatever the lengths; they are used only if the lengths confirm it.
  using PW = PackedWave<D, BK, BV, GQ, NG>;
  using RW = Raw<D, BK, BV, GQ, NG>;
  const SeqWork ss = seq_work_of(L, L.max_seq_len);
  const int per_seq = ss.w * L.g.Hkv;
  const int cpw_s = (per_seq * L.g.B + nw - 1) / nw;
  const int x0_s = w * cpw_s, x1_s = min(per_seq * L.g.B, x0_s + cpw_s);
  bool spec = ss.w > 0 && x0_s < x1_s;
  int b_s = 0, hkv_s = 0, xu_s = 0;
  SegRange r_s{0, 0, 0, 0};
  if (spec) {
    b_s = x0_s / per_seq;
    hkv_s = (x0_s - b_s * per_seq) / ss.w;
    xu_s = b_s * per_seq + hkv_s * ss.w;
    r_s = seg_range(L, ss, xu_s, x0_s, x1_s);
    spec = r_s.pc0 < r_s.pc1;
  }
  PW ws;
  RW ra_s;
  if (spec) seg_begin<D, BK, BV, GQ, NG>(L, (int64_t)b_s * L.g.Hkv + hkv_s, r_s, smem, lane, ws, ra_s);

  const BatchWork bw = batch_work(L, lane);  // one read of the lengths
  const int total = bw.total;
  const int cpw = (total + nw - 1) / nw;
  const int x0 = w * cpw;
  const int x1 = min(total, x0 + cpw);
  int x = x0;
  if (spec && bw.uniform) {  // confirmed: the speculative first segment stands
    seg_run<D, BK, BV, GQ, NG>(L, b_s, hkv_s, ss, r_s, w + b_s * L.g.Hkv + hkv_s, smem, lane,
                               ws, ra_s);
    x = xu_s + ss.w;
  }
  while (x < x1) {
    int b, base;
    wave_find_seq(L, bw, lane, x, b, base);
    b = __builtin_amdgcn_readfirstlane(b);
    base = __builtin_amdgcn_readfirstlane(base);
    const SeqWork sw = seq_work(L, b);
    const int hkv = (x - base) / sw.w;
    const int xu = base + hkv * sw.w;
    unit_segment<D, BK, BV, GQ, NG>(L, b, hkv, sw, xu, x0, x1, w + b * L.g.Hkv + hkv, smem,
                                    lane);
    x = xu + sw.w;
  }
}

// One workgroup per (KV head, sequence): merges the partials of the unit and
// writes its GQ outputs:
//   M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L.
// The unit's partials are contiguous (indices w + u for consecutive waves w).
// Each thread owns one float4 of the output and a 1/P share of the partials
// and merges them as a stream (running max, rescale when it grows), so the
// (m, l, o) loads of a partial do not wait for any reduction; the P shares are
// then merged through LDS.  Empty partials (m = -inf) carry weight 0.
template <int D, int GQ>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeLaunch L) {
  constexpr int DP = D + kPartPad;
  constexpr int NO = GQ * D / 4;                          // float4 outputs of the unit
  constexpr int P = NO >= kThreads ? 1 : kThreads / NO;   // partial shares per output
  constexpr int OPT = NO >= kThreads ? NO / kThreads : 1;  // outputs per thread
  constexpr int U = 4;                                     // partials in flight per thread
  static_assert(NO % kThreads == 0 || kThreads % NO == 0, "outputs tile the workgroup");
  __shared__ int red[2 * kThreads / 64];
  __shared__ float4 s_o[kThreads];
  __shared__ float2 s_ml[kThreads];
  const Geom& g = L.g;
  const int hkv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t out0 = ((int64_t)b * g.Hq + hkv * GQ) * D;
  const int n = L.seq_lens[b];
  if (n < 0 || n > g.C || n > L.max_seq_len) {
    for (int i = tid; i < GQ * D; i += kThreads) L.out[out0 + i] = 0x7e00;  // NaN
    return;
  }
  if (n == 0) {
    for (int i = tid; i < GQ * D; i += kThreads) L.out[out0 + i] = 0;
    return;
  }
  // flat position of this unit's work
  int tot = 0, pre = 0;
  for (int bb = tid; bb < g.B; bb += kThreads) {
    const int c = seq_work(L, bb).w;
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
  const SeqWork sw = seq_work(L, b);
  const int xu = pre * g.Hkv + hkv * sw.w;
  const int cpw = (total + L.n_workers - 1) / L.n_workers;
  const int w_first = xu / cpw, w_last = (xu + sw.w - 1) / cpw;
  const int S = w_last - w_first + 1;
  const float* base = L.ws + (int64_t)(w_first + b * g.Hkv + hkv) * GQ * DP;
  const int share = (P > 1) ? tid / NO : 0;

#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    const int t = (P > 1) ? tid % NO : tid + j * kThreads;
    const int oh = t / (D / 4), oc = (t % (D / 4)) * 4;
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
    if (share == 0) {
      const float inv = 1.0f / Ls;
      const int64_t o = out0 + oh * D + oc;
      L.out[o + 0] = f2h(O.x * inv);
      L.out[o + 1] = f2h(O.y * inv);
      L.out[o + 2] = f2h(O.z * inv);
      L.out[o + 3] = f2h(O.w * inv);
    }
  }
}

// Worker waves the partial kernel of this instantiation is launched with:
// resident waves per compute unit (from the kernel's resources) x CUs, cached
// per device.
template <int D, int BK, int BV, int GQ, int NG>
hipError_t workers_of(int cus, int* out) {
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return hipSuccess;
  }
  int nb = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &nb, decode_partial_kernel<D, BK, BV, GQ, NG>, 64, 0);
  if (e != hipSuccess) return e;
  if (nb < 1) nb = 1;
  const int w = nb * cus;
  if (dev >= 0 && dev < 64) cache[dev] = w;
  *out = w;
  return hipSuccess;
}

// Op: 0 = launch the partial kernel, 1 = query its worker count.
template <int D, int BK, int BV, int GQ, int NG>
hipError_t run(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  if (op == 1) return workers_of<D, BK, BV, GQ, NG>(cus, workers);
  decode_partial_kernel<D, BK, BV, GQ, NG><<<dim3(L.n_workers), 64, 0, st>>>(L);
  return hipGetLastError();
}

template <int D, int BK, int BV, int GQ>
hipError_t dispatch_ng(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  switch (D / L.g.G) {
    case 1: return run<D, BK, BV, GQ, 1>(L, op, cus, workers, st);
    case 2: return run<D, BK, BV, GQ, 2>(L, op, cus, workers, st);
    case 4:
      if constexpr (D == 128) return run<D, BK, BV, GQ, 4>(L, op, cus, workers, st);
      [[fallthrough]];
    default: return hipErrorInvalidValue;
  }
}

template <int D, int BK, int BV>
hipError_t dispatch_gq(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  switch (L.g.Hq / L.g.Hkv) {
    case 1: return dispatch_ng<D, BK, BV, 1>(L, op, cus, workers, st);
    case 2: return dispatch_ng<D, BK, BV, 2>(L, op, cus, workers, st);
    case 4: return dispatch_ng<D, BK, BV, 4>(L, op, cus, workers, st);
    case 8: return dispatch_ng<D, BK, BV, 8>(L, op, cus, workers, st);
    case 16: return dispatch_ng<D, BK, BV, 16>(L, op, cus, workers, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t dispatch_bits(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  const int bk = L.g.bK, bv = L.g.bV;
  if (bk == 2 && bv == 2) return dispatch_gq<D, 2, 2>(L, op, cus, workers, st);
  if (bk == 2 && bv == 4) return dispatch_gq<D, 2, 4>(L, op, cus, workers, st);
  if (bk == 4 && bv == 2) return dispatch_gq<D, 4, 2>(L, op, cus, workers, st);
  return dispatch_gq<D, 4, 4>(L, op, cus, workers, st);
}

hipError_t dispatch(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  return L.g.D == 64 ? dispatch_bits<64>(L, op, cus, workers, st)
                     : dispatch_bits<128>(L, op, cus, workers, st);
}

template <int D>
hipError_t combine_gq(const DecodeLaunch& L, hipStream_t st) {
  dim3 grid(L.g.Hkv, L.g.B);
  switch (L.g.Hq / L.g.Hkv) {
    case 1: decode_combine_kernel<D, 1><<<grid, kThreads, 0, st>>>(L); break;
    case 2: decode_combine_kernel<D, 2><<<grid, kThreads, 0, st>>>(L); break;
    case 4: decode_combine_kernel<D, 4><<<grid, kThreads, 0, st>>>(L); break;
    case 8: decode_combine_kernel<D, 8><<<grid, kThreads, 0, st>>>(L); break;
    case 16: decode_combine_kernel<D, 16><<<grid, kThreads, 0, st>>>(L); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t decode_workers(const Geom& g, int cus, int* workers) {
  DecodeLaunch L{};
  L.g = g;
  return dispatch(L, 1, cus, workers, nullptr);
}

hipError_t launch_decode_partial(const DecodeLaunch& L, hipStream_t st) {
  return dispatch(L, 0, 0, nullptr, st);
}

hipError_t launch_decode_combine(const DecodeLaunch& L, hipStream_t st) {
  return L.g.D == 64 ? combine_gq<64>(L, st) : combine_gq<128>(L, st);
}

}  // namespace kvq
