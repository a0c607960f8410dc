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
// Work decomposition: one workgroup (4 waves) per (split, KV head, sequence)
// over packed tokens; the GQA query heads of the KV head share every load.
// Each wave runs an online softmax over a contiguous run of 32-token chunks;
// the 4 wave states merge in LDS into one partial (max, sum, weighted values)
// per query head.  One extra workgroup per (KV head, sequence) covers the
// residual window with plain fp32 arithmetic.  The combine kernel merges
// partials: M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i-M) / L.
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
// hi/lo fp16 split of (a, b): a ~= hi.x + lo.x to ~2^-21 relative.  The
// remainders a - hi.x are exact fp32 subtractions, written as fmas of the fp16
// half so that the compiler fuses the conversion (v_fma_mix_f32).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pk_rtz(a, b);
  const h2 hh = __builtin_bit_cast(h2, hi);
  lo = pk_rtz(__builtin_fmaf((float)hh[0], -1.0f, a), __builtin_fmaf((float)hh[1], -1.0f, b));
}

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
// Token and channel permutations of the MFMA operands.
//
// Value side: the A operand of lane (channel c, lane group g) holds 8 codes of
// channel c; element j is the chunk token tok_v(g, j).  It comes straight from
// the packed value word(s): 4-bit words hold tokens 8w..8w+7 (nibble e = token
// 8w+e), and one mask of (w >> 4e) with 0x000F000F yields tokens 8g+e and
// 8g+4+e as an fp16 pair; 2-bit words hold 16 tokens and (w >> 2s) & 0x00030003
// yields tokens s and s+8 of the word.
// Key side: tile u (16 tokens) row r is token tok_v(r / 4, 4u + r % 4), so that
// the score tile's output registers (lane group g, register r' of tile u) hold
// exactly the tokens tok_v(g, 4u + r') that the value side wants in element
// 4u + r' of its B operand: the scores never leave their lanes.
// ---------------------------------------------------------------------------
template <int BV>
__device__ __forceinline__ constexpr int tok_v(int g, int j) {
  const int e = j >> 1, par = j & 1;
  return BV == 4 ? 8 * g + 4 * par + e : 16 * (g >> 1) + 8 * par + 4 * (g & 1) + e;
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

template <int D, int BK>
__device__ __forceinline__ void unpack_keys(const uint32_t (&w)[kKW<D, BK>],
                                            uint32_t (&a)[D / 32][4]) {
  if constexpr (BK == 2) {
#pragma unroll
    for (int wi = 0; wi < kKW<D, BK>; ++wi)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int ri = 8 * wi + s;
        a[ri >> 2][ri & 3] = (w[wi] >> (2 * s)) & 0x00030003u;
      }
  } else {
#pragma unroll
    for (int wi = 0; wi < kKW<D, BK>; ++wi)
#pragma unroll
      for (int s = 0; s < 4; ++s) a[wi][s] = (w[wi] >> (4 * s)) & 0x000F000Fu;
  }
}

template <int KW>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[KW]) {
  if constexpr (KW == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (KW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = p[0];
  }
}

// ---------------------------------------------------------------------------
// Residual window (fp16 tokens [t_begin, t_end)), plain fp32 arithmetic over
// the whole workgroup: 8 lanes per token for scores, one lane per (channel,
// head group) for the weighted value sum.  Writes partial `part_idx`.
// ---------------------------------------------------------------------------
template <int D, int GQ>
__device__ void residual_partial(const DecodeLaunch& L, int b, int hkv, int t_begin,
                                 int t_end, int part_idx, float* smem) {
  constexpr int kTPT = 8, CPT = D / kTPT;
  constexpr int TPC = kThreads / D, HPT = (GQ + TPC - 1) / TPC;
  const Geom& g = L.g;
  float* qf = smem;                      // [GQ][D]
  float* sc = qf + GQ * D;               // [GQ][kChunk]
  float* m_run = sc + GQ * kChunk;       // [GQ]
  float* l_run = m_run + GQ;
  float* alpha = l_run + GQ;
  const int tid = threadIdx.x;
  const int64_t unit = (int64_t)b * g.Hkv + hkv;
  for (int i = tid; i < GQ * D; i += kThreads)
    qf[i] = h2f(L.q[((int64_t)b * g.Hq + hkv * GQ) * D + i]) * L.scale_log2;
  if (tid < GQ) {
    m_run[tid] = kNegInf;
    l_run[tid] = 0.0f;
  }
  const int c_v = tid % D, hg = tid / D;
  float o[HPT];
#pragma unroll
  for (int i = 0; i < HPT; ++i) o[i] = 0.0f;
  __syncthreads();
  const uint16_t* kr = L.cache.k_res + unit * g.R * D;
  const uint16_t* vr = L.cache.v_res + unit * g.R * D;
  const int tok = tid / kTPT, sl = tid % kTPT;
  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int t = t0 + tok;
    const bool valid = t < t_end;
    float acc[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) acc[h] = 0.0f;
    if (valid) {
      const uint16_t* krow = kr + (int64_t)(t % g.R) * D + sl * CPT;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const float kv = h2f(krow[i]);
#pragma unroll
        for (int h = 0; h < GQ; ++h) acc[h] += qf[h * D + sl * CPT + i] * kv;
      }
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      acc[h] = xor_sum(acc[h], 1);
      acc[h] = xor_sum(acc[h], 2);
      acc[h] = xor_sum(acc[h], 4);
    }
    if (sl == 0) {
#pragma unroll
      for (int h = 0; h < GQ; ++h) sc[h * kChunk + tok] = valid ? acc[h] : kNegInf;
    }
    __syncthreads();
    for (int i = tid; i < GQ * kChunk; i += kThreads) {
      const int h = i / kChunk, tk = i % kChunk;
      const float x = sc[i];
      float cmax = x;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) cmax = xor_max(cmax, off);
      const float m_old = m_run[h];
      const float m_new = fmaxf(m_old, cmax);
      const float p = exp2f(x - m_new);
      float psum = p;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) psum = xor_sum(psum, off);
      sc[i] = p;
      if (tk == 0) {
        const float a = exp2f(m_old - m_new);
        alpha[h] = a;
        l_run[h] = l_run[h] * a + psum;
        m_run[h] = m_new;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int h = hg * HPT + i;
      if (h < GQ) o[i] *= alpha[h];
    }
    for (int tk = 0; tk < kChunk && t0 + tk < t_end; ++tk) {
      const float vv = h2f(vr[(int64_t)((t0 + tk) % g.R) * D + c_v]);
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int h = hg * HPT + i;
        if (h < GQ) o[i] += sc[h * kChunk + tk] * vv;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    const int h = hg * HPT + i;
    if (h >= GQ) continue;
    const int64_t bh = (int64_t)b * g.Hq + hkv * GQ + h;
    float* part = L.ws + (bh * (L.n_split + 1) + part_idx) * (D + 2);
    part[c_v] = o[i];
    if (c_v == 0) {
      part[D] = m_run[h];
      part[D + 1] = l_run[h];
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
  static constexpr int KW = kKW<D, BK>;           // key words per lane and row
  static constexpr int WR = D * BK / 32;          // words per key row
  static constexpr int SL = 16 / GQ;              // MFMA columns per head
  static constexpr int NF = (NG + SL - 1) / SL;   // value-side B fragments
  static constexpr int IPH = 4 * KC;              // fold items per head
  static constexpr int ITEMS = GQ * IPH;          // fold items per key group
  static constexpr int IPL = (ITEMS + 63) / 64;   // fold items per lane
  // LDS (bytes) per wave: q' fragments [2][GQ][4][KC] x 16 B, beta [GQ]
  static constexpr int kQB = 2 * GQ * 4 * KC * 16;
  static constexpr int kWaveLds = kQB + 16 * ((GQ * 4 + 15) / 16);
  static constexpr int gam(int n) { return (16 * n) / G; }  // group of value tile n
};

// Loads of one 32-token chunk (a lane's share).
template <int D, int BK, int BV, int GQ, int NG>
struct Raw {
  using C = Cfg<D, BK, BV, GQ, NG>;
  uint32_t kw[2][C::KW];              // key code words of score tiles 0, 1
  uint32_t vw[C::NT];                 // value code word per channel tile
  uint32_t vmA[C::NF][4], vmB[C::NF][4];  // value (scale, min) of the B elements
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
  int c_lo, c_hi;
  // lane constants
  int lane, col, lg, hcol, slot;
  int koff[2];
  int voff;
  int vmoff[NF][2];
  int kmoff[IPL][2];
  int fitem[IPL];
  float kscale, bscale;
  // state
  f4 oacc[NT];
  float m_run, l_run;
  float bias[NF];
  uint32_t bq[KP][KC][4];
  uint4 kmA[IPL], kmB[IPL];  // key (scale, min) for the next fold
  float beta_c;
  int cur_group;

  __device__ void init(int lane_) {
    lane = lane_;
    col = lane & 15;
    lg = lane >> 4;
    hcol = col / SL;
    slot = col % SL;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      koff[u] = tok_v<BV>(col >> 2, 4 * u + (col & 3)) * WR + lg * KW;
    voff = col * BV + (BV == 4 ? lg : (lg >> 1));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int gm = (f * SL + slot) % NG;
      vmoff[f][0] = gm * kVBlock + tok_v<BV>(lg, 0);
      vmoff[f][1] = gm * kVBlock + tok_v<BV>(lg, 1);
    }
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      const int it = lane + 64 * i;
      fitem[i] = it;
      const int r = it % IPH, gg = r / KC, kc = r % KC;
      kmoff[i][0] = key_run0<D, BK>(gg, kc);
      kmoff[i][1] = kmoff[i][0] + kKeyOff<BK>;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) oacc[n] = f4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.0f;
#pragma unroll
    for (int f = 0; f < NF; ++f) bias[f] = 0.0f;
    beta_c = 0.0f;
    cur_group = -1;
  }

  __device__ __forceinline__ void load(int ch, R& r) const {
    const uint32_t* kc = kcodes + (int64_t)ch * kChunk * WR;
#pragma unroll
    for (int u = 0; u < 2; ++u) load_words<KW>(kc + koff[u], r.kw[u]);
    const uint32_t* vc = vcodes + (int64_t)ch * D * BV;
#pragma unroll
    for (int n = 0; n < NT; ++n) r.vw[n] = vc[voff + 16 * n * BV];
    const uint32_t* vm = vmeta + (int64_t)ch * NG * kVBlock;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint4 a = *reinterpret_cast<const uint4*>(vm + vmoff[f][0]);
      const uint4 c = *reinterpret_cast<const uint4*>(vm + vmoff[f][1]);
      r.vmA[f][0] = a.x; r.vmA[f][1] = a.y; r.vmA[f][2] = a.z; r.vmA[f][3] = a.w;
      r.vmB[f][0] = c.x; r.vmB[f][1] = c.y; r.vmB[f][2] = c.z; r.vmB[f][3] = c.w;
    }
  }

  // Key meta of group grp for the next fold.
  __device__ __forceinline__ void load_kmeta(int grp) {
    const uint32_t* km = kmeta + (int64_t)grp * D;
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      if (fitem[i] < C::ITEMS) {
        kmA[i] = *reinterpret_cast<const uint4*>(km + kmoff[i][0]);
        kmB[i] = *reinterpret_cast<const uint4*>(km + kmoff[i][1]);
      }
    }
  }

  // q' = q * 2^-E * key scale (hi/lo fp16 fragments in LDS) and beta' =
  // q * 2^-E . key min, for the key group starting in this chunk.
  __device__ __forceinline__ void fold() {
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      const int it = fitem[i];
      float bpart = 0.0f;
      if (it < C::ITEMS) {
        const int h = it / IPH, rr = it % IPH, gg = rr / KC, kc = rr % KC;
        const float4 qa = *reinterpret_cast<const float4*>(qfs + h * D + kmoff[i][0]);
        const float4 qb = *reinterpret_cast<const float4*>(qfs + h * D + kmoff[i][1]);
        const float qA[4] = {qa.x, qa.y, qa.z, qa.w}, qBv[4] = {qb.x, qb.y, qb.z, qb.w};
        const uint32_t mA[4] = {kmA[i].x, kmA[i].y, kmA[i].z, kmA[i].w};
        const uint32_t mB[4] = {kmB[i].x, kmB[i].y, kmB[i].z, kmB[i].w};
        uint32_t hp[4], lp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split2(mul_lo(qA[e], mA[e]), mul_lo(qBv[e], mB[e]), hp[e], lp[e]);
          bpart = mul_hi(qA[e], mA[e], bpart);
          bpart = mul_hi(qBv[e], mB[e], bpart);
        }
        qB[((0 * GQ + h) * 4 + gg) * KC + kc] = make_uint4(hp[0], hp[1], hp[2], hp[3]);
        qB[((1 * GQ + h) * 4 + gg) * KC + kc] = make_uint4(lp[0], lp[1], lp[2], lp[3]);
      }
      bpart = group_sum<IPH>(bpart);
      if (it < C::ITEMS && (it % IPH) == 0) beta_l[it / IPH] = bpart;
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

  __device__ __forceinline__ void process(int ch, const R& r) {
    const int grp = (ch * kChunk) / G;
    if (grp != cur_group) {
      cur_group = grp;
      fold();
    }
    // key meta of the next chunk's group loads while this chunk runs; it is
    // issued unconditionally (the group index is clamped by the caller's
    // chunk range) so the memory counters stay exact on every path.
    load_kmeta(((ch + 1 < c_hi ? ch + 1 : ch) * kChunk) / G);
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
    // online softmax (exact running max; rescale only when it grows).  Each
    // lane tests its own 8 scores; the cross-lane maximum is only formed on
    // the (rare) path where some lane sees a larger score.
    float cm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    if (__any(cm > m_run)) {
      cm = xor_max(cm, 16);
      cm = xor_max(cm, 32);
      const float m_new = fmaxf(m_run, cm);
      const float a = exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= a;
#pragma unroll
      for (int n = 0; n < NT; ++n) oacc[n] *= a;
#pragma unroll
      for (int f = 0; f < NF; ++f) bias[f] *= a;
    }
    float p[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        p[u][q] = exp2f(s[u][q] - m_run);
        l_run += p[u][q];
      }
    // weighted value sum
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // elements 2i (run A) and 2i+1 (run B) = score tile i/2, rows 2(i%2), +1
        const float pa = p[i >> 1][2 * (i & 1)], pb = p[i >> 1][2 * (i & 1) + 1];
        split2(mul_lo(pa, r.vmA[f][i]), mul_lo(pb, r.vmB[f][i]), bh[i], bl[i]);
        bias[f] = mul_hi(pa, r.vmA[f][i], bias[f]);
        bias[f] = mul_hi(pb, r.vmB[f][i], bias[f]);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (C::gam(n) / SL != f) continue;  // compile-time
        uint32_t a[4];
        if constexpr (BV == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = (r.vw[n] >> (4 * e)) & 0x000F000Fu;
        } else {
          const int sh = 8 * (lg & 1);
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = (r.vw[n] >> (sh + 2 * e)) & 0x00030003u;
        }
        oacc[n] = mfma(a, bh, oacc[n]);
        oacc[n] = mfma(a, bl, oacc[n]);
      }
    }
  }
};

template <int D, int BK, int BV, int GQ, int NG>
__device__ void packed_partial(const DecodeLaunch& L, int b, int hkv, int split, int t0,
                               int t1, char* smem) {
  using C = Cfg<D, BK, BV, GQ, NG>;
  using W = PackedWave<D, BK, BV, GQ, NG>;
  using R = Raw<D, BK, BV, GQ, NG>;
  constexpr int NT = C::NT, SL = C::SL, NF = C::NF;
  const Geom& g = L.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t unit = (int64_t)b * g.Hkv + hkv;

  float* qfs = reinterpret_cast<float*>(smem);            // [GQ][D] q * 2^-E
  int* qexp = reinterpret_cast<int*>(qfs + GQ * D);       // [GQ]
  char* wbase = smem + (GQ * D + 16) * 4 + wave * C::kWaveLds;

  for (int i = tid; i < GQ * D; i += kThreads)
    qfs[i] = h2f(L.q[((int64_t)b * g.Hq + hkv * GQ) * D + i]) * L.scale_log2;
  __syncthreads();
  // per-head exponent E with max|qf| < 2^E, so that q * 2^-E * scale fits fp16
  for (int h = wave; h < GQ; h += kWaves) {
    float mx = 0.0f;
    for (int c = lane; c < D; c += 64) mx = fmaxf(mx, fabsf(qfs[h * D + c]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = xor_max(mx, off);
    int e = 0;
    if (mx > 0.0f) (void)frexpf(mx, &e);
    if (lane == 0) qexp[h] = e;
  }
  __syncthreads();
  for (int i = tid; i < GQ * D; i += kThreads) qfs[i] = ldexpf(qfs[i], -qexp[i / D]);
  __syncthreads();

  W w;
  w.kcodes = L.cache.k_codes + unit * g.C * C::WR;
  w.kmeta = reinterpret_cast<const uint32_t*>(L.cache.k_meta) + unit * (g.C / C::G) * D;
  w.vcodes = L.cache.v_codes + unit * (g.C / kVBlock) * D * BV;
  w.vmeta = reinterpret_cast<const uint32_t*>(L.cache.v_meta) +
            unit * (g.C / kVBlock) * NG * kVBlock;
  w.qfs = qfs;
  w.qB = reinterpret_cast<uint4*>(wbase);
  w.beta_l = reinterpret_cast<float*>(wbase + C::kQB);
  const int nchunks = (t1 - t0) / kChunk;
  const int c_lo = t0 / kChunk + (nchunks * wave) / kWaves;
  const int c_hi = t0 / kChunk + (nchunks * (wave + 1)) / kWaves;
  w.c_lo = c_lo;
  w.c_hi = c_hi;
  w.init(lane);
  const int e_h = qexp[w.hcol];
  w.kscale = ldexpf(1.0f, e_h + 24);  // codes are the fp16 numbers c * 2^-24
  w.bscale = ldexpf(1.0f, e_h);

  // two chunk buffers: the next chunk's loads are in flight while one is
  // used.  Prefetches past the wave's last chunk re-load that chunk (always in
  // bounds) instead of being skipped, so no load sits under a branch.
  R ra, rb;
  if (c_lo < c_hi) {
    const int last = c_hi - 1;
    w.load_kmeta((c_lo * kChunk) / C::G);
    w.load(c_lo, ra);
    for (int ch = c_lo; ch < c_hi; ch += 2) {
      w.load(min(ch + 1, last), rb);
      w.process(ch, ra);
      if (ch + 1 >= c_hi) break;
      w.load(min(ch + 2, last), ra);
      w.process(ch + 1, rb);
    }
  }

  // ---------------- merge lane groups, then waves ----------------
  float l_run = w.l_run;
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);
  float bias[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    bias[f] = xor_sum(w.bias[f], 16);
    bias[f] = xor_sum(bias[f], 32);
  }
  __syncthreads();  // fold buffers are reused for the merge below
  float* cmb = reinterpret_cast<float*>(smem);  // [kWaves][GQ][D + 2]
  float* mine = cmb + wave * GQ * (D + 2);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int gm = C::gam(n);
    if (gm % SL != w.slot) continue;
    const float bsum = bias[gm / SL];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      mine[w.hcol * (D + 2) + 16 * n + 4 * w.lg + q] = w.oacc[n][q] * 16777216.0f + bsum;
  }
  if (w.lg == 0 && w.slot == 0) {
    mine[w.hcol * (D + 2) + D] = w.m_run;
    mine[w.hcol * (D + 2) + D + 1] = l_run;
  }
  __syncthreads();
  for (int i = tid; i < GQ * D; i += kThreads) {
    const int h = i / D, c = i % D;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, cmb[(v * GQ + h) * (D + 2) + D]);
    float Ls = 0.0f, acc = 0.0f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float* sv = cmb + (v * GQ + h) * (D + 2);
      const float wt = (sv[D] == kNegInf) ? 0.0f : exp2f(sv[D] - M);
      Ls += sv[D + 1] * wt;
      acc += sv[c] * wt;
    }
    const int64_t bh = (int64_t)b * g.Hq + hkv * GQ + h;
    float* part = L.ws + (bh * (L.n_split + 1) + split) * (D + 2);
    part[c] = acc;
    if (c == 0) {
      part[D] = M;
      part[D + 1] = Ls;
    }
  }
}

template <int D, int BK, int BV, int GQ, int NG>
constexpr int kSmemBytes() {
  using C = Cfg<D, BK, BV, GQ, NG>;
  constexpr int packed = (GQ * D + 16) * 4 + kWaves * C::kWaveLds;
  constexpr int merge = kWaves * GQ * (D + 2) * 4;
  constexpr int resid = (GQ * D + GQ * kChunk + 3 * GQ) * 4;
  constexpr int m1 = packed > merge ? packed : merge;
  return m1 > resid ? m1 : resid;
}

// grid: (n_split + 1, Hkv, B).  x < n_split: packed tokens of split x;
// x == n_split: the residual window.
template <int D, int BK, int BV, int GQ, int NG>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecodeLaunch L) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes<D, BK, BV, GQ, NG>()];
  const Geom& g = L.g;
  const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int n = L.seq_lens[b];
  if (n <= 0 || n > g.C || n > L.max_seq_len) return;  // the combine writes 0 / NaN
  const int lq = packed_len(n, g.R);
  if (split == L.n_split) {
    residual_partial<D, GQ>(L, b, hkv, lq, n, L.n_split, reinterpret_cast<float*>(smem));
    return;
  }
  const int t0 = split * L.split_tokens;
  const int t1 = min(lq, t0 + L.split_tokens);
  if (t0 >= t1) return;  // no packed tokens here: the combine skips this split
  packed_partial<D, BK, BV, GQ, NG>(L, b, hkv, split, t0, t1, smem);
}

// Merges the partials of one (sequence, query head).
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeLaunch L) {
  const Geom& g = L.g;
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int64_t bh = (int64_t)b * g.Hq + h;
  const int n = L.seq_lens[b];
  if (n < 0 || n > g.C || n > L.max_seq_len) {
    L.out[bh * D + c] = 0x7e00;  // NaN: length outside [0, max_seq_len]
    return;
  }
  if (n == 0) {
    L.out[bh * D + c] = 0;
    return;
  }
  const int lq = packed_len(n, g.R);
  const int nsp = (lq + L.split_tokens - 1) / L.split_tokens;  // packed splits used
  const float* part = L.ws + bh * (L.n_split + 1) * (D + 2);
  const float* res = part + L.n_split * (D + 2);
  float M = res[D];
  for (int i = 0; i < nsp; ++i) M = fmaxf(M, part[i * (D + 2) + D]);
  float w = exp2f(res[D] - M);
  float Ls = res[D + 1] * w, acc = res[c] * w;
  for (int i = 0; i < nsp; ++i) {
    w = exp2f(part[i * (D + 2) + D] - M);
    Ls += part[i * (D + 2) + D + 1] * w;
    acc += part[i * (D + 2) + c] * w;
  }
  L.out[bh * D + c] = f2h(acc / Ls);
}

template <int D, int BK, int BV, int GQ>
hipError_t dispatch_ng(const DecodeLaunch& L, dim3 grid, hipStream_t st) {
  switch (D / L.g.G) {
    case 1: decode_partial_kernel<D, BK, BV, GQ, 1><<<grid, kThreads, 0, st>>>(L); break;
    case 2: decode_partial_kernel<D, BK, BV, GQ, 2><<<grid, kThreads, 0, st>>>(L); break;
    case 4:
      if constexpr (D == 128) {
        decode_partial_kernel<D, BK, BV, GQ, 4><<<grid, kThreads, 0, st>>>(L);
        break;
      }
      [[fallthrough]];
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int BK, int BV>
hipError_t dispatch_gq(const DecodeLaunch& L, hipStream_t st) {
  dim3 grid(L.n_split + 1, L.g.Hkv, L.g.B);
  switch (L.g.Hq / L.g.Hkv) {
    case 1: return dispatch_ng<D, BK, BV, 1>(L, grid, st);
    case 2: return dispatch_ng<D, BK, BV, 2>(L, grid, st);
    case 4: return dispatch_ng<D, BK, BV, 4>(L, grid, st);
    case 8: return dispatch_ng<D, BK, BV, 8>(L, grid, st);
    case 16: return dispatch_ng<D, BK, BV, 16>(L, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t dispatch_bits(const DecodeLaunch& L, hipStream_t st) {
  const int bk = L.g.bK, bv = L.g.bV;
  if (bk == 2 && bv == 2) return dispatch_gq<D, 2, 2>(L, st);
  if (bk == 2 && bv == 4) return dispatch_gq<D, 2, 4>(L, st);
  if (bk == 4 && bv == 2) return dispatch_gq<D, 4, 2>(L, st);
  return dispatch_gq<D, 4, 4>(L, st);
}

}  // namespace

hipError_t launch_decode_partial(const DecodeLaunch& L, hipStream_t st) {
  return L.g.D == 64 ? dispatch_bits<64>(L, st) : dispatch_bits<128>(L, st);
}

hipError_t launch_decode_combine(const DecodeLaunch& L, hipStream_t st) {
  dim3 grid(L.g.Hq, L.g.B);
  if (L.g.D == 64)
    decode_combine_kernel<64><<<grid, 64, 0, st>>>(L);
  else
    decode_combine_kernel<128><<<grid, 128, 0, st>>>(L);
  return hipGetLastError();
}

}  // namespace kvq
