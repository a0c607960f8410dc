// kvq_bq2_decode.hip — single-token decode attention over the rotated
// per-token 2-bit cache (KV1's BQ2_0; layout in kvq_bq2.h) on gfx950.
//
// [KV1] "Quantization Format: KV1.cpp BQ2_0": the cache holds H k and H v
// (H the normalized Sylvester Hadamard matrix, H H = I), quantized per
// position as code * d + m over the 64 channels, positions 0..3 in fp16;
// scores are unchanged by the rotation and the output is rotated back.  For
// query head h, with qH = H q in log2 units (sm_scale * log2 e folded in):
//   s_t = d_t (qH . code_t) + m_t sum_c qH_c
//   o   = sum_t (p_t dV_t) code_t + (sum_t p_t mV_t) (1, ..., 1)
//   out = H o / sum_t p_t
// Both contractions run on v_mfma_f32_16x16x32_f16 with the codes fed as fp16
// subnormals, as in kvq_decode.hip: the key side multiplies the codes by the
// rotated query and applies each position's d_t, m_t to the finished score;
// the value side multiplies the codes by p_t dV_t.
//
// Precision of the key side.  The two terms of s_t are large and nearly
// cancel (the dequantized keys are about zero-mean), so the code product must
// be accurate to ~2^-20 of its products' magnitude.  The matrix core sums the
// products of one column exactly only while they span no more than about 20
// bits (mantissa width plus exponent spread); wider spans lose the low bits of
// the smallest products, the same bits for every position, which shifts a
// head's scores uniformly.  So each head's query operand uses four columns:
// part 0 holds the components within 2^kBigSpan of the head's largest (11-bit
// values, 2-bit codes: exact sums), part 1 the rest and part 0's remainders,
// part 2 what part 1 leaves, part 3 zero; a quad of DPP adds recombines them.
// The value side has the same limit (softmax weights span many binades), so
// its four columns per head hold the hi and lo parts of the large weights
// (p >= 2^-kBigSpanV, whose products span few bits) and of the small ones.  The sinks
// take one more MFMA step on their fp16 vectors.  The work decomposition and
// the combine (which rotates the merged output back) are shared with the other
// format (kvq_device.h).
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kD = KVQ_BQ2_HEAD_DIM;
constexpr int kSinks = KVQ_BQ2_SINKS;
constexpr float kValEvenB = kValEven<2>, kValOddB = kValOdd<2>;
constexpr int kQTop = 14;     // the query operand's largest component is below 2^kQTop
constexpr int kBigSpan = 7;   // part 0 holds components above 2^(kQTop - kBigSpan)
constexpr int kBigSpanV = 6;  // value weights p >= 2^-kBigSpanV go to the large columns

// Work of a sequence of n positions: the 32-position chunks holding quantized
// positions (chunk 0 counts when n > 4), one work unit each, then the sink
// chunk, weighted rw (its fp16 bytes over a packed chunk's).
__device__ __forceinline__ SeqWork bq2_work_of(const Bq2Launch& L, int n) {
  SeqWork sw{0, 0, 0, 0};
  if (n <= 0 || n > L.g.C || n > L.max_seq_len) return sw;
  sw.n = n;
  sw.nq = n > kSinks ? (n + kChunk - 1) / kChunk : 0;
  sw.nr = 1;
  sw.w = sw.nq + L.rw;
  return sw;
}

struct Bq2Work {
  using Launch = Bq2Launch;
  static constexpr bool kRotateOut = true;
  static __device__ __forceinline__ SeqWork work_of(const Bq2Launch& L, int n) {
    return bq2_work_of(L, n);
  }
  static __device__ __forceinline__ int64_t row(const Bq2Launch& L, int b, int hkv, int j) {
    return (int64_t)b * L.g.Hq + hkv * (L.g.Hq / L.g.Hkv) + j;
  }
};

// Words in the global address space, and p as such a pointer made wave-uniform
// (its value in the first active lane): address arithmetic on it stays in
// scalar registers, and a load from it plus a lane offset takes the
// scalar-base + vector-offset form (no 64-bit vector add per load).  Only for
// pointers into global memory that are the same in every lane.
typedef __attribute__((address_space(1))) const uint32_t gword;
__device__ __forceinline__ gword* wave_uniform(const uint32_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane((uint32_t)v));
  return reinterpret_cast<gword*>(((uint64_t)hi << 32) | (uint64_t)lo);
}
// Two consecutive words (8-byte aligned) from global memory as one
// nontemporal load.
__device__ __forceinline__ void load_pair_nt(gword* p, uint32_t (&w)[2]) {
  typedef __attribute__((address_space(1))) const unsigned int __attribute__((ext_vector_type(2))) gu2;
  const auto v = __builtin_nontemporal_load((gu2*)p);
  w[0] = v.x;
  w[1] = v.y;
}

// A lane's share of one 32-position chunk.
struct Bq2Raw {
  uint32_t kw[2];  // key code words of score tiles 0, 1
  uint32_t vw[2];  // value code words (tiles 2m, 2m + 1 in word m)
  uint32_t km[2];  // key (d, m) of this lane's positions 8 lg + 2 i + k (i: quad position)
  uint32_t vm[2];  // value (d, m) of the same positions
};

// A lane's share of a unit's sink vectors, fetched with the first chunk:
// key rows min(i, 3) (i = lane % 16; rows at or past the sink count are zeroed
// at use), value channels 16 n + i (used by lane group 0 only).
struct Bq2Sinks {
  uint4 k[2];  // channels 32 kc + 8 g .. + 7 of key row min(i, 3)
  uint2 v[4];  // positions 0..3 of channel 16 n + i
};

template <int GQ>
struct Bq2Wave {
  static constexpr int SL = 16 / GQ;  // MFMA columns per head
  static_assert(SL >= 4, "the key-side operand needs four columns per head");

  const uint32_t* kcodes;
  const uint32_t* vcodes;
  const uint32_t* kmeta;
  const uint32_t* vmeta;
  int lane, col, lg, hcol, part, kpart;
  bool vbig;     // this lane's value columns hold the large weights
  uint32_t m_q1, m_q2;  // all ones where bit 0 / bit 1 of the lane's quad position is set
  uint32_t m_vbig;      // all ones on lanes whose value columns take the large weights
  float m1;      // -1 in a register
  float mpart;   // 0 on hi lanes, -1 on lo lanes: selects the part of a split
  float qbig;    // 2^(kQTop - kBigSpan): query components at or above go to key part 0
  float kscale;  // 2^(E - kQTop + 24 - L): code accumulation to log2 units (this lane's head)
  float sumq_k;  // sum_c qH_c of this lane's head (log2 units) / kscale
  float qexp;    // 2^(E - kQTop)
  f4 oacc[4];
  float m_run, m_even, m_odd;
  float l_run, l_odd;
  float bias, bias_odd;  // value-min terms of the two weight classes
  uint32_t bq[2][4];

  __device__ void init(int lane_) {
    lane = lane_;
    col = lane & 15;
    lg = lane >> 4;
    hcol = col / SL;
    part = (col % SL) & 1;
    kpart = (col % SL) & 3;
    vbig = kpart < 2;
    m_q1 = 0u - (uint32_t)(lane & 1);
    m_q2 = 0u - (uint32_t)((lane >> 1) & 1);
    m_vbig = vbig ? ~0u : 0u;
    m1 = opaque_m1();
    qbig = ldexpf(1.0f, kQTop - kBigSpan);
    mpart = part ? m1 : 0.0f;
#pragma unroll
    for (int n = 0; n < 4; ++n) oacc[n] = f4{0.f, 0.f, 0.f, 0.f};
    m_run = m_even = m_odd = kNegInf;
    l_run = l_odd = 0.0f;
    bias = bias_odd = 0.0f;
  }

  // (a, b) -> the fp16 pair of this lane's part: hi = rne(a, b), lo = the
  // remainders (exact fp32 differences) rounded to nearest (part 0 rounds
  // a - 0 * hi, i.e. is hi itself).
  __device__ __forceinline__ uint32_t part_of(float a, float b) const {
    const uint32_t hi = pk_rne(a, b);
    return pk_rne(__builtin_fmaf(lo_half(hi), mpart, a), __builtin_fmaf(hi_half(hi), mpart, b));
  }

  // Key-side operand pair of this lane's part (qa, qb: query components; f:
  // the pair's positional factor): part 0 = fp16 of the large components,
  // part 1 = fp16 of what remains, part 2 = fp16 of what remains then, part 3
  // = 0.  Every remainder is an exact fp32 difference.
  __device__ __forceinline__ uint32_t key_part(float qa, float qb, float f) const {
    const float a = qa * f, b = qb * f;
    const uint32_t h0 = pk_rne(fabsf(qa) >= qbig ? a : 0.0f, fabsf(qb) >= qbig ? b : 0.0f);
    const float ra = a - lo_half(h0), rb = b - hi_half(h0);
    const uint32_t h1 = pk_rne(ra, rb);
    const uint32_t h2 = pk_rne(ra - lo_half(h1), rb - hi_half(h1));
    return kpart == 0 ? h0 : kpart == 1 ? h1 : kpart == 2 ? h2 : 0u;
  }
  // Value-side operand pair of this lane's column (x: weights p * dV; p: the
  // weights; thr: the class's large-weight threshold): the large or the small
  // weights only, hi or lo part.
  __device__ __forceinline__ uint32_t value_part(float xa, float xb, float pa, float pb,
                                                 float thr) const {
    return part_of((pa >= thr) == vbig ? xa : 0.0f, (pb >= thr) == vbig ? xb : 0.0f);
  }
  // Sum of a result over the four columns of a part set (a quad of lanes).
  __device__ __forceinline__ float key_sum(float x) const {
    x += dpp<0xB1>(x);  // quad_perm [1, 0, 3, 2]
    x += dpp<0x4E>(x);  // quad_perm [2, 3, 0, 1]
    return x;
  }

  __device__ __forceinline__ void load(int ch, Bq2Raw& r) const {
    // chunk bases wave-uniform, lane offsets apart
    const int lm = 8 * lg + 2 * (lane & 3);
    load_pair_nt(wave_uniform(kcodes + ch * 128) + 2 * lane, r.kw);
    load_pair_nt(wave_uniform(vcodes + ch * 128) + 2 * lane, r.vw);
    load_pair_nt(wave_uniform(kmeta + ch * kChunk) + lm, r.km);
    load_pair_nt(wave_uniform(vmeta + ch * kChunk) + lm, r.vm);
  }

  // Scores arrive as s / sc (sc > 0 per lane: a power of two), the running
  // max is kept in log2 units; p = 2^(s - m) = 2^(fma(s/sc, sc, -m)).  The
  // four lanes of a quad (one head's columns) hold the same 8 code products
  // after the quad sum, so each works on positions 2 i, 2 i + 1 of the lane
  // group (i its quad position; x: their scores, pm: their weights) for the
  // maximum, the exponentials and the sums, which are per lane and summed
  // over the quad at the end.  Callers gather the 8 weights from the quad.
  template <bool kPacked>
  __device__ __forceinline__ void softmax(const float (&x)[2], float sc, float (&pm)[2]) {
    float cm = fmaxf(x[0], x[1]) * sc;
    if (__any(cm > m_run)) {
      cm = xor_max(cm, 1);
      cm = xor_max(cm, 2);
      cm = xor_max(cm, 16);
      cm = xor_max(cm, 32);
      const float m_new = fmaxf(m_run, cm);
      const float a = exp2_hw(m_run - m_new);
      m_run = m_new;
      m_even = kPacked ? m_new - kValEvenLog2<2> : m_new;
      m_odd = kPacked ? m_new - kValOddLog2<2> : m_new;
      l_run *= a;
      l_odd *= a;
      bias *= a;
      bias_odd *= a;
#pragma unroll
      for (int n = 0; n < 4; ++n) oacc[n] *= a;
    }
    // the lane's two positions are rows 2 (i % 2) + k: one weight class
    const bool odd = lane & 1;
    const float mref = odd ? m_odd : m_even;
    pm[0] = exp2_hw(__builtin_fmaf(x[0], sc, -mref));
    pm[1] = exp2_hw(__builtin_fmaf(x[1], sc, -mref));
    const float add = pm[0] + pm[1];
    if constexpr (kPacked) {
      l_run += odd ? 0.0f : add;
      l_odd += odd ? add : 0.0f;
    } else {
      l_run += add;
    }
  }

  // One chunk of quantized positions.  kEdge: chunk 0 (positions 0..3 are
  // the sinks) or a chunk reaching past n; its positions outside [4, n) are
  // masked (score -inf, value meta 0, so stale memory never reaches a sum).
  template <bool kEdge>
  __device__ __forceinline__ void process(int ch, Bq2Raw r, int n) {
    if constexpr (kEdge) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int t = ch * kChunk + 8 * lg + 2 * (lane & 3) + k;
        r.vm[k] = (t >= kSinks && t < n) ? r.vm[k] : 0u;
      }
    }
    float xs[2][4];
    uint32_t ka[2][2][4];
    unpack_keys_2x64(r.kw, ka);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma(ka[u][0], bq[0], acc);
      acc = mfma(ka[u][1], bq[1], acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[u][q] = key_sum(acc[q]);
    }
    // this lane's positions 8 lg + 2 i + k:
    // s / kscale = d (qH . code) 2^-(E - kQTop + 24) + m sum qH / kscale
    float s[2];
    quad_pick2(m_q1, m_q2, xs, s);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      s[k] = mul_lo(s[k], r.km[k], mul_hi(sumq_k, r.km[k]));
      if constexpr (kEdge) {
        const int t = ch * kChunk + 8 * lg + 2 * (lane & 3) + k;
        s[k] = (t >= kSinks && t < n) ? s[k] : kNegInf;
      }
    }
    float pm[2];
    softmax<true>(s, kscale, pm);
    // this lane's positions: weighted value scales p dV and the value-min term
    // (per lane, in the positions' class: odd quad positions are the odd class)
    float ym[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) ym[k] = mul_lo(pm[k], r.vm[k]);
    {
      const float bm = mul_hi(pm[1], r.vm[1], mul_hi(pm[0], r.vm[0]));
      const bool odd = lane & 1;
      bias += odd ? 0.0f : bm;
      bias_odd += odd ? bm : 0.0f;
    }
    // the lane's products split by weight size (the large-weight columns
    // take p >= the class threshold; odd quad positions are the odd class,
    // whose p carries the factor 1/4): one of each pair is the product, the
    // other 0.  All 8 positions of the lane group come back from the quad.
    float yb[2], ys[2];
    {
      const float thr = (lane & 1) ? ldexpf(kValOddB, -kBigSpanV) : ldexpf(1.0f, -kBigSpanV);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const bool big = pm[k] >= thr;
        yb[k] = big ? ym[k] : 0.0f;
        ys[k] = big ? 0.0f : ym[k];
      }
    }
    float Yb[2][4], Ys[2][4];
    quad_gather2(yb, Yb);
    quad_gather2(ys, Ys);
    // B operand: element j = position 8 lg + j, weight p_j dV_j (the part of
    // this lane's columns); pair e holds j = 2e, 2e + 1
    uint32_t b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ja = 2 * e, jb = 2 * e + 1;
      b[e] = part_of(bit_sel(m_vbig, Yb[ja >> 2][ja & 3], Ys[ja >> 2][ja & 3]),
                     bit_sel(m_vbig, Yb[jb >> 2][jb & 3], Ys[jb >> 2][jb & 3]));
    }
    // tile 2m + h: pair e of token 8 lg + 2e (+1) at bits 8h + 4(e/2) + 2(e%2)
    uint32_t va[4][4];
    unpack_values_2x64(r.vw, va);
#pragma unroll
    for (int n = 0; n < 4; ++n) oacc[n] = mfma(va[n], b, oacc[n]);
  }

  // Packed accumulation to real scale (codes were c * 2^(L-24), odd pairs carry
  // their class factor) with the value-min term added once per column pair.
  __device__ __forceinline__ void to_real() {
    float bt = __builtin_fmaf(bias_odd, 1.0f / kValOddB, bias * (1.0f / kValEvenB));
    bt = xor_sum(xor_sum(bt, 1), 2);  // per-lane terms: the quad, then the lane groups
    bt = xor_sum(xor_sum(bt, 16), 32);
    if (kpart != 0) bt = 0.0f;  // once per head: the four columns are summed
    constexpr float oscale = 16777216.0f / float(1 << kCodeLift<2>) / kValEvenB;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) oacc[n][q] = __builtin_fmaf(oacc[n][q], oscale, bt);
    l_run = __builtin_fmaf(l_odd, 1.0f / kValOddB, l_run * (1.0f / kValEvenB));
    l_odd = 0.0f;
    bias = bias_odd = 0.0f;
    m_even = m_odd = m_run;
  }

  // The sinks (positions 0 .. ns-1, ns <= 4) from their fp16 vectors: key
  // tile 0 rows 0..3 are positions 0..3; the query fragments are rebuilt in
  // natural channel order (element j of lane group g, k-chunk kc = channel
  // 32 kc + 8 g + j) from qfs (qH * 2^(kQTop - E)).
  __device__ __forceinline__ void load_sinks(const uint16_t* ksink, const uint16_t* vsink,
                                             Bq2Sinks& sk) const {
    const int i = lane & 15, row = min(i, kSinks - 1);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
      sk.k[kc] = *reinterpret_cast<const uint4*>(ksink + row * kD + 32 * kc + 8 * lg);
#pragma unroll
    for (int n = 0; n < 4; ++n)
      sk.v[n] = *reinterpret_cast<const uint2*>(vsink + (16 * n + i) * kSinks);
  }

  __device__ __forceinline__ void process_sinks(const Bq2Sinks& sk, int ns, const float* qfs) {
    uint32_t bn[2][4];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const float4 qa = *reinterpret_cast<const float4*>(qfs + hcol * kD + 32 * kc + 8 * lg);
      const float4 qb = *reinterpret_cast<const float4*>(qfs + hcol * kD + 32 * kc + 8 * lg + 4);
      bn[kc][0] = key_part(qa.x, qa.y, 1.0f);
      bn[kc][1] = key_part(qa.z, qa.w, 1.0f);
      bn[kc][2] = key_part(qb.x, qb.y, 1.0f);
      bn[kc][3] = key_part(qb.z, qb.w, 1.0f);
    }
    const int i = lane & 15;
    const bool krow = i < ns;
    uint32_t a[2][4];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      a[kc][0] = krow ? sk.k[kc].x : 0u;
      a[kc][1] = krow ? sk.k[kc].y : 0u;
      a[kc][2] = krow ? sk.k[kc].z : 0u;
      a[kc][3] = krow ? sk.k[kc].w : 0u;
    }
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma(a[0], bn[0], acc);
    acc = mfma(a[1], bn[1], acc);
    float s8[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // tile 0 row 4 lg + q is position 8 lg + q
      const float x = key_sum(acc[q]) * qexp;
      s8[0][q] = (lg == 0 && q < ns) ? x : kNegInf;
      s8[1][q] = kNegInf;
    }
    float s[2];
    quad_pick2(m_q1, m_q2, s8, s);
    float pm[2], p[2][4];
    softmax<false>(s, 1.0f, pm);
    quad_gather2(pm, p);
    uint32_t b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ja = 2 * e, jb = 2 * e + 1;
      const float pa = p[ja >> 2][ja & 3], pb = p[jb >> 2][jb & 3];
      b[e] = value_part(pa, pb, pa, pb, ldexpf(1.0f, -kBigSpanV));
    }
    // value tile n: element j of lane group 0 is position j of channel 16n + i
    const uint32_t keep0 = (ns > 0 ? 0x0000FFFFu : 0u) | (ns > 1 ? 0xFFFF0000u : 0u);
    const uint32_t keep1 = (ns > 2 ? 0x0000FFFFu : 0u) | (ns > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint2 v = lg == 0 ? sk.v[n] : make_uint2(0u, 0u);
      uint32_t av[4] = {v.x & keep0, v.y & keep1, 0u, 0u};
      oacc[n] = mfma(av, b, oacc[n]);
    }
  }
};

constexpr int kDP = kD + kPartPad;

// The value of x in lane l (wave-uniform).
__device__ __forceinline__ float lane_value(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Sets up the wave for unit `unit` and issues the loads of the range's first
// chunk and (if the range holds the sink chunk) of the sinks, before anything
// else, so that their latency overlaps the query's.
template <int GQ>
__device__ __forceinline__ void bq2_begin(const Bq2Launch& L, int64_t unit, const SegRange& r,
                                          int lane, Bq2Wave<GQ>& w, Bq2Raw& ra, Bq2Sinks& sk) {
  const Bq2Geom& g = L.g;
  w.init(lane);
  w.kcodes = L.cache.k_codes + unit * (g.C / kChunk) * 128;
  w.vcodes = L.cache.v_codes + unit * (g.C / kChunk) * 128;
  w.kmeta = reinterpret_cast<const uint32_t*>(L.cache.k_meta) + unit * g.C;
  w.vmeta = reinterpret_cast<const uint32_t*>(L.cache.v_meta) + unit * g.C;
  if (r.pc0 < r.pc1) w.load(r.pc0, ra);
  if (r.rk0 < r.rk1)
    w.load_sinks(L.cache.k_sink + unit * kSinks * kD, L.cache.v_sink + unit * kD * kSinks, sk);
}

// Runs range r of unit (b, hkv) -> partial p, bq2_begin having been done.
template <int GQ>
__device__ void bq2_run(const Bq2Launch& L, int b, int hkv, const SeqWork& sw, const SegRange& r,
                        int p, float* qfs, int lane, Bq2Wave<GQ>& w, Bq2Raw& ra,
                        const Bq2Sinks& sk) {
  const Bq2Geom& g = L.g;
  float* part_base = L.ws + (int64_t)p * GQ * kDP;
  Bq2Raw rb, rc, rd;

  // rotated query of the unit's GQ heads: qH = H q (in log2 units), per-head
  // exponent E with max |qH| < 2^E, qfs = qH * 2^(kQTop - E): the largest
  // component sits just below 2^kQTop, so the lo parts of the hi/lo split stay
  // normal fp16 numbers for every component above 2^(kQTop - 25) of the largest
  // (no key scale is folded into the query here, so fp16 has that headroom)
  // The butterflies pair lane l with l ^ d: DPP inside a quad (d = 1, 2) and a
  // row (d = 8, a rotation by half a row), lane shuffles otherwise.  sum_c qH_c
  // = 8 q_0 (every column of H but the first sums to 0).
  const uint16_t* qg = L.q + ((int64_t)b * g.Hq + hkv * GQ) * kD;
  int e_mine = 0;
  float sum_mine = 0.0f;
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float x = h2f(qg[h * kD + lane]);
    const float q0 = lane_value(x, 0);
    {
      float y = dpp<0xB1>(x);  // quad_perm [1, 0, 3, 2]: lane ^ 1
      x = (lane & 1) ? (y - x) : (x + y);
      y = dpp<0x4E>(x);        // quad_perm [2, 3, 0, 1]: lane ^ 2
      x = (lane & 2) ? (y - x) : (x + y);
      y = __shfl_xor(x, 4, 64);
      x = (lane & 4) ? (y - x) : (x + y);
      y = dpp<0x128>(x);       // row_ror:8: lane ^ 8
      x = (lane & 8) ? (y - x) : (x + y);
      y = __shfl_xor(x, 16, 64);
      x = (lane & 16) ? (y - x) : (x + y);
      y = __shfl_xor(x, 32, 64);
      x = (lane & 32) ? (y - x) : (x + y);
    }
    x *= 0.125f * L.scale_log2;
    // max |qH| over the wave: rotations inside each row, then the four rows
    float mx = fabsf(x);
    mx = fmaxf(mx, dpp<0x128>(mx));
    mx = fmaxf(mx, dpp<0x124>(mx));
    mx = fmaxf(mx, dpp<0x122>(mx));
    mx = fmaxf(mx, dpp<0x121>(mx));
    mx = fmaxf(fmaxf(lane_value(mx, 0), lane_value(mx, 16)),
               fmaxf(lane_value(mx, 32), lane_value(mx, 48)));
    int e = 0;
    if (mx > 0.0f) (void)frexpf(mx, &e);
    qfs[h * kD + lane] = ldexpf(x, kQTop - e);
    if (w.hcol == h) {
      e_mine = e;
      sum_mine = 8.0f * q0 * L.scale_log2;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  w.kscale = ldexpf(1.0f, e_mine - kQTop + 24 - kKeyAccLog2<2> - kCodeLift<2>);
  w.qexp = ldexpf(1.0f, e_mine - kQTop);
  w.sumq_k = sum_mine / w.kscale;  // exact: kscale is a power of two
  // key-side fragments in the key words' channel order: pair v of k-chunk kc
  // = channels 16 lg + 4 kc + v and + 8; odd pairs come out of their mask 4x
  // larger, so their query factor is 1/4
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c0 = 16 * w.lg + 4 * kc + v;
      const float f = (v & 1) ? kKeyOddQ<2> : kKeyEvenQ<2>;
      w.bq[kc][v] = w.key_part(qfs[w.hcol * kD + c0], qfs[w.hcol * kD + c0 + 8], f);
    }

  if (r.pc0 < r.pc1) {
    // masked chunks (chunk 0, a last chunk reaching past n) are peeled off,
    // so the pipelined loop over the others has no branch but the rescale
    int lo = r.pc0;
    const int hi = r.pc1;
    if (lo == 0) {  // ra holds chunk 0
      w.template process<true>(0, ra, sw.n);
      if (++lo < hi) w.load(lo, ra);
    }
    const bool tail = sw.nq * kChunk > sw.n;
    const int end = (tail && hi == sw.nq && hi - 1 >= lo) ? hi - 1 : hi;
    if (lo < end) {
      // four chunk buffers: the loads of the next three chunks are in flight
      // while one is used (a chunk here is only 1.25 KB, 8 registers a lane).
      // Prefetches past the last chunk re-load that chunk (always in bounds)
      // instead of being skipped, so no load sits under a branch.
      const int last = end - 1;
      int ch = lo;
      w.load(min(ch + 1, last), rb);
      w.load(min(ch + 2, last), rc);
      for (; ch + 3 <= last; ch += 4) {  // ra, rb, rc hold chunks ch .. ch + 2 on entry
        w.load(ch + 3, rd);
        w.template process<false>(ch, ra, sw.n);
        w.load(min(ch + 4, last), ra);
        w.template process<false>(ch + 1, rb, sw.n);
        w.load(min(ch + 5, last), rb);
        w.template process<false>(ch + 2, rc, sw.n);
        w.load(min(ch + 6, last), rc);
        w.template process<false>(ch + 3, rd, sw.n);
      }
      if (ch <= last) w.template process<false>(ch, ra, sw.n);
      if (ch + 1 <= last) w.template process<false>(ch + 1, rb, sw.n);
      if (ch + 2 <= last) w.template process<false>(ch + 2, rc, sw.n);
    }
    if (end < hi) {
      w.load(end, ra);
      w.template process<true>(end, ra, sw.n);
    }
  }
  w.to_real();
  if (r.rk0 < r.rk1) w.process_sinks(sk, min(sw.n, kSinks), qfs);

  // partial: the four columns summed, max, sum over the four lane groups
  float l = w.l_run;  // per lane: summed over the quad, then the lane groups
  l = xor_sum(xor_sum(l, 1), 2);
  l = xor_sum(xor_sum(l, 16), 32);
  float* part = part_base + w.hcol * kDP;
  const bool writer = (w.col % Bq2Wave<GQ>::SL) == 0;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    f4 o = w.oacc[n];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = w.key_sum(o[q]);
    if (writer)
      *reinterpret_cast<float4*>(part + 16 * n + 4 * w.lg) = make_float4(o[0], o[1], o[2], o[3]);
  }
  if (writer && w.lg == 0) {
    part[kD] = w.m_run;
    part[kD + 1] = l;
  }
  // the next segment of this wave rewrites qfs
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Unit (b, hkv), work range [x0, x1) -> partial p.
template <int GQ>
__device__ void bq2_segment(const Bq2Launch& L, int b, int hkv, const SeqWork& sw, int xu,
                            int x0, int x1, int p, float* qfs, int lane) {
  const SegRange r = seg_range(L, sw, xu, x0, x1);
  if (r.pc0 >= r.pc1 && r.rk0 >= r.rk1) {  // only part of the sink chunk's weight
    float* part_base = L.ws + (int64_t)p * GQ * kDP;
    for (int i = lane; i < GQ * kDP; i += 64) part_base[i] = (i % kDP == kD) ? kNegInf : 0.0f;
    return;
  }
  Bq2Wave<GQ> w;
  Bq2Raw ra;
  Bq2Sinks sk;
  bq2_begin<GQ>(L, (int64_t)b * L.g.Hkv + hkv, r, lane, w, ra, sk);
  bq2_run<GQ>(L, b, hkv, sw, r, p, qfs, lane, w, ra, sk);
}

// One wave per workgroup; grid = the number of worker waves.
template <int GQ>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void bq2_partial_kernel(Bq2Launch L) {
  __shared__ __attribute__((aligned(16))) float qfs[GQ * kD];
  const int lane = threadIdx.x;
  const int w = blockIdx.x, nw = gridDim.x;
  const BatchWork bw = batch_work<Bq2Work>(L, lane);  // one read of the lengths
  const int total = bw.total;
  const int cpw = (total + nw - 1) / nw;
  const int x0 = w * cpw;
  const int x1 = min(total, x0 + cpw);
  int x = x0;
  while (x < x1) {
    int b, base;
    wave_find_seq<Bq2Work>(L, bw, lane, x, b, base);
    b = __builtin_amdgcn_readfirstlane(b);
    base = __builtin_amdgcn_readfirstlane(base);
    const int n = b < 64 ? __builtin_amdgcn_readlane(bw.n, b) : L.seq_lens[b];
    const SeqWork sw = bq2_work_of(L, n);
    const int hkv = (x - base) / sw.w;
    const int xu = base + hkv * sw.w;
    bq2_segment<GQ>(L, b, hkv, sw, xu, x0, x1, w + b * L.g.Hkv + hkv, qfs, lane);
    x = xu + sw.w;
  }
}

template <int GQ>
hipError_t workers_of(int cus, int* out) {
  static std::atomic<int> cache[64];  // 0: not queried yet (host threads may race here)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cache[dev].load(std::memory_order_relaxed) > 0) {
    *out = cache[dev].load(std::memory_order_relaxed);
    return hipSuccess;
  }
  int nb = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, bq2_partial_kernel<GQ>, 64, 0);
  if (e != hipSuccess) return e;
  if (nb < 1) nb = 1;
  const int w = nb * cus;
  if (dev >= 0 && dev < 64) cache[dev].store(w, std::memory_order_relaxed);
  *out = w;
  return hipSuccess;
}

// op 0: launch the partial kernel; 1: its worker count; 2: launch the combine.
template <int GQ>
hipError_t run(const Bq2Launch& L, int op, int cus, int* workers, hipStream_t st) {
  if (op == 1) return workers_of<GQ>(cus, workers);
  if (op == 0)
    bq2_partial_kernel<GQ><<<dim3(L.n_workers), 64, 0, st>>>(L);
  else if (L.g.B * L.g.Hkv < kCombineRowUnits && GQ > 1)
    decode_combine_kernel<Bq2Work, kD, GQ, 1><<<dim3(L.g.Hkv * GQ, L.g.B), kThreads, 0, st>>>(L);
  else
    decode_combine_kernel<Bq2Work, kD, GQ><<<dim3(L.g.Hkv, L.g.B), kThreads, 0, st>>>(L);
  return hipGetLastError();
}

hipError_t dispatch(const Bq2Launch& L, int op, int cus, int* workers, hipStream_t st) {
  switch (L.g.Hq / L.g.Hkv) {
    case 1: return run<1>(L, op, cus, workers, st);
    case 2: return run<2>(L, op, cus, workers, st);
    case 4: return run<4>(L, op, cus, workers, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t bq2_decode_workers(const Bq2Geom& g, int cus, int* workers) {
  Bq2Launch L{};
  L.g = g;
  return dispatch(L, 1, cus, workers, nullptr);
}

hipError_t launch_bq2_decode_partial(const Bq2Launch& L, hipStream_t st) {
  return dispatch(L, 0, 0, nullptr, st);
}

hipError_t launch_bq2_decode_combine(const Bq2Launch& L, hipStream_t st) {
  return dispatch(L, 2, 0, nullptr, st);
}

}  // namespace kvq
