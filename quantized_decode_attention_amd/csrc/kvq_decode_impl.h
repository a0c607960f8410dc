// kvq_decode_impl.h — decode attention over the packed cache plus
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
// shifted to the top of an fp16 mantissa and masked out of a packed word *is*
// the fp16 number c * 2^(L - 24), which the matrix cores multiply exactly)
// and the fp32 factors (q * scale, p * scale) split into a high and a low fp16
// part, two MFMAs accumulating into the same fp32 tile.
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
// Scores are kept in log2 units (sm_scale * log2 e applied to the finished
// dot products).
//
// A paged cache (block table, kvq_paged.h) differs only in where a packed
// chunk sits: its slot comes from the sequence's table row, of which each lane
// holds one entry; everything else is the dense path.
#pragma once
#include "kvq_device.h"

namespace kvq {
namespace {

// Row stride (floats) of the scaled query in LDS: D + 4, so that rows sit 4
// banks apart and the lanes of different rows reading the same channels hit
// different banks (a stride of D would put all rows on one bank).
template <int D>
constexpr int kQS = D + 4;

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
  // Value side.  When half of a head's MFMA columns can hold all its value
  // groups (kVSplit: at least four columns, NG <= SL / 2), column bit 0
  // selects the hi or lo fp16 part of the weights and the other bits a value
  // group (VH groups per fragment), so a value tile takes one MFMA and the
  // parts are added once, when the partial is written; otherwise each column
  // of a head is a group (VH = SL) and the hi and lo parts are two MFMAs into
  // one accumulator.  (With more groups than that the split would need a
  // second weight fragment, whose VALU work costs more than the MFMAs saved:
  // 54.0 against 52.8 us at four groups and four columns per head.)
  static constexpr bool kVSplit = SL >= 4 && NG <= SL / 2;
  static constexpr int VH = kVSplit ? SL / 2 : SL;
  static constexpr int NF = (NG + VH - 1) / VH;   // value-side B fragments
  static constexpr int IPH = 4 * KC;              // fold items per head
  static constexpr int ITEMS = GQ * IPH;          // fold items per key group
  static constexpr int IPL = (ITEMS + 63) / 64;   // fold items per lane
  // a lane's fold items are lane + 64 i: with IPH dividing 64 they all cover
  // the same channels (item modulo IPH), so one key-meta load serves them all
  static_assert(64 % IPH == 0, "fold items of a lane must share their channels");
  static constexpr bool VL = NF >= 2;
  // A chunk's LDS slot, the destination of its direct loads: key codes, value
  // codes, value meta, then the key meta of the chunk's key group, each in the
  // cache's byte order, so every lane reads back exactly the words it would
  // have loaded (byte offsets kSlot*).  A ring of kRing slots per wave: while
  // one chunk is used, the loads of the next kRing - 1 are in flight.
  static constexpr int KB = 4 * D * BK, VB = 4 * D * BV, VMB = 128 * NG, KMB = 4 * D;
  static constexpr int kSlotV = KB, kSlotVM = KB + VB, kSlotKM = KB + VB + VMB;
  static constexpr int kSlot = KB + VB + VMB + KMB;
  static constexpr int NI = (KB + 1023) / 1024 + (VB + 1023) / 1024 + (VMB + 1023) / 1024 +
                            (KMB + 1023) / 1024;  // direct loads per chunk
  static_assert(NI <= 20, "vmcnt must hold the ring's loads");
  // LDS (bytes) per wave: q' fragments (16 B slots, below), beta [GQ] (+ a
  // spare), two chunk slots
  // With one MFMA column per row (16 rows per KV head) every lane forms its
  // own q' fragments and no staging is needed.
  static constexpr bool kDirectFold = SL == 1;
  // q' fragment slots: one block of 4 KC slots (lane group, k-chunk) per head
  // and part, the two parts of a head adjacent, each block padded by a slot.
  // The 16 lanes of a fragment read differ only in head and part, so the
  // padding puts their slots on distinct banks (unpadded they all share one).
  static constexpr int kQBlk = 4 * KC + 1;
  static constexpr int qb_slot(int part, int h, int r) { return (2 * h + part) * kQBlk + r; }
  static constexpr int kQB = kDirectFold ? 0 : 2 * GQ * kQBlk * 16;
  static constexpr int kBetaB = kDirectFold ? 0 : 16 * ((GQ * 4 + 4 + 15) / 16);
  static constexpr int kRing = 2;
  static constexpr int kWaveLds = kQB + kBetaB + kRing * kSlot;
  static constexpr int gam(int n) { return (16 * n) / G; }  // group of value tile n
  static constexpr int frag(int n) { return gam(n) / VH; }  // its value-side fragment
  static_assert(G >= 32, "value tiles 2k and 2k + 1 share a group");
};

// The LDS slot a 32-token chunk is loaded into (Cfg::kSlot bytes).
template <int D, int BK, int BV, int GQ, int NG>
struct Raw {
  uint32_t* s;
};

// N consecutive words from LDS (N = 1, 2, 4, 8 or 16; 4 N-byte aligned up to 16).
template <int N>
__device__ __forceinline__ void lds_words(const uint32_t* p, uint32_t (&w)[N]) {
  if constexpr (N == 1) {
    w[0] = p[0];
  } else if constexpr (N == 2) {
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

constexpr float kPlainLog2 = 14.0f;
constexpr float kPlain = 16384.0f;

template <int D, int BK, int BV, int GQ, int NG, bool PG>
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
  uint32_t* ring;  // the wave's chunk slots
  // lane constants
  int lane, col, lg, hcol, slot;
  int gsel;            // value group selector of this lane's column (within a fragment)
  uint32_t lane16;     // 16 * lane: a lane's piece of a direct load
  int kofs, vofs;      // this lane's key / value words inside a chunk
  int vmofs[NF];       // value meta run of fragment f inside a chunk
  int kmofs;           // key meta run of this lane's fold items inside a group
  int kmoff[2];        // channels of those items (runs A and B)
  int fitem[IPL];
  float kscale, bscale;
  float m1;  // -1 in a register (split2)
  uint32_t m_slot1, m_slot2;  // all ones where bit 0 / bit 1 of slot is set
  // state
  f4 oacc[NT];
  float m_run, l_run;
  float m_even, m_odd;  // m_run less the classes' log2 factors (packed chunks)
  float m_plain;        // m_run - kPlainLog2 (fp16 window weights)
  float l_odd;          // sum of odd-class weights (scaled by kValOdd)
  float bias[NF];       // value-min term; odd class kept apart in bias_odd
  float bias_odd[NF];
  uint32_t bq[KP][KC][4];
  float beta_c;
  int cur_group;
  int hide;  // newest positions this lane's row must not see: T - 1 - its query token
  // paged cache: lane l holds entry tbase + l of the sequence's block-table
  // row (a window of 64 pages, moved on when a chunk leaves it)
  const int32_t* trow;
  int tab, tbase, maxp, npages, cpp_log2, hkv_, Hkv;
  bool bad;  // a table entry outside the pool was met: the partial is NaN

  __device__ void init(int lane_) {
    lane = lane_;
    lane16 = 16u * (uint32_t)lane_;
    m1 = opaque_m1();
    col = lane & 15;
    lg = lane >> 4;
    hcol = col / SL;
    slot = col % SL;
    m_slot1 = 0u - (uint32_t)(slot & 1);
    m_slot2 = 0u - (uint32_t)((slot >> 1) & 1);  // (from 4 columns per head: the quad position's bits)
    kofs = lane * 2 * KW;
    vofs = lane * C::NW;
    gsel = C::kVSplit ? slot >> 1 : slot;
#pragma unroll
    for (int f = 0; f < NF; ++f) vmofs[f] = (lg * NG + (f * C::VH + gsel) % NG) * 8;
#pragma unroll
    for (int i = 0; i < IPL; ++i) fitem[i] = lane + 64 * i;
    {
      const int r = lane % IPH, gg = r / KC, kc = r % KC;
      kmofs = r * 8;
      kmoff[0] = key_run0<D, BK>(gg, kc);
      kmoff[1] = kmoff[0] + kKeyOff<BK>;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) oacc[n] = f4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    m_even = kNegInf;
    m_odd = kNegInf;
    m_plain = kNegInf;
    l_run = 0.0f;
    l_odd = 0.0f;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      bias[f] = 0.0f;
      bias_odd[f] = 0.0f;
    }
    beta_c = 0.0f;
    cur_group = -1;
    hide = 0;
  }

  // Paged: the block-table window starting at page p0.
  __device__ __forceinline__ void set_table(const Geom& g, int b, int hkv, int p0) {
    trow = g.table + (int64_t)b * g.maxp;
    maxp = g.maxp;
    npages = g.npages;
    cpp_log2 = g.cpp_log2;
    hkv_ = hkv;
    Hkv = g.Hkv;
    bad = false;
    tbase = p0;
    tab = tbase + lane < maxp ? trow[tbase + lane] : 0;
  }

  // Slot of packed chunk ch in the buffers the bases point to: the chunk
  // itself for a dense unit; for a paged one, its page from the table window
  // (a page outside the pool reads page 0 and marks the partial bad).
  __device__ __forceinline__ int64_t slot_of(int ch) {
    if constexpr (!PG) {
      return ch;
    } else {
      const int page = ch >> cpp_log2;
      if ((unsigned)(page - tbase) >= 64u) {  // outside the window: move it here
        tbase = page;
        tab = tbase + lane < maxp ? trow[tbase + lane] : 0;
      }
      int pg = __builtin_amdgcn_readlane(tab, page - tbase);
      if ((unsigned)pg >= (unsigned)npages) {
        pg = 0;
        bad = true;
      }
      return (((int64_t)pg * Hkv + hkv_) << cpp_log2) + (ch & ((1 << cpp_log2) - 1));
    }
  }

  // Issues chunk ch's direct loads into slot r, nontemporal wherever the bytes
  // are read once per step (codes, value meta, and the key meta when a key
  // group is one chunk): loads that do not allocate in the caches stream HBM
  // faster.  A key group longer than a chunk has its meta read by each of its
  // chunks, so that one is loaded plain.  Earlier reads of the slot are
  // finished first.
  __device__ __forceinline__ void load(int ch, R& r) {
    const int64_t sl = slot_of(ch);
    const char* kc = reinterpret_cast<const char*>(kcodes + sl * (D * BK));
    const char* vc = reinterpret_cast<const char*>(vcodes + sl * (D * BV));
    const char* vm = reinterpret_cast<const char*>(vmeta + sl * (4 * NG * 8));
    const char* km = reinterpret_cast<const char*>(kmeta + (sl * kChunk) / G * D);
    const uint32_t base = lds_addr(r.s);
    lds_dma_begin();
    lds_copy<C::KB, true>(kc, base, lane16, lane);
    lds_copy<C::VB, true>(vc, base + C::kSlotV, lane16, lane);
    lds_copy<C::VMB, true>(vm, base + C::kSlotVM, lane16, lane);
    lds_copy<C::KMB, G == kChunk>(km, base + C::kSlotKM, lane16, lane);
  }

  // Waits until every chunk loaded but the last `ahead` is in its slot.
  template <int ahead>
  __device__ __forceinline__ void wait_chunks() const {
    wait_vm<ahead * C::NI>();
  }
  // Slot i of the ring (0 <= i < kRing).
  __device__ __forceinline__ R slot_at(int i) const { return R{ring + i * (C::kSlot / 4)}; }

  // A chunk's code words and value meta as this lane uses them.  They are read
  // from the slot when the chunk's turn comes, before the key-group fold, so
  // that the LDS latency of these reads overlaps the fold and the scores
  // instead of following the fold's barrier and the softmax.
  struct Words {
    uint32_t kw[2][KW];   // key code words of the two score tiles
    uint32_t vw[C::NW];   // value code words
    uint32_t vmA[NF][4];  // value (scale, min) of tokens 8 lg + 2 i (run A)
    uint32_t vmB[NF][4];  // ... and 8 lg + 2 i + 1 (run B)
  };
  __device__ __forceinline__ void read_words(const R& r, Words& cw) const {
    uint32_t w[2 * KW];
    lds_words<2 * KW>(r.s + kofs, w);
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      cw.kw[0][k] = w[k];
      cw.kw[1][k] = w[KW + k];
    }
    lds_words<C::NW>(r.s + C::kSlotV / 4 + vofs, cw.vw);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      // value meta of tokens 8 lg + j: even j feed B elements 2i (run A), odd
      // j elements 2i + 1 (run B)
      const uint4* st = reinterpret_cast<const uint4*>(r.s + C::kSlotVM / 4 + vmofs[f]);
      const uint4 x = st[0], y = st[1];
      cw.vmA[f][0] = x.x; cw.vmA[f][1] = x.z; cw.vmA[f][2] = y.x; cw.vmA[f][3] = y.z;
      cw.vmB[f][0] = x.y; cw.vmB[f][1] = x.w; cw.vmB[f][2] = y.y; cw.vmB[f][3] = y.w;
    }
  }

  // q' = q * 2^-E * key scale (hi/lo fp16 fragments in LDS) and beta' =
  // q * 2^-E . key min, for the key group starting in this chunk.
  // One fold item: channel runs A (qa, ma) and B (qb, mb) of 4 pairs each ->
  // the hi and lo fp16 pairs of q' and this item's part of beta.
  __device__ __forceinline__ float fold_item(const float4& qa, const float4& qb, const uint4& ma,
                                             const uint4& mb, uint32_t (&hp)[4],
                                             uint32_t (&lp)[4]) const {
    const float qA[4] = {qa.x, qa.y, qa.z, qa.w}, qBv[4] = {qb.x, qb.y, qb.z, qb.w};
    const uint32_t mA[4] = {ma.x, ma.y, ma.z, ma.w};
    const uint32_t mB[4] = {mb.x, mb.y, mb.z, mb.w};
    float beven = 0.0f, bodd = 0.0f;  // odd channels (their q' carries kKeyOddQ)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      split2(mul_lo(qA[e], mA[e]), mul_lo(qBv[e], mB[e]), m1, hp[e], lp[e]);
      if (e & 1) {
        bodd = mul_hi(qA[e], mA[e], bodd);
        bodd = mul_hi(qBv[e], mB[e], bodd);
      } else {
        beven = mul_hi(qA[e], mA[e], beven);
        beven = mul_hi(qBv[e], mB[e], beven);
      }
    }
    // beta = q . min with the channel factors taken back out
    return __builtin_fmaf(bodd, 1.0f / kKeyOddQ<BK>, beven * (1.0f / kKeyEvenQ<BK>));
  }

  // Direct form (one column per row): lane (row hcol, lane group lg) forms the
  // items (hcol, lg, kc) it consumes itself; beta sums over the lane groups.
  __device__ __forceinline__ void fold_direct(const R& r) {
    float bsum = 0.0f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int rr = lg * KC + kc;  // the item's run in the group's meta
      uint32_t w[8];
      lds_words<8>(r.s + C::kSlotKM / 4 + rr * 8, w);
      const int ca = key_run0<D, BK>(lg, kc), cb = ca + kKeyOff<BK>;
      const float4 qa = *reinterpret_cast<const float4*>(qfs + hcol * kQS<D> + ca);
      const float4 qb = *reinterpret_cast<const float4*>(qfs + hcol * kQS<D> + cb);
      uint32_t hp[4], lp[4];
      bsum += fold_item(qa, qb, make_uint4(w[0], w[2], w[4], w[6]),
                        make_uint4(w[1], w[3], w[5], w[7]), hp, lp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bq[0][kc][i] = hp[i];
        bq[1][kc][i] = lp[i];
      }
    }
    beta_c = xor_sum(xor_sum(bsum, 16), 32) * bscale;
  }

  __device__ __forceinline__ void fold(const R& r) {
    if constexpr (C::kDirectFold) {
      fold_direct(r);
      return;
    }
    // key meta of the group: entry e of an item is channel run A + e/2 (even
    // e) or run B + e/2 (odd); lanes past the fold items read an in-range run
    // too (the run depends on the item modulo a head's items)
    uint4 kmA, kmB;
    {
      uint32_t w[8];
      lds_words<8>(r.s + C::kSlotKM / 4 + kmofs, w);
      kmA = make_uint4(w[0], w[2], w[4], w[6]);
      kmB = make_uint4(w[1], w[3], w[5], w[7]);
    }
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      const int it = fitem[i];
      float bpart = 0.0f;
      // (when the items fill the wave exactly the test is compile-time true)
      if (C::ITEMS % 64 == 0 || it < C::ITEMS) {
        const int h = it / IPH, rr = it % IPH, gg = rr / KC, kc = rr % KC;
        const float4 qa = *reinterpret_cast<const float4*>(qfs + h * kQS<D> + kmoff[0]);
        const float4 qb = *reinterpret_cast<const float4*>(qfs + h * kQS<D> + kmoff[1]);
        uint32_t hp[4], lp[4];
        bpart = fold_item(qa, qb, kmA, kmB, hp, lp);
        qB[C::qb_slot(0, h, gg * KC + kc)] = make_uint4(hp[0], hp[1], hp[2], hp[3]);
        qB[C::qb_slot(1, h, gg * KC + kc)] = make_uint4(lp[0], lp[1], lp[2], lp[3]);
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
        const uint4 v = qB[C::qb_slot(part, hcol, lg * KC + kc)];
        bq[p][kc][0] = v.x; bq[p][kc][1] = v.y; bq[p][kc][2] = v.z; bq[p][kc][3] = v.w;
      }
    beta_c = beta_l[hcol] * bscale;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Scores.  A lane of column col and lane group lg holds, in the two score
  // tiles' accumulators, rows 4 lg + q of tile u: position j = 4 u + q of its
  // 8 positions 8 lg + j of the chunk.  With two or more columns per head
  // (kColSplit) the hi and lo parts of q' sit in neighbouring columns and are
  // added across the lane pair.
  //
  // With two or more columns per head (kShare) the lanes of a quad belong to
  // one head (a head's columns are consecutive and, from 4 up, 4-aligned)
  // and would all hold the same 8 scores.  Each takes NS of them instead for
  // the maximum, the exponentials and the sums: positions 2 i + k for quad
  // position i with 4 or more columns per head (NS = 2; other quads of the
  // same head do the same work), 4 slot + k with 2 (NS = 4).  The weights of
  // all 8 are gathered back from the quad with DPP moves.  The running sums
  // are then per lane and summed over the quad at the end.
  static constexpr bool kShare = SL >= 2;
  static constexpr bool kQuad = SL >= 4;
  static constexpr int NS = kQuad ? 2 : kShare ? 4 : 8;  // scores a lane works on

  static __device__ __forceinline__ float pair_add(float x) { return x + dpp<0xB1>(x); }

  // offset (in the lane group's 8 positions) of this lane's score k
  __device__ __forceinline__ int pos_of(int k) const {
    return kQuad ? 2 * (slot & 3) + k : kShare ? 4 * slot + k : k;
  }

  // This lane's raw dot products (hi + lo) from the score tiles.
  __device__ __forceinline__ void lane_scores(const f4 (&acc)[2], float (&x)[NS]) const {
    if constexpr (kQuad) {
      // the lane pair (quad positions 0, 1 or 2, 3) shares tile i / 2: add
      // hi + lo on it, then each lane keeps rows 2 (i % 2) + k
      float f[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = pair_add(bit_sel(m_slot2, acc[1][q], acc[0][q]));
#pragma unroll
      for (int k = 0; k < 2; ++k) x[k] = bit_sel(m_slot1, f[2 + k], f[k]);
    } else if constexpr (SL == 2) {  // lane slot keeps tile slot
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = bit_sel(m_slot1, pair_add(acc[1][q]), pair_add(acc[0][q]));
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) x[4 * u + q] = kColSplit ? pair_add(acc[u][q]) : acc[u][q];
    }
  }

  // Online softmax over a chunk's scores (exact running max; rescale only
  // when it grows).  Each lane tests its own scores; the cross-lane maximum
  // is only formed on the (rare) path where some lane sees a larger score.
  // kPacked: weights carry the value classes' factors (rows q < 2: kValEven,
  // q >= 2: kValOdd) and their sums are kept per class; otherwise plain.
  // p receives the weights of all 8 positions.
  __device__ __forceinline__ void rescale(float cm) {
    if constexpr (kShare) {
      cm = xor_max(cm, 1);
      if constexpr (kQuad) cm = xor_max(cm, 2);
    }
    cm = xor_max(cm, 16);
    cm = xor_max(cm, 32);
    const float m_new = fmaxf(m_run, cm);
    const float a = exp2_hw(m_run - m_new);
    m_run = m_new;
    m_even = m_new - kValEvenLog2<BV>;
    m_odd = m_new - kValOddLog2<BV>;
    m_plain = m_new - kPlainLog2;
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

  template <bool kPacked>
  __device__ __forceinline__ void softmax(const float (&s)[NS], float (&p)[2][4]) {
    float cm = s[0];
#pragma unroll
    for (int k = 1; k < NS; ++k) cm = fmaxf(cm, s[k]);
    if (__any(cm > m_run)) rescale(cm);
    float pm[NS];
    if constexpr (kPacked && kQuad) {  // a lane's two rows share a class
      const bool odd = slot & 1;
      const float mref = odd ? m_odd : m_even;
      pm[0] = exp2_hw(s[0] - mref);
      pm[1] = exp2_hw(s[1] - mref);
      const float add = pm[0] + pm[1];
      l_run += odd ? 0.0f : add;
      l_odd += odd ? add : 0.0f;
    } else {
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if constexpr (kPacked) {  // row (k % 4) < 2: even class
          pm[k] = exp2_hw(s[k] - ((k & 3) < 2 ? m_even : m_odd));
          if ((k & 3) < 2)
            l_run += pm[k];
          else
            l_odd += pm[k];
        } else {
          pm[k] = exp2_hw(s[k] - m_plain);
          l_run += pm[k];
        }
      }
    }
    if constexpr (kQuad) {
      quad_gather2(pm, p);  // position j = 4 u + q from quad lane j / 2
    } else if constexpr (SL == 2) {
      // tile u from the head's lane of slot u: quad positions (0, 1) or (2, 3)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        p[0][q] = dpp<0xA0>(pm[q]);
        p[1][q] = dpp<0xF5>(pm[q]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) p[u][q] = pm[4 * u + q];
    }
  }

  // Packed accumulation to real scale (codes were fp16 numbers c * 2^(L-24),
  // pairs carry kValEven) with its value-min term added; class sums folded.
  // Afterwards the state is plain (as the residual path needs), in units of
  // kPlain: the fp16 window's weights are 2^(s - m + kPlainLog2), so that
  // their hi/lo fp16 split keeps the lo part out of the subnormals down to
  // weights of 2^-17 (a small weight times a large fp16 value would otherwise
  // carry an absolute error of 2^-25 |v|).  Partials and sums share the
  // factor, so the combine's ratios are unchanged.
  __device__ __forceinline__ void to_real() {
    // the value-min term is summed over the four lane groups (token subsets)
    float btot[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const float bt = __builtin_fmaf(bias_odd[f], kPlain / kValOdd<BV>,
                                      bias[f] * (kPlain / kValEven<BV>));
      btot[f] = xor_sum(xor_sum(bt, 16), 32);
      bias[f] = 0.0f;
      bias_odd[f] = 0.0f;
    }
    constexpr float oscale = 16777216.0f / float(1 << kCodeLift<BV>) / kValEven<BV> * kPlain;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      // (split columns: the value-min term goes to the hi part's column only)
      const float bsum = C::kVSplit ? bit_sel(m_slot1, 0.0f, btot[C::frag(n)]) : btot[C::frag(n)];
#pragma unroll
      for (int q = 0; q < 4; ++q) oacc[n][q] = __builtin_fmaf(oacc[n][q], oscale, bsum);
    }
    l_run = __builtin_fmaf(l_odd, kPlain / kValOdd<BV>, l_run * (kPlain / kValEven<BV>));
    l_odd = 0.0f;
    m_even = m_run;
    m_odd = m_run;
  }

  // Key-side B fragments for fp16 keys: q * 2^-E in natural channel order
  // (element j of lane group g, k-chunk kc = channel 32 kc + 8 g + j), hi or
  // lo part.  (Before the residual window, to_real() brings the packed
  // accumulation to real scale; the two steps are apart because a mixed chunk
  // with packed values and fp16 keys needs only this one.)
  __device__ __forceinline__ void plain_query() {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const float4 qa = *reinterpret_cast<const float4*>(qfs + hcol * kQS<D> + 32 * kc + 8 * lg);
      const float4 qb = *reinterpret_cast<const float4*>(qfs + hcol * kQS<D> + 32 * kc + 8 * lg + 4);
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

  // fp16 windows.  Keys come straight from the key window's slot rows (slot
  // p % Rk); values are stored in the value consumer order (slot p % Rv), so
  // tile n's A operand is one 16-byte load per lane.
  // Value operands of the 32 positions t0 + [0, 32) (t0 a multiple of 32).
  __device__ __forceinline__ void window_values_load(int t0, int Rv, const uint16_t* vres,
                                                     uint4 (&va)[NT]) const {
    const uint4* vq = reinterpret_cast<const uint4*>(vres) +
                      (int64_t)((t0 % Rv) / kChunk) * (D / 16) * 64 + lane;
#pragma unroll
    for (int n = 0; n < NT; ++n) va[n] = vq[n * 64];
  }
  // Weighted sum of those values (real-scale accumulators); slots past n_tok
  // are zeroed in registers: their weight is 0, and the window may hold
  // anything there.
  __device__ __forceinline__ void window_values_mma(const uint4 (&va)[NT], int t0, int n_tok,
                                                    const float (&p)[2][4]) {
    uint32_t vmask[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 8 * lg + 2 * i;
      vmask[i] = (t < n_tok ? 0x0000ffffu : 0u) | (t + 1 < n_tok ? 0xffff0000u : 0u);
    }
    uint32_t bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      split2(p[i >> 1][2 * (i & 1)], p[i >> 1][2 * (i & 1) + 1], m1, bh[i], bl[i]);
    if constexpr (C::kVSplit) {  // this lane's column takes the hi or the lo part
#pragma unroll
      for (int i = 0; i < 4; ++i) bh[i] ^= (bl[i] ^ bh[i]) & m_slot1;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint32_t a[4] = {va[n].x & vmask[0], va[n].y & vmask[1], va[n].z & vmask[2],
                             va[n].w & vmask[3]};
      oacc[n] = mfma(a, bh, oacc[n]);
      if constexpr (!C::kVSplit) oacc[n] = mfma(a, bl, oacc[n]);
    }
  }
  // Scores of positions t0 + [0, 32) from the key window (B fragments from
  // plain_query()); positions this lane's row must not see get -inf.
  __device__ __forceinline__ void window_scores(int t0, int n_tok, int Rk, const uint16_t* kres,
                                                float (&s)[NS]) {
    // scores: tile u row r = token key_row_token(u, r)
    const float kscale_r = bscale;  // keys are real fp16 values here
    f4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tin = t0 + key_row_token(u, col);
      const int slot_in = (tin < n_tok ? tin : n_tok - 1) % Rk;
      const uint4* krow = reinterpret_cast<const uint4*>(kres + (int64_t)slot_in * D);
      acc[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint4 kv = krow[4 * kc + lg];
        const uint32_t a[4] = {kv.x, kv.y, kv.z, kv.w};
        acc[u] = mfma(a, bq[0][kc], acc[u]);
        if constexpr (!kColSplit) acc[u] = mfma(a, bq[1][kc], acc[u]);
      }
    }
    float x[NS];
    lane_scores(acc, x);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const bool valid = t0 + 8 * lg + pos_of(k) < n_tok - hide;
      s[k] = valid ? x[k] * kscale_r : kNegInf;
    }
  }

  // Residual chunk: fp16 keys and values of positions t0 + [0, 32) (those >=
  // n_tok masked).
  __device__ __forceinline__ void process_residual(int t0, int n_tok, int Rk, int Rv,
                                                   const uint16_t* kres,
                                                   const uint16_t* vres) {
    uint4 va[NT];
    window_values_load(t0, Rv, vres, va);  // first: the loads overlap the score MFMAs
    float s[NS];
    window_scores(t0, n_tok, Rk, kres, s);
    float p[2][4];
    softmax<false>(s, p);
    window_values_mma(va, t0, n_tok, p);
  }

  // Mixed chunk ch with packed keys and fp16 values (the key window is the
  // shorter one): scores from the codes, weights plain (the accumulators are
  // at real scale), values from the value window.
  __device__ __forceinline__ void process_mixed_keys(int ch, const R& r, int n_tok, int Rv,
                                                     const uint16_t* vres) {
    uint4 va[NT];
    window_values_load(ch * kChunk, Rv, vres, va);
    Words cw;
    read_words(r, cw);
    float s[NS];
    packed_scores<true>(ch, r, cw, n_tok - 1 - hide, s);
    float p[2][4];
    softmax<false>(s, p);
    window_values_mma(va, ch * kChunk, n_tok, p);
  }

  // Mixed chunk ch with fp16 keys and packed values: scores from the key
  // window (after plain_query()), weights in the packed classes (the
  // accumulators are still at code scale), values from the codes.
  __device__ __forceinline__ void process_mixed_values(int ch, const R& r, int n_tok, int Rk,
                                                       const uint16_t* kres) {
    Words cw;
    read_words(r, cw);
    float s[NS];
    window_scores(ch * kChunk, n_tok, Rk, kres, s);
    float p[2][4];
    softmax<true>(s, p);
    packed_values(cw, p);
  }

  // kMask: positions after last_vis (this lane's row, 32-token chunk ch) get
  // score -inf (the causal mask of a multi-token query; their codes and meta
  // are real cache data, so their weight 0 is exact).
  template <bool kMask = false>
  __device__ __forceinline__ void process(int ch, const R& r, int last_vis = 0) {
    Words cw;
    read_words(r, cw);
    float s[NS];
    packed_scores<kMask>(ch, r, cw, last_vis, s);
    float p[2][4];
    softmax<true>(s, p);
    packed_values(cw, p);
  }

  // Scores of packed chunk ch (folding the key group's meta when it starts):
  // s = 2^(E+24) * (codes x q') + beta; with kMask, positions after last_vis
  // get -inf.
  template <bool kMask>
  __device__ __forceinline__ void packed_scores(int ch, const R& r, const Words& cw,
                                                int last_vis, float (&s)[NS]) {
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
    f4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t a[KC][4];
      unpack_keys<D, BK>(cw.kw[u], a);
      acc[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        acc[u] = mfma(a[kc], bq[0][kc], acc[u]);
        if constexpr (!kColSplit) acc[u] = mfma(a[kc], bq[1][kc], acc[u]);
      }
    }
    float x[NS];
    lane_scores(acc, x);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      s[k] = __builtin_fmaf(x[k], kscale, beta_c);
      if constexpr (kMask)
        s[k] = ch * kChunk + 8 * lg + pos_of(k) <= last_vis ? s[k] : kNegInf;
    }
  }

  // Weighted sum of a packed chunk's values (code-scale accumulators, weights
  // in the packed classes) and its value-min term.
  __device__ __forceinline__ void packed_values(const Words& cw, const float (&p)[2][4]) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t(&mA)[4] = cw.vmA[f];
      const uint32_t(&mB)[4] = cw.vmB[f];
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // elements 2i (run A) and 2i+1 (run B) = score tile i/2, rows 2(i%2), +1;
        // odd i is the odd class
        const float pa = p[i >> 1][2 * (i & 1)], pb = p[i >> 1][2 * (i & 1) + 1];
        split2(mul_lo(pa, mA[i]), mul_lo(pb, mB[i]), m1, bh[i], bl[i]);
        float& bacc = (i & 1) ? bias_odd[f] : bias[f];
        bacc = mul_hi(pa, mA[i], bacc);
        bacc = mul_hi(pb, mB[i], bacc);
      }
      if constexpr (C::kVSplit) {  // this lane's column takes the hi or the lo part
#pragma unroll
        for (int i = 0; i < 4; ++i) bh[i] ^= (bl[i] ^ bh[i]) & m_slot1;
      }
      if constexpr (BV != 4) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if (C::frag(n) != f) continue;  // compile-time
          uint32_t a[4];
          unpack_value_tile<BV>(cw.vw, n, a);
          oacc[n] = mfma(a, bh, oacc[n]);
          if constexpr (!C::kVSplit) oacc[n] = mfma(a, bl, oacc[n]);
        }
      } else {
        // 4-bit tiles in pairs (a group holds at least two 16-channel tiles)
#pragma unroll
        for (int n = 0; n < NT; n += 2) {
          if (C::frag(n) != f) continue;  // compile-time
          uint32_t a0[4], a1[4];
          unpack_value_tiles2<BV>(cw.vw, n, a0, a1);
          oacc[n] = mfma(a0, bh, oacc[n]);
          oacc[n + 1] = mfma(a1, bh, oacc[n + 1]);
          if constexpr (!C::kVSplit) {
            oacc[n] = mfma(a0, bl, oacc[n]);
            oacc[n + 1] = mfma(a1, bl, oacc[n + 1]);
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Work of a sequence in this format: packed 32-token chunks (one work unit
// each) followed by the 32-token chunks of its fp16 residual window (rw work
// units each: rw ~ fp16 bytes / packed bytes per token, so that work units
// stand for equal HBM traffic).  The decomposition itself (kvq_device.h) cuts
// the flat list of all units' work into equal shares, one per worker wave.
// ---------------------------------------------------------------------------
// With separate key and value windows the two packed lengths differ: chunks
// below both are packed, chunks between them mixed (packed for one tensor,
// in the window for the other; rw work units like a residual chunk), the
// rest residual.
__device__ __forceinline__ SeqWork seq_work_of(const DecodeLaunch& L, int n) {
  SeqWork sw{0, 0, 0, 0};
  if (n <= 0 || n > L.g.C || n > L.max_seq_len) return sw;
  const int lqk = packed_len(n, L.g.R), lqv = packed_len(n, L.g.Rv);
  const int lo = min(lqk, lqv), hi = max(lqk, lqv);
  sw.n = n;
  sw.nq = lo / kChunk;
  sw.nm = (hi - lo) / kChunk;
  sw.keys_packed = lqk > lqv;
  sw.nr = sw.nm + (n - hi + kChunk - 1) / kChunk;
  sw.w = sw.nq + sw.nr * L.rw;
  return sw;
}

__device__ __forceinline__ SeqWork seq_work(const DecodeLaunch& L, int b) {
  return seq_work_of(L, L.seq_lens[b]);
}

// Row j of unit (b, hkv) is query token j / (Hq/Hkv) of the last T, head
// hkv * Hq/Hkv + j % (Hq/Hkv): q and out are [B][T][Hq][D].
__device__ __forceinline__ int64_t qrow(const DecodeLaunch& L, int b, int hkv, int j) {
  const int gr = L.g.Hq / L.g.Hkv;
  return ((int64_t)b * L.T + j / gr) * L.g.Hq + hkv * gr + j % gr;
}

struct KiviWork {
  using Launch = DecodeLaunch;
  static constexpr bool kRotateOut = false;
  static __device__ __forceinline__ int64_t row(const DecodeLaunch& L, int b, int hkv, int j) {
    return qrow(L, b, hkv, j);
  }
  static __device__ __forceinline__ SeqWork work_of(const DecodeLaunch& L, int n) {
    return seq_work_of(L, n);
  }
};

template <int D, int BK, int BV, int GQ, int NG>
constexpr int kWaveSmem = GQ * kQS<D> * 4 + Cfg<D, BK, BV, GQ, NG>::kWaveLds;

// Sets up the wave for unit (b, hkv) and issues the loads of the range's first
// packed chunk into ra (before anything else, so that their latency overlaps
// the query's).
template <int D, int BK, int BV, int GQ, int NG, bool PG>
__device__ __forceinline__ void seg_begin(const DecodeLaunch& L, int b, int hkv, const SegRange& r,
                                          char* smem, int lane, PackedWave<D, BK, BV, GQ, NG, PG>& w,
                                          Raw<D, BK, BV, GQ, NG>& ra) {
  using C = Cfg<D, BK, BV, GQ, NG>;
  const Geom& g = L.g;
  char* wl = smem + GQ * kQS<D> * 4;
  // dense: the unit's rows (chunk slot = chunk); paged: the pools
  const int64_t unit = PG ? 0 : (int64_t)b * g.Hkv + hkv;
  w.kcodes = L.cache.k_codes + unit * g.C * C::WR;
  w.kmeta = reinterpret_cast<const uint32_t*>(L.cache.k_meta) + unit * (g.C / C::G) * D;
  w.vcodes = L.cache.v_codes + unit * (g.C / kVBlock) * D * BV;
  w.vmeta = reinterpret_cast<const uint32_t*>(L.cache.v_meta) +
            unit * (g.C / kVBlock) * NG * kVBlock;
  w.qfs = reinterpret_cast<float*>(smem);
  w.qB = reinterpret_cast<uint4*>(wl);
  w.beta_l = reinterpret_cast<float*>(wl + C::kQB);
  w.ring = reinterpret_cast<uint32_t*>(wl + C::kQB + C::kBetaB);
  w.init(lane);
  ra.s = w.ring;
  if constexpr (PG) w.set_table(g, b, hkv, r.pc0 >> g.cpp_log2);
  if (r.pc0 < r.pc1) w.load(r.pc0, ra);
}

// Runs the range of unit (b, hkv) -> partial p, seg_begin having been done.
template <int D, int BK, int BV, int GQ, int NG, bool PG>
__device__ __forceinline__ void seg_run(const DecodeLaunch& L, int b, int hkv, const SeqWork& sw,
                                        const SegRange& r, int p, char* smem, int lane,
                                        PackedWave<D, BK, BV, GQ, NG, PG>& w,
                                        Raw<D, BK, BV, GQ, NG>& ra) {
  using C = Cfg<D, BK, BV, GQ, NG>;
  using R = Raw<D, BK, BV, GQ, NG>;
  constexpr int NT = C::NT;
  constexpr int QPH = D / 64;  // query values per lane and head
  constexpr int DP = D + kPartPad;
  const Geom& g = L.g;
  const int64_t unit = (int64_t)b * g.Hkv + hkv;
  float* part_base = L.ws + (int64_t)p * GQ * DP;
  float* qfs = reinterpret_cast<float*>(smem);  // [GQ][kQS] q * 2^-E_h
  const int pc0 = r.pc0, pc1 = r.pc1, rk0 = r.rk0, rk1 = r.rk1;
  constexpr int kRing = C::kRing;
  // query of the unit's GQ heads; per-head exponent E with max|q| < 2^E so
  // that q * 2^-E * key scale fits fp16.  The softmax scale (sm_scale log2 e)
  // is not folded into q: it multiplies the finished scores (kscale, bscale),
  // so q * 2^-E stays the fp16 query exactly, q' = q 2^-E scale is an exact
  // 22-bit product and its hi/lo split is exact too.
  int eh[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const uint16_t* qg = L.q + qrow(L, b, hkv, h) * D;
    float qv[QPH];
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < QPH; ++k) {
      qv[k] = h2f(qg[lane + 64 * k]);
      mx = fmaxf(mx, fabsf(qv[k]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = xor_max(mx, off);
    int e = 0;
    if (mx > 0.0f) (void)frexpf(mx, &e);
    eh[h] = e;
#pragma unroll
    for (int k = 0; k < QPH; ++k)  // channel lane + 64 k has the parity of lane
      qfs[h * kQS<D> + lane + 64 * k] =
          ldexpf(qv[k], -e) * ((lane & 1) ? kKeyOddQ<BK> : kKeyEvenQ<BK>);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  int e_mine = 0;
#pragma unroll
  for (int h = 0; h < GQ; ++h)
    if (w.hcol == h) e_mine = eh[h];
  // codes are the fp16 numbers c * 2^(L - 24), pairs carry the key-side
  // factor; scores in log2 units
  w.kscale = ldexpf(L.scale_log2, e_mine + 24 - kKeyAccLog2<BK> - kCodeLift<BK>);
  w.bscale = ldexpf(L.scale_log2, e_mine);

  // rows of query token i (of the last T) do not see the newest T - 1 - i
  // positions; packed chunks holding a position past n - T are processed
  // apart, with the mask (never for a single query token: the newest packed
  // position is at most n - 2)
  w.hide = L.T - 1 - w.hcol / (g.Hq / g.Hkv);
  const int last_vis = sw.n - 1 - w.hide;
  const int pm = min(pc1, max(pc0, (sw.n - L.T + 1) / kChunk));
  if (pc0 < pm) {
    // chunk pc0 + i in ring slot i % kRing (seg_begin loaded pc0 into slot
    // 0); while one is used, up to kRing - 1 later ones are in flight
    const int last = pm - 1;
    if constexpr (kRing == 2) {
      // pairs, so that the compiler can schedule one chunk's fold against the
      // previous chunk's value products; ra holds chunk ch on entry
      R rb = w.slot_at(1);
      int ch = pc0;
      for (; ch < last; ch += 2) {
        w.load(ch + 1, rb);
        w.template wait_chunks<1>();
        w.process(ch, ra);
        if (ch + 2 <= last) {
          w.load(ch + 2, ra);
          w.template wait_chunks<1>();
        } else {
          w.template wait_chunks<0>();
        }
        w.process(ch + 1, rb);
      }
      if (ch == last) {  // odd count: the last chunk is in ra
        w.template wait_chunks<0>();
        w.process(ch, ra);
      }
    } else {
#pragma unroll
      for (int k = 1; k < kRing - 1; ++k)
        if (pc0 + k <= last) {
          R rk = w.slot_at(k);
          w.load(pc0 + k, rk);
        }
      int ch = pc0, si = 0;
      for (; ch + kRing - 1 <= last; ++ch) {  // steady: kRing - 1 chunks ahead
        R rn = w.slot_at(si == 0 ? kRing - 1 : si - 1);
        w.load(ch + kRing - 1, rn);
        w.template wait_chunks<kRing - 1>();
        w.process(ch, w.slot_at(si));
        si = si + 1 == kRing ? 0 : si + 1;
      }
      for (; ch <= last; ++ch) {  // the chunks already in flight
        if (kRing == 3 && ch < last)
          w.template wait_chunks<1>();
        else
          w.template wait_chunks<0>();
        w.process(ch, w.slot_at(si));
        si = si + 1 == kRing ? 0 : si + 1;
      }
    }
  }
  for (int ch = pm; ch < pc1; ++ch) {  // ra holds chunk pc0 if pm == pc0
    if (ch != pc0) w.load(ch, ra);
    w.template wait_chunks<0>();
    w.template process<true>(ch, ra, last_vis);
  }
  // chunks past the packed ones: k < nm mixed (chunk nq + k), then residual
  // (positions (nq + k) * 32 ..); both are in the windows' slots p % Rk, p % Rv
  const uint16_t* kres = L.cache.k_res + unit * g.R * D;
  const uint16_t* vres = L.cache.v_res + unit * g.Rv * D;
  bool real = false;  // accumulators at real scale
  const int mk1 = min(rk1, sw.nm);
  if (rk0 < mk1) {
    if (sw.keys_packed) {
      w.to_real();
      real = true;
      for (int k = rk0; k < mk1; ++k) {
        w.load(sw.nq + k, ra);
        w.template wait_chunks<0>();
        w.process_mixed_keys(sw.nq + k, ra, sw.n, g.Rv, vres);
      }
    } else {
      w.plain_query();
      for (int k = rk0; k < mk1; ++k) {
        w.load(sw.nq + k, ra);
        w.template wait_chunks<0>();
        w.process_mixed_values(sw.nq + k, ra, sw.n, g.R, kres);
      }
    }
  }
  const int r0 = max(rk0, sw.nm);
  if (r0 < rk1) {
    if (!real) w.to_real();
    real = true;
    if (sw.keys_packed || rk0 >= mk1) w.plain_query();  // unless mixed chunks did it
    for (int k = r0; k < rk1; ++k)
      w.process_residual((sw.nq + k) * kChunk, sw.n, g.R, g.Rv, kres, vres);
  }

  // partial: O (value-min term included), max, sum of this wave's tokens
  if (!real) w.to_real();
  float l_run = w.l_run;
  if constexpr (PackedWave<D, BK, BV, GQ, NG, PG>::kShare) {  // per-lane sums
    l_run = xor_sum(l_run, 1);
    if constexpr (PackedWave<D, BK, BV, GQ, NG, PG>::kQuad) l_run = xor_sum(l_run, 2);
  }
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);
  if constexpr (PG) {
    if (w.bad) {  // finite max, NaN sum and values: the combine's output is NaN
      w.m_run = 0.0f;
      l_run = __builtin_nanf("");
#pragma unroll
      for (int n = 0; n < NT; ++n) w.oacc[n] = f4{l_run, l_run, l_run, l_run};
    }
  }
  float* part = part_base + w.hcol * DP;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    f4 o = w.oacc[n];
    if constexpr (C::kVSplit) {  // hi + lo parts: neighbouring columns
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = PackedWave<D, BK, BV, GQ, NG, PG>::pair_add(o[q]);
      if (w.slot & 1) continue;
    }
    if (C::gam(n) % C::VH != w.gsel) continue;
    *reinterpret_cast<float4*>(part + 16 * n + 4 * w.lg) = make_float4(o[0], o[1], o[2], o[3]);
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
template <int D, int BK, int BV, int GQ, int NG, bool PG>
__device__ __forceinline__ void unit_segment(const DecodeLaunch& L, int b, int hkv,
                                             const SeqWork& sw, int xu, int x0, int x1, int p,
                                             char* smem, int lane) {
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
  PackedWave<D, BK, BV, GQ, NG, PG> w;
  Raw<D, BK, BV, GQ, NG> ra;
  seg_begin<D, BK, BV, GQ, NG, PG>(L, b, hkv, r, smem, lane, w, ra);
  seg_run<D, BK, BV, GQ, NG, PG>(L, b, hkv, sw, r, p, smem, lane, w, ra);
}

// One wave per workgroup; grid = the number of worker waves.
template <int D, int BK, int BV, int GQ, int NG, bool PG>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeLaunch L) {
  __shared__ __attribute__((aligned(16))) char smem[kWaveSmem<D, BK, BV, GQ, NG>];
  const int lane = threadIdx.x;
  const int w = blockIdx.x, nw = gridDim.x;
  const BatchWork bw = batch_work<KiviWork>(L, lane);  // one read of the lengths
  const int total = bw.total;
  const int cpw = (total + nw - 1) / nw;
  const int x0 = w * cpw;
  const int x1 = min(total, x0 + cpw);
  int x = x0;
  while (x < x1) {
    int b, base;
    wave_find_seq<KiviWork>(L, bw, lane, x, b, base);
    b = __builtin_amdgcn_readfirstlane(b);
    base = __builtin_amdgcn_readfirstlane(base);
    const SeqWork sw = seq_work(L, b);
    const int hkv = (x - base) / sw.w;
    const int xu = base + hkv * sw.w;
    unit_segment<D, BK, BV, GQ, NG, PG>(L, b, hkv, sw, xu, x0, x1, w + b * L.g.Hkv + hkv, smem,
                                    lane);
    x = xu + sw.w;
  }
  wait_vm<0>();  // no direct load into this wave's LDS outlives it
}

// Worker waves the partial kernel of this instantiation is launched with:
// resident waves per compute unit (from the kernel's resources) x CUs, cached
// per device.
template <int D, int BK, int BV, int GQ, int NG, bool PG>
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
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &nb, decode_partial_kernel<D, BK, BV, GQ, NG, PG>, 64, 0);
  if (e != hipSuccess) return e;
  if (nb < 1) nb = 1;
  const int w = nb * cus;
  if (dev >= 0 && dev < 64) cache[dev].store(w, std::memory_order_relaxed);
  *out = w;
  return hipSuccess;
}

// Op: 0 = launch the partial kernel, 1 = query its worker count.
template <int D, int BK, int BV, int GQ, int NG, bool PG>
hipError_t run(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  if (op == 1) return workers_of<D, BK, BV, GQ, NG, PG>(cus, workers);
  decode_partial_kernel<D, BK, BV, GQ, NG, PG><<<dim3(L.n_workers), 64, 0, st>>>(L);
  return hipGetLastError();
}

template <int D, int BK, int BV, int GQ, bool PG>
hipError_t dispatch_ng(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  switch (D / L.g.G) {
    case 1: return run<D, BK, BV, GQ, 1, PG>(L, op, cus, workers, st);
    case 2: return run<D, BK, BV, GQ, 2, PG>(L, op, cus, workers, st);
    case 4:
      if constexpr (D == 128) return run<D, BK, BV, GQ, 4, PG>(L, op, cus, workers, st);
      [[fallthrough]];
    default: return hipErrorInvalidValue;
  }
}

template <int D, int BK, int BV, bool PG>
hipError_t dispatch_gq(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  switch (L.gq) {
    case 1: return dispatch_ng<D, BK, BV, 1, PG>(L, op, cus, workers, st);
    case 2: return dispatch_ng<D, BK, BV, 2, PG>(L, op, cus, workers, st);
    case 4: return dispatch_ng<D, BK, BV, 4, PG>(L, op, cus, workers, st);
    case 8: return dispatch_ng<D, BK, BV, 8, PG>(L, op, cus, workers, st);
    case 16: return dispatch_ng<D, BK, BV, 16, PG>(L, op, cus, workers, st);
    default: return hipErrorInvalidValue;
  }
}

// The partial kernels of one head dim, key width and cache form (each
// translation unit that includes this file instantiates one such set).
template <int D, int BK, bool PG>
hipError_t dispatch_bv(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  switch (L.g.bV) {
    case 2: return dispatch_gq<D, BK, 2, PG>(L, op, cus, workers, st);
    case 4: return dispatch_gq<D, BK, 4, PG>(L, op, cus, workers, st);
    case 8: return dispatch_gq<D, BK, 8, PG>(L, op, cus, workers, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace kvq
