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
// (a 4-bit scale is at most 8734, a 2-bit one is not scaled up).  8-bit
// fields are shifted down to bit 0 of their half before the mask, so every
// pair is code * 2^-24 and no factor is needed.
template <int BK> constexpr float kKeyEvenQ = BK == 4 ? 4.0f : 1.0f;
template <int BK> constexpr float kKeyOddQ = BK == 8 ? 1.0f : 0.25f;
template <int BK> constexpr int kKeyAccLog2 = BK == 4 ? 2 : 0;

// Value side, likewise: the odd pairs of a value word (VGPR e odd: tokens
// 8g + 2e, 8g + 2e + 1 with e odd, i.e. score registers q = 2, 3) come out of
// their mask as code * 16 (4-bit) or * 4 (2-bit) * 2^-24.  Their softmax
// weights are taken 4x smaller (2^(s - m - 2)) and the even pairs' weights
// kValEven times larger, so every pair contributes kValEven * p * code * dV.
// (4 * 8734 and 43669 stay inside fp16.)  8-bit pairs are all code * 2^-24:
// both classes keep factor 1.
template <int BV> constexpr float kValEven = BV == 4 ? 4.0f : 1.0f;
template <int BV> constexpr float kValOdd = BV == 8 ? 1.0f : 0.25f;
template <int BV> constexpr float kValEvenLog2 = BV == 4 ? 2.0f : 0.0f;
template <int BV> constexpr float kValOddLog2 = BV == 8 ? 0.0f : -2.0f;

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
  } else if constexpr (BK == 4) {
    // field s of a half: (w >> 8 (s/2)) masked at bits 4 (s%2)
#pragma unroll
    for (int wi = 0; wi < kKW<D, BK>; ++wi)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[wi][s] = (w[wi] >> (8 * (s >> 1))) & ((s & 1) ? 0x00F000F0u : 0x000F000Fu);
  } else {
    // k-chunk kc from words 2kc + (s/2): pair s is that word >> 8 (s%2),
    // bytes 0 and 2 of the result
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc)
#pragma unroll
      for (int s = 0; s < 4; ++s) a[kc][s] = (w[2 * kc + (s >> 1)] >> (8 * (s & 1))) & 0x00FF00FFu;
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
// uniform: every length equals max_seq_len.
struct BatchWork {
  int c, inc, head_total, total;
  int n;  // lane b < 64: length of sequence b
  bool uniform;
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
  bw.uniform = __ballot(n != L.max_seq_len) == 0;
  for (int b0 = 64; b0 < L.g.B; b0 += 64) {  // batches beyond 64 sequences
    const int nb = b0 + lane < L.g.B ? L.seq_lens[b0 + lane] : L.max_seq_len;
    int s = b0 + lane < L.g.B ? Fmt::work_of(L, nb).w * L.g.Hkv : 0;
    s = wave_scan_incl(s);
    bw.total += __builtin_amdgcn_readlane(s, 63);
    bw.uniform = bw.uniform && __ballot(nb != L.max_seq_len) == 0;
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
// One workgroup per (KV head, sequence): merges the partials of the unit and
// writes its GQ outputs:
//   M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L.
// The unit's partials are contiguous (indices w + u for consecutive waves w).
// Each thread owns one float4 of the output and a 1/P share of the partials
// and merges them as a stream (running max, rescale when it grows), so the
// (m, l, o) loads of a partial do not wait for any reduction; the P shares are
// then merged through LDS.  Empty partials (m = -inf) carry weight 0.
template <class Fmt, int D, int GQ>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(typename Fmt::Launch L) {
  constexpr int DP = D + kPartPad;
  constexpr int NO = GQ * D / 4;                          // float4 outputs of the unit
  constexpr int P = NO >= kThreads ? 1 : kThreads / NO;   // partial shares per output
  constexpr int OPT = NO >= kThreads ? NO / kThreads : 1;  // outputs per thread
  constexpr int U = 4;                                     // partials in flight per thread
  static_assert(NO % kThreads == 0 || kThreads % NO == 0, "outputs tile the workgroup");
  constexpr bool kRotate = Fmt::kRotateOut;  // out = H o per head (64 channels)
  static_assert(!kRotate || (D == 64 && OPT == 1), "rotation covers one 64-channel head");
  __shared__ int red[2 * kThreads / 64];
  __shared__ float4 s_o[kThreads];
  __shared__ float2 s_ml[kThreads];
  __shared__ float s_rot[kRotate ? GQ * D : 1];
  const auto& g = L.g;
  const int hkv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = L.seq_lens[b];
  if (n < 0 || n > g.C || n > L.max_seq_len) {
    for (int i = tid; i < GQ * D; i += kThreads)
      L.out[Fmt::row(L, b, hkv, i / D) * D + i % D] = 0x7e00;  // NaN
    return;
  }
  if (n == 0) {
    for (int i = tid; i < GQ * D; i += kThreads) L.out[Fmt::row(L, b, hkv, i / D) * D + i % D] = 0;
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
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;  // a row that sees no position: 0
    const int64_t o = Fmt::row(L, b, hkv, oh) * D + oc;
    if constexpr (kRotate) {
      // out_c = sum_j H[c][j] o_j, H[c][j] = (-1)^popcount(c & j) / 8
      if (share == 0) {
        s_rot[oh * D + oc + 0] = O.x * inv;
        s_rot[oh * D + oc + 1] = O.y * inv;
        s_rot[oh * D + oc + 2] = O.z * inv;
        s_rot[oh * D + oc + 3] = O.w * inv;
      }
      __syncthreads();
      if (share == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = oc + e;
          float acc = 0.0f;
          for (int j = 0; j < D; ++j) {
            const float r = s_rot[oh * D + j];
            acc += (__builtin_popcount(c & j) & 1) ? -r : r;
          }
          L.out[o + e] = f2h(acc * 0.125f);
        }
      }
    } else if (share == 0) {
      L.out[o + 0] = f2h(O.x * inv);
      L.out[o + 1] = f2h(O.y * inv);
      L.out[o + 2] = f2h(O.z * inv);
      L.out[o + 3] = f2h(O.w * inv);
    }
  }
}
}  // namespace
}  // namespace kvq
