// kvq_quant.hip — group quantization into the packed layout, residual append
// with lazy flush, and the prefill residual copy (gfx950).
//
// The group quantizer follows the "Quantization Format: KV1.cpp BQ2_0" section
// of the KV1-1.2B model card (affine codes, scale = (max - min) / (2^b - 1) in
// fp32, scale and min rounded to fp16 and those rounded values used for the
// codes, round half to even, clamp), generalised from 2 to b bits.  Keys are
// grouped per channel over G tokens and values per token over G channels, as
// the KIVI repository page ("core capabilities", "Overview") describes.
//
// Bit-exactness: this file is compiled with -ffp-contract=off and without
// fast-math; '/' on float is the correctly rounded IEEE division, rintf is
// v_rndne_f32 (ties to even) and the fp16 conversion rounds to nearest even.
#include "kvq_internal.h"

namespace kvq {
namespace {


// Scale and min of one group from its fp32 min and max.
struct GroupParams {
  uint16_t d16, m16;
  float scale, minv;
};

__device__ __forceinline__ GroupParams group_params(float mn, float mx,
                                                    int bits) {
  // a zero min or max is taken as +0 so the stored bits do not depend on the
  // order in which -0 and +0 were seen
  mn = (mn == 0.0f) ? 0.0f : mn;
  mx = (mx == 0.0f) ? 0.0f : mx;
  const float levels = (float)((1 << bits) - 1);
  const float range = mx - mn;      // IEEE fp32 subtract
  const float d32 = range / levels;  // IEEE fp32 divide
  GroupParams p;
  p.d16 = f2h(d32);
  if ((p.d16 & 0x7fffu) == 0) p.d16 = 0;
  p.m16 = f2h(mn);
  p.scale = h2f(p.d16);
  p.minv = h2f(p.m16);
  return p;
}

__device__ __forceinline__ uint32_t group_code(float x, const GroupParams& p,
                                               int bits) {
  if (p.scale == 0.0f) return 0u;
  const float y = (x - p.minv) / p.scale;  // fp32 subtract, IEEE divide
  float r = rintf(y);                      // round half to even
  const float levels = (float)((1 << bits) - 1);
  r = fminf(fmaxf(r, 0.0f), levels);
  return (uint32_t)r;
}

// Place of channel c inside a key group's D meta entries: entry 8 r + e is the
// channel that element e of k-chunk r (lane group g = r / (D/32), chunk
// kc = r % (D/32)) feeds: g D/4 + base(kc) + e/2 + off (e%2).  Inverse:
// within its slice, channel cs sits in word cs / (32/BITS) at field s'; the
// field's half (low / high 16 bits) gives e % 2, its place in the half gives
// the chunk and e / 2.  For 8 bits base = 8 kc and off = 4 (as for 4 bits):
// cs = 8 kc + p gives e = 2 (p % 4) + p / 4.
template <int BITS>
__device__ __forceinline__ int key_meta_entry(int c, int D) {
  const int g = c / (D / 4), cs = c % (D / 4);
  if constexpr (BITS == 8) {
    const int kc = cs / 8, p = cs % 8;
    return 8 * (g * (D / 32) + kc) + 2 * (p % 4) + p / 4;
  } else {
    constexpr int per = 32 / BITS;  // fields per word
    constexpr int hp = per / 2;     // fields per half word
    const int wi = cs / per, sp = cs % per;
    const int half = sp / hp, s = sp % hp;
    const int kc = wi * (hp / 4) + s / 4;
    const int r = g * (D / 32) + kc;
    return 8 * r + 2 * (s % 4) + half;
  }
}

// Channel (within its lane group's slice) of field f of slice word ws: 2 and
// 4 bits in channel order; 8 bits: word 2 kc + s holds 8 kc + 2 s + (0, 1, 4,
// 5)[f], the order in which the decode kernel's byte masks feed its pairs.
template <int BITS>
__device__ __forceinline__ int key_field_channel(int ws, int f) {
  if constexpr (BITS == 8) return 8 * (ws >> 1) + 2 * (ws & 1) + (f & 1) + 4 * (f >> 1);
  else return ws * (32 / BITS) + f;
}

// Place of (slot s, channel c) inside one unit's v_res window: entry
// [s/32][c/16][16 g + c%16][j] with s % 32 = 8 g + j (the value consumer order).
__device__ __forceinline__ int64_t value_res_index(int D, int s, int c) {
  const int k = s / 32, tau = s % 32, gg = tau / 8, j = tau % 8;
  return (((int64_t)k * (D / 16) + c / 16) * 64 + 16 * gg + c % 16) * 8 + j;
}

// Token rows [32 blk, 32 blk + 32) of a unit's residual value window, read
// from its consumer order into LDS rows tile[t * D + c].
__device__ __forceinline__ void load_value_window(uint16_t* tile, const uint16_t* vres,
                                                  int blk, int D) {
  const uint4* src = reinterpret_cast<const uint4*>(vres) + (int64_t)blk * (D / 16) * 64;
  for (int x = threadIdx.x; x < (D / 16) * 64; x += blockDim.x) {
    const uint4 w = src[x];  // slots 8g + 0..7 of channel 16n + i
    const int n = x / 64, l = x % 64, gg = l / 16, c = 16 * n + l % 16;
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[(8 * gg + 2 * e) * D + c] = (uint16_t)(ww[e] & 0xffffu);
      tile[(8 * gg + 2 * e + 1) * D + c] = (uint16_t)(ww[e] >> 16);
    }
  }
}

// Loads n_halves fp16 values (a multiple of 8, 16-byte aligned) into LDS.
__device__ __forceinline__ void load_tile(uint16_t* tile, const uint16_t* src,
                                          int n_halves) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(tile);
  for (int i = threadIdx.x; i < n_halves / 8; i += blockDim.x) d[i] = s[i];
}

// LDS of one quantizer workgroup: a tile of fp16 token rows and its codes.
// Keys use G rows, values one 32-token block; sized for the larger.
__host__ __device__ inline int quant_rows(const Geom& g) { return g.G > kVBlock ? g.G : kVBlock; }
inline size_t quant_lds_bytes(const Geom& g) { return (size_t)quant_rows(g) * g.D * 3; }

// One key group: G token rows of D channels in `tile` (already loaded),
// first position `pos` (a multiple of G).  Per channel: min/max over the G
// tokens, split over kThreads / D threads per channel.
template <int BITS>
__device__ void key_group(const Geom& g, int64_t unit, int32_t pos, uint32_t* k_codes,
                          uint16_t* k_meta, const uint16_t* tile, uint8_t* codes) {
  const int G = g.G, D = g.D;
  // slot of the group's first chunk; its other chunks follow it (a page holds
  // whole key groups).  A table entry outside the pool: nothing is written.
  const int64_t cs0 = chunk_slot(g, unit, pos / kVBlock);
  if (cs0 < 0) return;  // uniform over the workgroup
  const int tpc = kThreads / D;            // threads per channel (2 or 4)
  const int c = threadIdx.x / tpc, part = threadIdx.x % tpc;
  const int tn = G / tpc;                  // tokens of this thread
  float mn = h2f(tile[(part * tn) * D + c]), mx = mn;
  for (int t = part * tn + 1; t < (part + 1) * tn; ++t) {
    const float v = h2f(tile[t * D + c]);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  for (int off = 1; off < tpc; off <<= 1) {  // partners are neighbouring lanes
    mn = fminf(mn, __shfl_xor(mn, off, 64));
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  const GroupParams p = group_params(mn, mx, BITS);
  if (part == 0) {
    uint32_t* meta32 = reinterpret_cast<uint32_t*>(k_meta);
    meta32[cs0 * kVBlock / G * D + key_meta_entry<BITS>(c, D)] =
        (uint32_t)p.d16 | ((uint32_t)p.m16 << 16);
  }
  for (int t = part * tn; t < (part + 1) * tn; ++t)
    codes[t * D + c] = (uint8_t)group_code(h2f(tile[t * D + c]), p, BITS);
  __syncthreads();
  // words of the natural token rows, stored at their consumer-order places:
  // row word w' is word w' % KW of slice w' / KW, placed at lane 16 g + i,
  // half u for the token's key row (i, u) in its 32-token block
  constexpr int kPer = 32 / BITS;  // codes per word
  const int W = D * BITS / 32;     // words per token row
  const int KW = W / 4;            // words per slice
  for (int x = threadIdx.x; x < G * W; x += blockDim.x) {
    const int t = x / W, wr = x % W;
    const uint8_t* cc = codes + t * D + (wr / KW) * (D / 4);  // the word's slice
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      word |= (uint32_t)cc[key_field_channel<BITS>(wr % KW, k)] << (k * BITS);
    const int p_tok = pos + t, tau = p_tok % kVBlock;
    const int u = (tau >> 2) & 1, i = 4 * (tau >> 3) + (tau & 3);
    const int lane = 16 * (wr / KW) + i;
    k_codes[(cs0 + p_tok / kVBlock - pos / kVBlock) * (D * BITS) + (2 * lane + u) * KW +
            wr % KW] = word;
  }
}

// One 32-token value block in `tile` (already loaded), first position `pos`
// (a multiple of 32).  Per token: D/G groups of G consecutive channels; the
// 32 * D/G (token, group) items are split over the workgroup's threads.
template <int BITS>
__device__ void value_block(const Geom& g, int64_t unit, int32_t pos, uint32_t* v_codes,
                            uint16_t* v_meta, const uint16_t* tile, uint8_t* codes) {
  const int G = g.G, D = g.D, NG = D / G;
  const int64_t cs = chunk_slot(g, unit, pos / kVBlock);
  if (cs < 0) return;  // a table entry outside the pool: nothing is written
  const int items = kVBlock * NG;                    // 64 .. 128
  const int tpi = kThreads / items;                  // threads per item (2 .. 8)
  const int it = threadIdx.x / tpi, part = threadIdx.x % tpi;
  const int t = it / NG, gm = it % NG;
  const int cn = G / tpi;                            // channels of this thread
  const uint16_t* row = tile + t * D + gm * G + part * cn;
  float mn = h2f(row[0]), mx = mn;
  for (int c = 1; c < cn; ++c) {
    const float v = h2f(row[c]);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  for (int off = 1; off < tpi; off <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, 64));
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  const GroupParams p = group_params(mn, mx, BITS);
  if (part == 0) {
    // entry [block][t / 8][gm][t % 8]
    uint32_t* meta32 = reinterpret_cast<uint32_t*>(v_meta);
    meta32[((cs * 4 + t / 8) * NG + gm) * 8 + t % 8] =
        (uint32_t)p.d16 | ((uint32_t)p.m16 << 16);
  }
  for (int c = 0; c < cn; ++c)
    codes[t * D + gm * G + part * cn + c] = (uint8_t)group_code(h2f(row[c]), p, BITS);
  __syncthreads();
  // consumer order: lane 16 g + i holds tokens 8g + j; 4 bits: word n is
  // channel 16n + i, token j at bit 4 (j/2) + 16 (j%2); 2 bits: word m holds
  // channels 16 (2m + h) + i, token j at bit 8h + 2 (j/2) + 16 (j%2); 8 bits:
  // words 2n, 2n + 1 are channel 16n + i, token j in word 2n + j/4 at bit
  // 8 ((j%4)/2) + 16 (j%2)
  const int NW = D * BITS / 64;  // words per lane
  uint32_t* blk = v_codes + cs * (D * BITS);
  for (int x = threadIdx.x; x < 64 * NW; x += blockDim.x) {
    const int lane = x / NW, w = x % NW;
    const int gg = lane / 16, i = lane % 16;
    uint32_t word = 0;
    if constexpr (BITS == 8) {
      const int c = 16 * (w / 2) + i;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * (w % 2) + jj;
        word |= (uint32_t)codes[(8 * gg + j) * D + c] << (8 * (jj / 2) + 16 * (jj % 2));
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4 / BITS; ++h) {
        const int c = 16 * (w * (4 / BITS) + h) + i;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int bit = 8 * h + BITS * (j / 2) + 16 * (j % 2);
          word |= (uint32_t)codes[(8 * gg + j) * D + c] << bit;
        }
      }
    }
    blk[x] = word;
  }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void quantize_keys_kernel(
    Geom g, const uint16_t* __restrict__ src, int64_t src_unit_stride,
    int32_t pos0, uint32_t* __restrict__ k_codes, uint16_t* __restrict__ k_meta) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* tile = lds;
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds + quant_rows(g) * g.D);
  const int64_t unit = (int64_t)blockIdx.z * g.Hkv + blockIdx.y;
  const int j = blockIdx.x;
  load_tile(tile, src + unit * src_unit_stride + (int64_t)j * g.G * g.D, g.G * g.D);
  __syncthreads();
  key_group<BITS>(g, unit, pos0 + j * g.G, k_codes, k_meta, tile, codes);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void quantize_values_kernel(
    Geom g, const uint16_t* __restrict__ src, int64_t src_unit_stride,
    int32_t pos0, uint32_t* __restrict__ v_codes, uint16_t* __restrict__ v_meta) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* tile = lds;
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds + quant_rows(g) * g.D);
  const int64_t unit = (int64_t)blockIdx.z * g.Hkv + blockIdx.y;
  const int blk = blockIdx.x;
  load_tile(tile, src + unit * src_unit_stride + (int64_t)blk * kVBlock * g.D, kVBlock * g.D);
  __syncthreads();
  value_block<BITS>(g, unit, pos0 + blk * kVBlock, v_codes, v_meta, tile, codes);
}

// Copies positions [pos0, pos0 + n_tok) of key rows (values == false; window
// of R slots, token rows) or value rows (window of Rv slots, value consumer
// order) src [unit][.][D] (first row = position pos0) to slots p % window.
__global__ __launch_bounds__(kThreads) void residual_copy_kernel(
    Geom g, const uint16_t* __restrict__ src, int64_t src_unit_stride, int32_t pos0,
    int32_t n_tok, uint16_t* __restrict__ window, bool values) {
  const int64_t vecs_per_row = g.D / 8;
  const int64_t total = (int64_t)g.B * g.Hkv * n_tok * vecs_per_row;
  const int W = values ? g.Rv : g.R;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i % vecs_per_row;
    const int64_t t = (i / vecs_per_row) % n_tok;
    const int64_t unit = i / (vecs_per_row * n_tok);
    const int64_t slot = (pos0 + t) % W;
    const uint4 x = reinterpret_cast<const uint4*>(src)[unit * src_unit_stride / 8 +
                                                        t * vecs_per_row + e];
    if (!values) {
      reinterpret_cast<uint4*>(window)[(unit * W + slot) * vecs_per_row + e] = x;
    } else {
      // channels 8e .. 8e+7 of the slot go to their window places
      const uint32_t xx[4] = {x.x, x.y, x.z, x.w};
      uint16_t* vu = window + unit * W * g.D;
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const uint16_t val = (uint16_t)((h & 1) ? (xx[h / 2] >> 16) : (xx[h / 2] & 0xffffu));
        vu[value_res_index(g.D, (int)slot, (int)(8 * e + h))] = val;
      }
    }
  }
}

// Grid (KV head, sequence, 1 + R/G + Rv/32); keys have a window of R slots,
// values of Rv (R = Rv unless set apart).  z = 0 writes the new token to key
// slot n % R when no key flush is due, and to value slot n % Rv when no value
// flush is due.  A key flush is due when n > 0 and n % R == 0 (the key window
// holds positions n - R .. n - 1 in slots 0 .. R-1): z = 1 .. R/G quantize
// its key groups.  A value flush likewise with Rv: z = R/G + 1 .. its 32-token
// value blocks.  Each in its own workgroup; the workgroup that reads slot 0
// of a flushing window (key group 0, value block 0) writes the new token
// there after its read, so no workgroup waits for another.  Workgroups with
// nothing to do return at once.
template <int BK, int BV>
__global__ __launch_bounds__(kThreads) void append_kernel(
    Geom g, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ seq_lens, uint32_t* __restrict__ k_codes,
    uint32_t* __restrict__ v_codes, uint16_t* __restrict__ k_meta,
    uint16_t* __restrict__ v_meta, uint16_t* __restrict__ k_res,
    uint16_t* __restrict__ v_res) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int b = blockIdx.y, z = blockIdx.z;
  const int64_t unit = (int64_t)b * g.Hkv + blockIdx.x;
  const int32_t n = seq_lens[b];
  if (n < 0 || n >= g.C) return;  // caller error: leave the cache untouched
  uint16_t* kr = k_res + unit * g.R * g.D;
  uint16_t* vr = v_res + unit * g.Rv * g.D;
  const bool kflush = n > 0 && n % g.R == 0;
  const bool vflush = n > 0 && n % g.Rv == 0;
  const int nk = g.R / g.G;  // key groups of the key window
  if (z == 0) {
    if (!kflush)
      for (int c = threadIdx.x; c < g.D; c += blockDim.x)
        kr[(int64_t)(n % g.R) * g.D + c] = k_new[unit * g.D + c];
    if (!vflush)
      for (int c = threadIdx.x; c < g.D; c += blockDim.x)
        vr[value_res_index(g.D, n % g.Rv, c)] = v_new[unit * g.D + c];
    return;
  }
  uint16_t* tile = lds;
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds + quant_rows(g) * g.D);
  if (z <= nk) {
    if (!kflush) return;
    const int j = z - 1;
    load_tile(tile, kr + (int64_t)j * g.G * g.D, g.G * g.D);
    __syncthreads();
    if (j == 0)  // slot 0 has been read: the new token goes there
      for (int c = threadIdx.x; c < g.D; c += blockDim.x) kr[c] = k_new[unit * g.D + c];
    key_group<BK>(g, unit, n - g.R + j * g.G, k_codes, k_meta, tile, codes);
  } else {
    if (!vflush) return;
    const int blk = z - 1 - nk;
    load_value_window(tile, vr, blk, g.D);
    __syncthreads();
    if (blk == 0)
      for (int c = threadIdx.x; c < g.D; c += blockDim.x)
        vr[value_res_index(g.D, 0, c)] = v_new[unit * g.D + c];
    value_block<BV>(g, unit, n - g.Rv + blk * kVBlock, v_codes, v_meta, tile, codes);
  }
}

// T tokens per sequence in one launch (the new tokens of a multi-token decode
// step): one workgroup per (sequence, KV head) appends them in order, each as
// append_kernel would, so the cache ends bit-identical to T single appends.
// A token that arrives for a full window first quantizes the whole window
// here, one key group or value block after another through the LDS tile
// (the window then holds every earlier token of this call, written above).
template <int BK, int BV>
__global__ __launch_bounds__(kThreads) void append_tokens_kernel(
    Geom g, int T, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ seq_lens, uint32_t* __restrict__ k_codes,
    uint32_t* __restrict__ v_codes, uint16_t* __restrict__ k_meta,
    uint16_t* __restrict__ v_meta, uint16_t* __restrict__ k_res,
    uint16_t* __restrict__ v_res) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int b = blockIdx.y, hkv = blockIdx.x;
  const int64_t unit = (int64_t)b * g.Hkv + hkv;
  const int32_t n = seq_lens[b];
  if (n < 0 || n > g.C - T) return;  // caller error: leave the cache untouched
  uint16_t* kr = k_res + unit * g.R * g.D;
  uint16_t* vr = v_res + unit * g.Rv * g.D;
  // the first position of the call that finds a window full (a multiple of
  // the window length, above 0): with none, every token is a plain copy, done
  // at once
  const int32_t p1 = n > 0 ? n : 1;
  const bool kflush = (p1 + g.R - 1) / g.R * g.R < n + T;
  const bool vflush = (p1 + g.Rv - 1) / g.Rv * g.Rv < n + T;
  if (!kflush && !vflush) {
    for (int i = threadIdx.x; i < T * g.D; i += blockDim.x) {
      const int t = i / g.D, c = i % g.D;
      const int32_t pos = n + t;
      const int64_t src = (((int64_t)b * T + t) * g.Hkv + hkv) * g.D + c;
      kr[(int64_t)(pos % g.R) * g.D + c] = k_new[src];
      vr[value_res_index(g.D, pos % g.Rv, c)] = v_new[src];
    }
    return;
  }
  uint16_t* tile = lds;
  uint8_t* codes = reinterpret_cast<uint8_t*>(lds + quant_rows(g) * g.D);
  for (int t = 0; t < T; ++t) {
    const int32_t pos = n + t;
    const int64_t src = (((int64_t)b * T + t) * g.Hkv + hkv) * g.D;  // [B][T][Hkv][D]
    if (pos > 0 && pos % g.R == 0) {
      for (int j = 0; j < g.R / g.G; ++j) {
        load_tile(tile, kr + (int64_t)j * g.G * g.D, g.G * g.D);
        __syncthreads();
        key_group<BK>(g, unit, pos - g.R + j * g.G, k_codes, k_meta, tile, codes);
        __syncthreads();
      }
    }
    if (pos > 0 && pos % g.Rv == 0) {
      for (int blk = 0; blk < g.Rv / kVBlock; ++blk) {
        load_value_window(tile, vr, blk, g.D);
        __syncthreads();
        value_block<BV>(g, unit, pos - g.Rv + blk * kVBlock, v_codes, v_meta, tile, codes);
        __syncthreads();
      }
    }
    for (int c = threadIdx.x; c < g.D; c += blockDim.x) {
      kr[(int64_t)(pos % g.R) * g.D + c] = k_new[src + c];
      vr[value_res_index(g.D, pos % g.Rv, c)] = v_new[src + c];
    }
    __syncthreads();  // a later token's flush reads these slots
  }
}

}  // namespace

hipError_t launch_quantize_keys(const Geom& g, const uint16_t* src,
                                int64_t src_unit_stride, int32_t pos0,
                                int32_t n_tok, uint32_t* k_codes,
                                uint16_t* k_meta, hipStream_t st) {
  if (n_tok == 0) return hipSuccess;
  dim3 grid(n_tok / g.G, g.Hkv, g.B);
  if (g.bK == 2)
    quantize_keys_kernel<2><<<grid, kThreads, quant_lds_bytes(g), st>>>(
        g, src, src_unit_stride, pos0, k_codes, k_meta);
  else if (g.bK == 4)
    quantize_keys_kernel<4><<<grid, kThreads, quant_lds_bytes(g), st>>>(
        g, src, src_unit_stride, pos0, k_codes, k_meta);
  else
    quantize_keys_kernel<8><<<grid, kThreads, quant_lds_bytes(g), st>>>(
        g, src, src_unit_stride, pos0, k_codes, k_meta);
  return hipGetLastError();
}

hipError_t launch_quantize_values(const Geom& g, const uint16_t* src,
                                  int64_t src_unit_stride, int32_t pos0,
                                  int32_t n_tok, uint32_t* v_codes,
                                  uint16_t* v_meta, hipStream_t st) {
  if (n_tok == 0) return hipSuccess;
  dim3 grid(n_tok / kVBlock, g.Hkv, g.B);
  if (g.bV == 2)
    quantize_values_kernel<2><<<grid, kThreads, quant_lds_bytes(g), st>>>(
        g, src, src_unit_stride, pos0, v_codes, v_meta);
  else if (g.bV == 4)
    quantize_values_kernel<4><<<grid, kThreads, quant_lds_bytes(g), st>>>(
        g, src, src_unit_stride, pos0, v_codes, v_meta);
  else
    quantize_values_kernel<8><<<grid, kThreads, quant_lds_bytes(g), st>>>(
        g, src, src_unit_stride, pos0, v_codes, v_meta);
  return hipGetLastError();
}

hipError_t launch_residual_copy(const Geom& g, const uint16_t* src, int64_t src_unit_stride,
                                int32_t pos0, int32_t n_tok, uint16_t* window, bool values,
                                hipStream_t st) {
  if (n_tok == 0) return hipSuccess;
  const int64_t total = (int64_t)g.B * g.Hkv * n_tok * (g.D / 8);
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  residual_copy_kernel<<<grid, kThreads, 0, st>>>(g, src, src_unit_stride, pos0, n_tok, window,
                                                  values);
  return hipGetLastError();
}

hipError_t launch_append(const Geom& g, const uint16_t* k_new,
                         const uint16_t* v_new, const int32_t* seq_lens,
                         const kvq_cache& c, hipStream_t st) {
  dim3 grid(g.Hkv, g.B, 1 + g.R / g.G + g.Rv / kVBlock);
#define KVQ_APPEND(BK, BV)                                                    \
  append_kernel<BK, BV><<<grid, kThreads, quant_lds_bytes(g), st>>>(          \
      g, k_new, v_new, seq_lens, c.k_codes, c.v_codes, c.k_meta, c.v_meta,    \
      c.k_res, c.v_res)
  const int code = 10 * g.bK + g.bV;
  switch (code) {
    case 22: KVQ_APPEND(2, 2); break;
    case 24: KVQ_APPEND(2, 4); break;
    case 28: KVQ_APPEND(2, 8); break;
    case 42: KVQ_APPEND(4, 2); break;
    case 44: KVQ_APPEND(4, 4); break;
    case 48: KVQ_APPEND(4, 8); break;
    case 82: KVQ_APPEND(8, 2); break;
    case 84: KVQ_APPEND(8, 4); break;
    case 88: KVQ_APPEND(8, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef KVQ_APPEND
  return hipGetLastError();
}

hipError_t launch_append_tokens(const Geom& g, int T, const uint16_t* k_new,
                                const uint16_t* v_new, const int32_t* seq_lens,
                                const kvq_cache& c, hipStream_t st) {
  dim3 grid(g.Hkv, g.B);
#define KVQ_APPEND_T(BK, BV)                                                  \
  append_tokens_kernel<BK, BV><<<grid, kThreads, quant_lds_bytes(g), st>>>(   \
      g, T, k_new, v_new, seq_lens, c.k_codes, c.v_codes, c.k_meta, c.v_meta, \
      c.k_res, c.v_res)
  const int code = 10 * g.bK + g.bV;
  switch (code) {
    case 22: KVQ_APPEND_T(2, 2); break;
    case 24: KVQ_APPEND_T(2, 4); break;
    case 28: KVQ_APPEND_T(2, 8); break;
    case 42: KVQ_APPEND_T(4, 2); break;
    case 44: KVQ_APPEND_T(4, 4); break;
    case 48: KVQ_APPEND_T(4, 8); break;
    case 82: KVQ_APPEND_T(8, 2); break;
    case 84: KVQ_APPEND_T(8, 4); break;
    case 88: KVQ_APPEND_T(8, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef KVQ_APPEND_T
  return hipGetLastError();
}

}  // namespace kvq
