// kvq_bq2_quant.hip — stores positions of the rotated per-token 2-bit cache
// format (KV1's BQ2_0; layout in kvq_bq2.h) on gfx950: Hadamard rotation,
// fp16 sinks for positions 0..3, one quantized block per other position.
//
// [KV1] "Quantization Format: KV1.cpp BQ2_0": every head vector is multiplied
// by the normalized 64x64 Sylvester Hadamard matrix H before it is stored;
// then, per position and KV head, the 64 rotated values form one block with
// d = fp16(max((max - min)/3, 1e-6)), m = fp16(min) and
// code = clamp(rne((x - m)/d), 0, 3) computed in fp32 from the fp16-rounded
// d and m; positions 0..3 keep full precision (fp16 here).
//
// One wave handles one position of one (sequence, KV head) unit, lane c
// holding channel c.  H x is a fast Walsh-Hadamard transform across the 64
// lanes in fp64: every partial sum of the fp16 inputs (multiples of 2^-24
// below 2^16, times +-1) needs at most 46 significant bits, so the transform
// is the exact product whatever its order, and it is rounded once to fp32.
// Built with -ffp-contract=off and without fast-math: '/' on float is the
// correctly rounded IEEE division, rintf rounds half to even and the fp16
// conversion rounds to nearest even, so the codes match a plain fp32 reading.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kD = KVQ_BQ2_HEAD_DIM;
constexpr int kSinks = KVQ_BQ2_SINKS;

// H x for the 64 lanes' values (exact in fp64), rounded once to fp32.
__device__ __forceinline__ float rotate(uint16_t bits, int lane) {
  double x = (double)h2f(bits);
#pragma unroll
  for (int d = 1; d < kD; d <<= 1) {
    const double y = __shfl_xor(x, d, 64);
    x = (lane & d) ? (y - x) : (x + y);  // butterfly (a, b) -> (a + b, a - b)
  }
  return (float)(x * 0.125);
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

struct Block {
  uint32_t dm;    // fp16 d in bits 0..15, fp16 m in bits 16..31
  uint32_t code;  // this lane's 2-bit code
};

// One block over the wave's 64 values ([KV1] Quantization Format, fp32).
__device__ __forceinline__ Block quantize(float x) {
  float mn = wave_min(x);
  const float mx = wave_max(x);
  if (mn == 0.0f) mn = 0.0f;  // a zero min is stored as +0
  float d32 = (mx - mn) / 3.0f;  // fp32 subtract, IEEE divide
  if (!(d32 > 1e-6f)) d32 = 1e-6f;
  const uint16_t d16 = f2h(d32), m16 = f2h(mn);
  const float y = (x - h2f(m16)) / h2f(d16);  // d16 >= 2^-24 * 17 > 0
  const float r = fminf(fmaxf(rintf(y), 0.0f), 3.0f);
  return Block{(uint32_t)d16 | ((uint32_t)m16 << 16), (uint32_t)r};
}

// OR over the 16 lanes of each row (DPP rotations inside a row).
__device__ __forceinline__ uint32_t row_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);  // row_ror:4
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x122, 0xF, 0xF, false);  // row_ror:2
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x121, 0xF, 0xF, false);  // row_ror:1
  return v;
}

// Key codes of position t: lane group g builds word g (channels 16g..16g+15,
// channel 16g + f at bit 2f); the word sits at [t/32][16g + i][u] with
// tau = t % 32 = 8 (i/4) + 4u + i%4.
__device__ __forceinline__ void store_key_word(const Bq2Geom& g, uint32_t* k_codes,
                                               int64_t unit, int t, uint32_t code, int lane) {
  const uint32_t w = row_or(code << (2 * (lane & 15)));
  const int tau = t & 31;
  const int i = 4 * (tau >> 3) + (tau & 3), u = (tau >> 2) & 1;
  if ((lane & 15) == 0)
    k_codes[((unit * (g.C / 32) + t / 32) * 64 + 16 * (lane >> 4) + i) * 2 + u] = w;
}

// Value word of channel c = lane for a lane group's tokens j: the field of
// token j sits at bit 8h + 2(j/2) + 16(j%2) of word [16 gv + i][m], with
// channel c = 16 (2m + h) + i.
__device__ __forceinline__ int value_field(int j, int lane) {
  return 8 * ((lane >> 4) & 1) + 2 * (j >> 1) + 16 * (j & 1);
}
__device__ __forceinline__ int64_t value_word_index(const Bq2Geom& g, int64_t unit, int t,
                                                    int lane) {
  const int gv = (t & 31) >> 3, i = lane & 15, m = lane >> 5;
  return ((unit * (g.C / 32) + t / 32) * 64 + 16 * gv + i) * 2 + m;
}

// One workgroup of four waves per (32-position chunk, KV head, sequence); wave
// w takes positions 32k + 8w + j, j < 8, one after the other, so that it
// writes whole value words (each holds eight positions of two channels).
__global__ __launch_bounds__(kThreads) void bq2_prefill_kernel(Bq2Geom g, const uint16_t* k,
                                                               const uint16_t* v, int n,
                                                               kvq_bq2_cache c) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int chunk = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * g.Hkv + hkv;
  const int t0 = chunk * 32 + 8 * w;
  uint32_t vword = 0;
  bool any = false;
  for (int j = 0; j < 8; ++j) {
    const int t = t0 + j;
    if (t >= n) break;
    const int64_t row = (unit * n + t) * kD + lane;
    const float kx = rotate(k[row], lane);
    const float vx = rotate(v[row], lane);
    if (t < kSinks) {
      c.k_sink[(unit * kSinks + t) * kD + lane] = f2h(kx);
      c.v_sink[(unit * kD + lane) * kSinks + t] = f2h(vx);
      continue;
    }
    any = true;
    const Block kb = quantize(kx), vb = quantize(vx);
    store_key_word(g, c.k_codes, unit, t, kb.code, lane);
    if (lane == 0) {
      reinterpret_cast<uint32_t*>(c.k_meta)[unit * g.C + t] = kb.dm;
      reinterpret_cast<uint32_t*>(c.v_meta)[unit * g.C + t] = vb.dm;
    }
    vword |= vb.code << value_field(j, lane);
  }
  if (!any) return;
  // channels 16 (2m) + i and 16 (2m + 1) + i (lanes l and l ^ 16) share a word
  const uint32_t other = __shfl_xor(vword, 16, 64);
  if (((lane >> 4) & 1) == 0) c.v_codes[value_word_index(g, unit, t0, lane)] = vword | other;
}

// One wave per (KV head, sequence): position t = seq_lens[b].
__global__ __launch_bounds__(64) void bq2_append_kernel(Bq2Geom g, const uint16_t* k_new,
                                                        const uint16_t* v_new,
                                                        const int32_t* seq_lens,
                                                        kvq_bq2_cache c) {
  const int lane = threadIdx.x;
  const int hkv = blockIdx.x, b = blockIdx.y;
  const int t = seq_lens[b];
  if (t < 0 || t >= g.C) return;
  const int64_t unit = (int64_t)b * g.Hkv + hkv;
  const float kx = rotate(k_new[unit * kD + lane], lane);
  const float vx = rotate(v_new[unit * kD + lane], lane);
  if (t < kSinks) {
    c.k_sink[(unit * kSinks + t) * kD + lane] = f2h(kx);
    c.v_sink[(unit * kD + lane) * kSinks + t] = f2h(vx);
    return;
  }
  const Block kb = quantize(kx), vb = quantize(vx);
  store_key_word(g, c.k_codes, unit, t, kb.code, lane);
  if (lane == 0) {
    reinterpret_cast<uint32_t*>(c.k_meta)[unit * g.C + t] = kb.dm;
    reinterpret_cast<uint32_t*>(c.v_meta)[unit * g.C + t] = vb.dm;
  }
  // this position's two fields of the shared value word (read-modify-write)
  const int j = t & 7;
  const uint32_t mine = vb.code << value_field(j, lane);
  const uint32_t both = mine | __shfl_xor(mine, 16, 64);
  if (((lane >> 4) & 1) == 0) {
    const uint32_t mask = (3u << value_field(j, 0)) | (3u << (value_field(j, 0) + 8));
    uint32_t* wp = c.v_codes + value_word_index(g, unit, t, lane);
    *wp = (*wp & ~mask) | both;
  }
}

}  // namespace

hipError_t launch_bq2_prefill(const Bq2Geom& g, const uint16_t* k, const uint16_t* v,
                              int32_t n, const kvq_bq2_cache& cache, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  dim3 grid((n + 31) / 32, g.Hkv, g.B);
  bq2_prefill_kernel<<<grid, kThreads, 0, st>>>(g, k, v, n, cache);
  return hipGetLastError();
}

hipError_t launch_bq2_append(const Bq2Geom& g, const uint16_t* k_new, const uint16_t* v_new,
                             const int32_t* seq_lens, const kvq_bq2_cache& cache,
                             hipStream_t st) {
  dim3 grid(g.Hkv, g.B);
  bq2_append_kernel<<<grid, 64, 0, st>>>(g, k_new, v_new, seq_lens, cache);
  return hipGetLastError();
}

}  // namespace kvq
