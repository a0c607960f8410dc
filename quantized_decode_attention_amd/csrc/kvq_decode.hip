// kvq_decode.hip — single-token decode attention over the packed cache plus
// the fp16 residual window: split-context partial softmax and combine (gfx950).
//
// What is computed (KIVI repository page, "Overview": attention over keys
// quantized per channel and values quantized per token, with the recent tokens
// kept in fp16; KV1-1.2B model card, "Quickstart": attending over the
// dequantized cache gives the exact low-bit result):
//   s_t = sm_scale * q . k_t,  out = sum_t softmax(s)_t v_t
// with k_t = code * scale + min from the key group's per-channel (scale, min)
// for packed tokens, the fp16 residual for the rest, and v_t likewise from the
// token's per-group (scale, min).
//
// Per-group fold (algebra on the dequantizer): for key group j,
//   q . k_t = sum_c (q_c * scale_jc) * code_tc + sum_c q_c * min_jc
// so the query is scaled once per group and the codes enter the dot product as
// small integers.  Scores are kept in log2 units (sm_scale * log2 e folded into
// q) so the softmax uses exp2.
//
// One workgroup = (split, KV head, sequence); the GQA query heads of the KV head
// share every code and meta load.  A split covers `split_tokens` positions (a
// multiple of G, so key groups never straddle splits); its partial is the
// running (max, sum, weighted value sum) of an online softmax.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kChunk = 32;          // tokens per inner iteration (= value block)
constexpr int kThreadsPerToken = 8;  // score lanes per token
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int packed_len(int n, int R) {
  return n <= 0 ? 0 : n - (((n - 1) % R) + 1);
}

__device__ __forceinline__ float reduce_max32(float x) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float reduce_sum32(float x) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// `bits` consecutive-field codes of CPT channels starting at bit `bitoff` of a
// token row, returned as the low CPT*BK bits of a 64-bit word.
template <int CPT, int BK>
__device__ __forceinline__ uint64_t load_key_slice(const uint32_t* row,
                                                   int bitoff) {
  constexpr int kBits = CPT * BK;
  if constexpr (kBits == 64) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + bitoff / 32);
    return (uint64_t)w.x | ((uint64_t)w.y << 32);
  } else {
    const uint32_t w = row[bitoff / 32];
    return (uint64_t)(w >> (bitoff % 32));
  }
}

template <int D, int BK, int BV, int GQ>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecodeLaunch L) {
  constexpr int CPT = D / kThreadsPerToken;      // channels per score lane
  constexpr int TPC = kThreads / D;              // threads per channel (V)
  constexpr int HPT = (GQ + TPC - 1) / TPC;      // heads per V thread
  constexpr int kMaxNG = D / 32;                 // value groups per token, max

  __shared__ float qf[GQ][D];        // q * sm_scale * log2 e
  __shared__ float qk[GQ][D];        // qf * key scale of the current group
  __shared__ float beta[GQ];         // qf . key min of the current group
  __shared__ float sc[GQ][kChunk];   // scores, then probabilities
  __shared__ float2 vm[kChunk][kMaxNG];  // value (scale, min) of the chunk
  __shared__ float m_run[GQ], l_run[GQ], alpha[GQ];

  const Geom& g = L.g;
  const int tid = threadIdx.x;
  const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int64_t unit = (int64_t)b * g.Hkv + hkv;
  const int n = L.seq_lens[b];
  const bool direct = (L.n_split == 1);
  const int c_v = tid % D;      // channel of this thread in the V phase
  const int hg = tid / D;       // head group of this thread in the V phase

  if (n < 0 || n > g.C || n > L.max_seq_len || (n == 0)) {
    // invalid length -> NaN; empty sequence -> 0 (combine does the same when
    // there is more than one split)
    if (direct) {
      const uint16_t val = (n == 0) ? (uint16_t)0 : (uint16_t)0x7e00;
      for (int i = tid; i < GQ * D; i += kThreads)
        L.out[((int64_t)b * g.Hq + hkv * GQ) * D + i] = val;
    }
    return;
  }
  const int t_begin = split * L.split_tokens;
  if (t_begin >= n) return;  // empty split: the combine ignores it
  const int t_end = min(n, t_begin + L.split_tokens);
  const int lq = packed_len(n, g.R);
  const int NG = D / g.G;

  for (int i = tid; i < GQ * D; i += kThreads)
    (&qf[0][0])[i] =
        h2f(L.q[((int64_t)b * g.Hq + hkv * GQ) * D + i]) * L.scale_log2;
  if (tid < GQ) {
    m_run[tid] = kNegInf;
    l_run[tid] = 0.0f;
  }
  float o[HPT];
#pragma unroll
  for (int i = 0; i < HPT; ++i) o[i] = 0.0f;
  __syncthreads();

  const int tok = tid / kThreadsPerToken;  // score phase: token in chunk
  const int sl = tid % kThreadsPerToken;   // score phase: channel slice
  const uint32_t* kc_unit = L.cache.k_codes + unit * g.C * (D * BK / 32);
  const uint32_t* kmeta = reinterpret_cast<const uint32_t*>(L.cache.k_meta) +
                          unit * (g.C / g.G) * D;
  const uint32_t* vmeta = reinterpret_cast<const uint32_t*>(L.cache.v_meta) +
                          unit * g.C * NG;
  const uint32_t* vc_unit = L.cache.v_codes + unit * (g.C / kVBlock) * D * BV;
  const uint16_t* kr = L.cache.k_res + unit * g.R * D;
  const uint16_t* vr = L.cache.v_res + unit * g.R * D;

  int cur_group = -1;
  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const bool packed = t0 < lq;  // chunks never straddle lq (both % 32 == 0)
    if (packed) {
      const int j = t0 / g.G;
      if (j != cur_group) {
        // fold the group's per-channel scale into q; min into beta
        for (int i = tid; i < GQ * D; i += kThreads) {
          const int c = i % D;
          (&qk[0][0])[i] = (&qf[0][0])[i] * h2f((uint16_t)(kmeta[j * D + c] & 0xffffu));
        }
        const int wave = tid / 64, lane = tid % 64;
        for (int h = wave; h < GQ; h += kThreads / 64) {
          float acc = 0.0f;
          for (int c = lane; c < D; c += 64)
            acc += qf[h][c] * h2f((uint16_t)(kmeta[j * D + c] >> 16));
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
          if (lane == 0) beta[h] = acc;
        }
        cur_group = j;
      }
      for (int i = tid; i < kChunk * NG; i += kThreads) {
        const uint32_t mv = vmeta[(int64_t)(t0 + i / NG) * NG + i % NG];
        vm[i / NG][i % NG] = make_float2(h2f((uint16_t)(mv & 0xffffu)),
                                         h2f((uint16_t)(mv >> 16)));
      }
      __syncthreads();
      // scores: 8 lanes per token, CPT channels each
      const int t = t0 + tok;  // always < lq <= t_end here
      const uint64_t bits = load_key_slice<CPT, BK>(
          kc_unit + (int64_t)t * (D * BK / 32), sl * CPT * BK);
      float acc[GQ];
#pragma unroll
      for (int h = 0; h < GQ; ++h) acc[h] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const float code = (float)((bits >> (i * BK)) & ((1u << BK) - 1u));
#pragma unroll
        for (int h = 0; h < GQ; ++h) acc[h] += qk[h][sl * CPT + i] * code;
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        acc[h] += __shfl_xor(acc[h], 1, 64);
        acc[h] += __shfl_xor(acc[h], 2, 64);
        acc[h] += __shfl_xor(acc[h], 4, 64);
      }
      if (sl == 0) {
#pragma unroll
        for (int h = 0; h < GQ; ++h) sc[h][tok] = acc[h] + beta[h];
      }
    } else {
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
          for (int h = 0; h < GQ; ++h) acc[h] += qf[h][sl * CPT + i] * kv;
        }
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        acc[h] += __shfl_xor(acc[h], 1, 64);
        acc[h] += __shfl_xor(acc[h], 2, 64);
        acc[h] += __shfl_xor(acc[h], 4, 64);
      }
      if (sl == 0) {
#pragma unroll
        for (int h = 0; h < GQ; ++h) sc[h][tok] = valid ? acc[h] : kNegInf;
      }
    }
    __syncthreads();
    // online softmax over the chunk: 32 lanes per head
    for (int i = tid; i < GQ * kChunk; i += kThreads) {
      const int h = i / kChunk, tk = i % kChunk;
      const float x = sc[h][tk];
      const float cmax = reduce_max32(x);
      const float m_old = m_run[h];
      const float m_new = fmaxf(m_old, cmax);  // finite: one valid token
      const float p = exp2f(x - m_new);
      const float psum = reduce_sum32(p);
      sc[h][tk] = p;
      if (tk == 0) {
        const float a = exp2f(m_old - m_new);
        alpha[h] = a;
        l_run[h] = l_run[h] * a + psum;
        m_run[h] = m_new;
      }
    }
    __syncthreads();
    // V accumulation: this thread owns channel c_v of heads hg*HPT + i
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int h = hg * HPT + i;
      if (h < GQ) o[i] *= alpha[h];
    }
    if (packed) {
      const uint32_t* w = vc_unit + ((int64_t)(t0 / kVBlock) * D + c_v) * BV;
      uint32_t words[BV];
#pragma unroll
      for (int k = 0; k < BV; ++k) words[k] = w[k];
      const int gm = c_v / g.G;
#pragma unroll
      for (int tk = 0; tk < kChunk; ++tk) {
        const uint32_t code =
            (words[(tk * BV) / 32] >> ((tk * BV) % 32)) & ((1u << BV) - 1u);
        const float2 sm = vm[tk][gm];
        const float vv = (float)code * sm.x + sm.y;
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
          const int h = hg * HPT + i;
          if (h < GQ) o[i] += sc[h][tk] * vv;
        }
      }
    } else {
      for (int tk = 0; tk < kChunk && t0 + tk < t_end; ++tk) {
        const float vv = h2f(vr[(int64_t)((t0 + tk) % g.R) * D + c_v]);
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
          const int h = hg * HPT + i;
          if (h < GQ) o[i] += sc[h][tk] * vv;
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    const int h = hg * HPT + i;
    if (h >= GQ) continue;
    const int64_t bh = (int64_t)b * g.Hq + hkv * GQ + h;
    if (direct) {
      L.out[bh * D + c_v] = f2h(o[i] / l_run[h]);
    } else {
      float* part = L.ws + (bh * L.n_split + split) * (D + 2);
      part[c_v] = o[i];
      if (c_v == 0) {
        part[D] = m_run[h];
        part[D + 1] = l_run[h];
      }
    }
  }
}

// Merges the splits of one (sequence, query head):
//   M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeLaunch L) {
  const Geom& g = L.g;
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int64_t bh = (int64_t)b * g.Hq + h;
  const int n = L.seq_lens[b];
  if (n < 0 || n > g.C || n > L.max_seq_len) {
    L.out[bh * D + c] = 0x7e00;  // NaN
    return;
  }
  if (n == 0) {
    L.out[bh * D + c] = 0;
    return;
  }
  const int ns = (n + L.split_tokens - 1) / L.split_tokens;
  const float* part = L.ws + bh * L.n_split * (D + 2);
  float M = kNegInf;
  for (int i = 0; i < ns; ++i) M = fmaxf(M, part[i * (D + 2) + D]);
  float Ls = 0.0f, acc = 0.0f;
  for (int i = 0; i < ns; ++i) {
    const float w = exp2f(part[i * (D + 2) + D] - M);
    Ls += part[i * (D + 2) + D + 1] * w;
    acc += part[i * (D + 2) + c] * w;
  }
  L.out[bh * D + c] = f2h(acc / Ls);
}

template <int D, int BK, int BV>
hipError_t dispatch_gq(const DecodeLaunch& L, hipStream_t st) {
  dim3 grid(L.n_split, L.g.Hkv, L.g.B);
  switch (L.g.Hq / L.g.Hkv) {
    case 1: decode_partial_kernel<D, BK, BV, 1><<<grid, kThreads, 0, st>>>(L); break;
    case 2: decode_partial_kernel<D, BK, BV, 2><<<grid, kThreads, 0, st>>>(L); break;
    case 4: decode_partial_kernel<D, BK, BV, 4><<<grid, kThreads, 0, st>>>(L); break;
    case 8: decode_partial_kernel<D, BK, BV, 8><<<grid, kThreads, 0, st>>>(L); break;
    case 16: decode_partial_kernel<D, BK, BV, 16><<<grid, kThreads, 0, st>>>(L); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
  if (L.n_split == 1) return hipSuccess;
  dim3 grid(L.g.Hq, L.g.B);
  if (L.g.D == 64)
    decode_combine_kernel<64><<<grid, 64, 0, st>>>(L);
  else
    decode_combine_kernel<128><<<grid, 128, 0, st>>>(L);
  return hipGetLastError();
}

}  // namespace kvq
