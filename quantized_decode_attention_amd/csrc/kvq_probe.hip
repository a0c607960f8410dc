// kvq_probe.hip — a plain streaming read (measurement aid, kvq_probe.h):
// every wave reads a contiguous share of the buffer with 16-byte loads, four
// in flight per lane, and folds them into one word so that none is dropped.
#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kProbeBlocks = 256 * 8;  // 8 workgroups of 4 waves per compute unit
constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* buf, int64_t n16,
                                                                    uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;  // 16-byte units per workgroup
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + 3 * kProbeThreads < b1; i += 4 * kProbeThreads) {
    const uint4 a = buf[i], b = buf[i + kProbeThreads], c = buf[i + 2 * kProbeThreads],
                d = buf[i + 3 * kProbeThreads];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < b1; i += kProbeThreads) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // one word per workgroup, so the loads are live
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + threadIdx.x / 64] = acc;
}

// The sweep form: single-wave workgroups, each reading one contiguous share in
// batches of U 16-byte loads per lane (64 U loads per wave), two batches in
// flight (the next batch is requested before the current one is folded), with
// plain or nontemporal loads.  An index past the share is clamped to its last
// unit (a cached re-read), so no load sits under a branch.
template <int U, bool NT>
__device__ __forceinline__ void batch_load(const uint4* buf, int64_t i, int64_t b1, int lane,
                                           uint4 (&v)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int64_t k = i + 64 * u + lane;
    k = k < b1 ? k : b1 - 1;
    if constexpr (NT) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(buf) + k);
      v[u] = make_uint4(t.x, t.y, t.z, t.w);
    } else {
      v[u] = buf[k];
    }
  }
}

template <int U>
__device__ __forceinline__ uint32_t batch_fold(const uint4 (&v)[U]) {
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  return acc;
}

template <int U, bool NT>
__global__ __launch_bounds__(64) void stream_read_sweep_kernel(const uint4* buf, int64_t n16,
                                                               uint32_t* sink) {
  constexpr int64_t kBatch = 64 * U;
  const int64_t per = ((n16 + gridDim.x - 1) / gridDim.x + kBatch - 1) / kBatch * kBatch;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  const int lane = threadIdx.x;
  uint32_t acc = 0;
  uint4 ra[U], rb[U];
  int64_t i = b0;
  if (i < b1) batch_load<U, NT>(buf, i, b1, lane, ra);
  for (; i < b1; i += 2 * kBatch) {  // ra holds batch i on entry
    batch_load<U, NT>(buf, i + kBatch, b1, lane, rb);
    acc ^= batch_fold<U>(ra);
    batch_load<U, NT>(buf, i + 2 * kBatch, b1, lane, ra);
    acc ^= batch_fold<U>(rb);
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) sink[blockIdx.x] = acc;
}

// The same share read with direct loads into LDS (global_load_lds_dwordx4, as
// the decode kernel streams its chunks): batches of U 1 KB loads into one half
// of a per-wave ring, two batches in flight, each batch read back from LDS
// once it is in.  Loads past the share are clamped to its last 16 bytes.
template <int U, bool NT>
__global__ __launch_bounds__(64) void stream_read_lds_kernel(const uint4* buf, int64_t n16,
                                                             uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint4 ring[2][U][64];
  constexpr int64_t kBatch = 64 * U;
  const int64_t per = ((n16 + gridDim.x - 1) / gridDim.x + kBatch - 1) / kBatch * kBatch;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  const int lane = threadIdx.x;
  const uint32_t lane16 = 16u * lane;
  uint32_t acc = 0;
  auto issue = [&](int64_t i, int half) {
    lds_dma_begin();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // the instruction's 64 pieces; a piece past the share re-reads its last
      const int64_t k0 = i + 64 * u;
      const uint4* g = buf + (k0 < b1 ? k0 : b1 - 64 > b0 ? b1 - 64 : b0);
      lds_dma16<NT>(g, lds_addr(&ring[half][u][0]), lane16);
    }
  };
  int64_t i = b0;
  if (i < b1) issue(i, 0);
  int half = 0;
  for (; i < b1; i += kBatch) {
    if (i + kBatch < b1) {
      issue(i + kBatch, half ^ 1);
      wait_vm<U>();
    } else {
      wait_vm<0>();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint4 v = ring[half][u][lane];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    half ^= 1;
  }
  wait_vm<0>();
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) sink[blockIdx.x] = acc;
}

// mode: 0 plain loads, 1 nontemporal, 2 direct-to-LDS nontemporal, 3 direct-to-LDS plain
template <int U>
hipError_t sweep_launch(const void* buf, size_t bytes, uint32_t* sink, int waves, int mode,
                        hipStream_t st) {
  const uint4* b = static_cast<const uint4*>(buf);
  const int64_t n16 = (int64_t)(bytes / 16);
  switch (mode) {
    case 0: stream_read_sweep_kernel<U, false><<<waves, 64, 0, st>>>(b, n16, sink); break;
    case 1: stream_read_sweep_kernel<U, true><<<waves, 64, 0, st>>>(b, n16, sink); break;
    case 2: stream_read_lds_kernel<U, true><<<waves, 64, 0, st>>>(b, n16, sink); break;
    default: stream_read_lds_kernel<U, false><<<waves, 64, 0, st>>>(b, n16, sink); break;
  }
  return hipGetLastError();
}

// The decode partial kernel's chunk stream alone (kvq_probe_chunk_stream): a
// chunk's loads (up to 8 direct 1 KB loads, listed by the host: source,
// per-chunk stride, LDS offset, half-wave or full) go into one of two LDS
// slots, the next chunk is requested before the current one is read back, and
// spin dependent multiply-adds stand in for the arithmetic.  NI = loads per
// chunk (vmcnt takes an immediate: the launch picks the instantiation).
struct ChunkLoads {
  const char* src[8];
  int64_t stride[8];
  uint32_t dst[8];
  int32_t half[8];
};

template <int NI>
__global__ __launch_bounds__(64) void chunk_stream_kernel(ChunkLoads cl, int64_t n_chunks,
                                                          int spin, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char ring[2][4096];
  const int lane = threadIdx.x;
  const uint32_t lane16 = 16u * lane;
  const int64_t per = (n_chunks + gridDim.x - 1) / gridDim.x;
  const int64_t c0 = (int64_t)blockIdx.x * per;
  const int64_t c1 = c0 + per < n_chunks ? c0 + per : n_chunks;
  auto issue = [&](int64_t c, int s) {
    lds_dma_begin();
    const uint32_t base = lds_addr(&ring[s][0]);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t d = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(base + cl.dst[i]));
      if (!cl.half[i] || lane < 32) lds_dma16<true>(cl.src[i] + c * cl.stride[i], d, lane16);
    }
  };
  float x = (float)lane;
  uint32_t acc = 0;
  if (c0 < c1) issue(c0, 0);
  for (int64_t c = c0; c < c1; ++c) {
    const int s = (int)((c - c0) & 1);
    if (c + 1 < c1) {
      issue(c + 1, s ^ 1);
      wait_vm<NI>();
    } else {
      wait_vm<0>();
    }
    acc ^= reinterpret_cast<const uint32_t*>(&ring[s][0])[lane];
    for (int i = 0; i < spin; ++i) x = __builtin_fmaf(x, 0.999f, 0.5f);
  }
  wait_vm<0>();
  acc ^= __builtin_bit_cast(uint32_t, x);
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) sink[blockIdx.x] = acc;
}

}  // namespace

int probe_sink_words() { return kProbeBlocks * (kProbeThreads / 64); }

hipError_t launch_chunk_stream(const void* const (&bufs)[4], int64_t n_chunks,
                               const int32_t (&bytes)[4], int spin, int waves, uint32_t* sink,
                               hipStream_t st) {
  ChunkLoads cl{};
  int ni = 0;
  uint32_t dst = 0;
  for (int p = 0; p < 4; ++p) {
    for (int o = 0; o < bytes[p]; o += 1024) {
      if (ni == 8) return hipErrorInvalidValue;
      cl.src[ni] = static_cast<const char*>(bufs[p]) + o;
      cl.stride[ni] = bytes[p];
      cl.dst[ni] = dst + o;
      cl.half[ni] = o + 1024 > bytes[p];  // a 512-byte rest: half the lanes
      ++ni;
    }
    dst += bytes[p];
  }
  switch (ni) {
#define KVQ_CHUNK_CASE(N) \
    case N: chunk_stream_kernel<N><<<waves, 64, 0, st>>>(cl, n_chunks, spin, sink); break;
    KVQ_CHUNK_CASE(1) KVQ_CHUNK_CASE(2) KVQ_CHUNK_CASE(3) KVQ_CHUNK_CASE(4)
    KVQ_CHUNK_CASE(5) KVQ_CHUNK_CASE(6) KVQ_CHUNK_CASE(7) KVQ_CHUNK_CASE(8)
#undef KVQ_CHUNK_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_read_sweep(const void* buf, size_t bytes, uint32_t* sink, int waves,
                                    int loads, int mode, hipStream_t st) {
  switch (loads) {
    case 1: return sweep_launch<1>(buf, bytes, sink, waves, mode, st);
    case 2: return sweep_launch<2>(buf, bytes, sink, waves, mode, st);
    case 4: return sweep_launch<4>(buf, bytes, sink, waves, mode, st);
    case 8: return sweep_launch<8>(buf, bytes, sink, waves, mode, st);
    case 16: return sweep_launch<16>(buf, bytes, sink, waves, mode, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  stream_read_kernel<<<kProbeBlocks, kProbeThreads, 0, st>>>(
      static_cast<const uint4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace kvq
