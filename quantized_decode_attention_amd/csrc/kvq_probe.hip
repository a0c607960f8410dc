// kvq_probe.hip — a plain streaming read (measurement aid, kvq_probe.h):
// every wave reads a contiguous share of the buffer with 16-byte loads, four
// in flight per lane, and folds them into one word so that none is dropped.
#include "kvq_internal.h"

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

}  // namespace

int probe_sink_words() { return kProbeBlocks * (kProbeThreads / 64); }

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  stream_read_kernel<<<kProbeBlocks, kProbeThreads, 0, st>>>(
      static_cast<const uint4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace kvq
