// Stand-ins for the device-side launchers of libkvq, so that its host code
// (kvq_api.cpp: argument checks, sizes, error text) can be built alone under
// the host sanitizers and run without a GPU.  Every launcher reports that no
// device is present.
#include "../../quantized_decode_attention_amd/csrc/kvq_internal.h"

namespace kvq {

hipError_t launch_quantize_keys(const Geom&, const uint16_t*, int64_t, int32_t, int32_t,
                                uint32_t*, uint16_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_quantize_values(const Geom&, const uint16_t*, int64_t, int32_t, int32_t,
                                  uint32_t*, uint16_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_residual_copy(const Geom&, const uint16_t*, int64_t, int32_t, int32_t,
                                uint16_t*, bool, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_append(const Geom&, const uint16_t*, const uint16_t*, const int32_t*,
                         const kvq_cache&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_append_tokens(const Geom&, int, const uint16_t*, const uint16_t*,
                                const int32_t*, const kvq_cache&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t decode_workers(const Geom&, int, int, int*) { return hipErrorNoDevice; }
hipError_t launch_decode_partial(const DecodeLaunch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_combine(const DecodeLaunch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bq2_prefill(const Bq2Geom&, const uint16_t*, const uint16_t*, int32_t,
                              const kvq_bq2_cache&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bq2_append(const Bq2Geom&, const uint16_t*, const uint16_t*, const int32_t*,
                             const kvq_bq2_cache&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t bq2_decode_workers(const Bq2Geom&, int, int*) { return hipErrorNoDevice; }
hipError_t launch_bq2_decode_partial(const Bq2Launch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bq2_decode_combine(const Bq2Launch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(void**, size_t*) { return hipErrorNoDevice; }
int probe_sink_words() { return 8192; }
hipError_t launch_stream_read(const void*, size_t, uint32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_stream_read_sweep(const void*, size_t, uint32_t*, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_chunk_stream(const void* const (&)[4], int64_t, const int32_t (&)[4], int, int,
                               uint32_t*, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace kvq
