// kvq_decode.hip — the decode combine kernel and the routing of partial-kernel
// launches to their translation unit (head dim, dense or paged cache).
#include "kvq_decode_impl.h"

namespace kvq {
namespace {

hipError_t partial_entry(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  const bool paged = L.g.table != nullptr;
  if (L.g.D == 64)
    return paged ? decode_partial_paged_d64(L, op, cus, workers, st)
                 : decode_partial_d64(L, op, cus, workers, st);
  return paged ? decode_partial_paged_d128(L, op, cus, workers, st)
               : decode_partial_d128(L, op, cus, workers, st);
}

template <int D>
hipError_t combine_gq(const DecodeLaunch& L, hipStream_t st) {
  dim3 grid(L.g.Hkv, L.g.B);
  switch (L.gq) {
    case 1: decode_combine_kernel<KiviWork, D, 1><<<grid, kThreads, 0, st>>>(L); break;
    case 2: decode_combine_kernel<KiviWork, D, 2><<<grid, kThreads, 0, st>>>(L); break;
    case 4: decode_combine_kernel<KiviWork, D, 4><<<grid, kThreads, 0, st>>>(L); break;
    case 8: decode_combine_kernel<KiviWork, D, 8><<<grid, kThreads, 0, st>>>(L); break;
    case 16: decode_combine_kernel<KiviWork, D, 16><<<grid, kThreads, 0, st>>>(L); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t decode_workers(const Geom& g, int gq, int cus, int* workers) {
  DecodeLaunch L{};
  L.g = g;
  L.gq = gq;
  return partial_entry(L, 1, cus, workers, nullptr);
}

hipError_t launch_decode_partial(const DecodeLaunch& L, hipStream_t st) {
  return partial_entry(L, 0, 0, nullptr, st);
}

hipError_t launch_decode_combine(const DecodeLaunch& L, hipStream_t st) {
  return L.g.D == 64 ? combine_gq<64>(L, st) : combine_gq<128>(L, st);
}

}  // namespace kvq
