// kvq_decode.hip — the decode combine kernel and the routing of partial-kernel
// launches to their instantiation set (head dim, key bits, dense or paged).
#include "kvq_decode_impl.h"

namespace kvq {
namespace {

using SetFn = hipError_t (*)(const DecodeLaunch&, int, int, int*, hipStream_t);

hipError_t partial_entry(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  // [paged][head dim 64 / 128][key bits 2 / 4 / 8]
  static const SetFn sets[2][2][3] = {
      {{decode_partial_d64_k2, decode_partial_d64_k4, decode_partial_d64_k8},
       {decode_partial_d128_k2, decode_partial_d128_k4, decode_partial_d128_k8}},
      {{decode_partial_paged_d64_k2, decode_partial_paged_d64_k4, decode_partial_paged_d64_k8},
       {decode_partial_paged_d128_k2, decode_partial_paged_d128_k4,
        decode_partial_paged_d128_k8}}};
  const int bk = L.g.bK == 2 ? 0 : L.g.bK == 4 ? 1 : L.g.bK == 8 ? 2 : -1;
  if (bk < 0 || (L.g.D != 64 && L.g.D != 128)) return hipErrorInvalidValue;
  return sets[L.g.table != nullptr][L.g.D == 128][bk](L, op, cus, workers, st);
}

template <int D, int GQ>
hipError_t combine_rows(const DecodeLaunch& L, hipStream_t st) {
  if (L.g.B * L.g.Hkv < kCombineRowUnits && GQ > 1)
    decode_combine_kernel<KiviWork, D, GQ, 1><<<dim3(L.g.Hkv * GQ, L.g.B), kThreads, 0, st>>>(L);
  else if constexpr (GQ * D > 4 * kThreads)  // more outputs than threads: groups of rows,
    // two threads per output (16 rows at D = 128: four workgroups of four rows
    // per unit; T = 4 partial + combine 95.7 -> 94.5 us on one box)
    decode_combine_kernel<KiviWork, D, GQ, 2 * kThreads / D>
        <<<dim3(L.g.Hkv * (GQ * D / (2 * kThreads)), L.g.B), kThreads, 0, st>>>(L);
  else
    decode_combine_kernel<KiviWork, D, GQ><<<dim3(L.g.Hkv, L.g.B), kThreads, 0, st>>>(L);
  return hipGetLastError();
}

template <int D>
hipError_t combine_gq(const DecodeLaunch& L, hipStream_t st) {
  switch (L.gq) {
    case 1: return combine_rows<D, 1>(L, st);
    case 2: return combine_rows<D, 2>(L, st);
    case 4: return combine_rows<D, 4>(L, st);
    case 8: return combine_rows<D, 8>(L, st);
    case 16: return combine_rows<D, 16>(L, st);
    default: return hipErrorInvalidValue;
  }
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
