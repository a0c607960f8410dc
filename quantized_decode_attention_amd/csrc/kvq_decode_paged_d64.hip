// kvq_decode_paged_d64.hip — the decode partial kernels for head dim 64 over
// the paged cache (one translation unit per head dim and cache form, so that
// they compile in parallel; the kernels are in kvq_decode_impl.h).
#include "kvq_decode_impl.h"

namespace kvq {

hipError_t decode_partial_paged_d64(const DecodeLaunch& L, int op, int cus, int* workers,
                             hipStream_t st) {
  return dispatch_bits<64, true>(L, op, cus, workers, st);
}

}  // namespace kvq
