// kvq_decode_d128.hip — the decode partial kernels for head dim 128 over
// the dense cache (one translation unit per head dim and cache form, so that
// they compile in parallel; the kernels are in kvq_decode_impl.h).
#include "kvq_decode_impl.h"

namespace kvq {

hipError_t decode_partial_d128(const DecodeLaunch& L, int op, int cus, int* workers,
                             hipStream_t st) {
  return dispatch_bits<128, false>(L, op, cus, workers, st);
}

}  // namespace kvq
