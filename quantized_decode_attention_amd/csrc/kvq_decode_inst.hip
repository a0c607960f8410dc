// kvq_decode_inst.hip — one set of decode partial kernels: head dim KVQ_D,
// key bits KVQ_BK, dense (KVQ_PAGED 0) or paged (1) cache, under the entry
// name KVQ_INST.  The build compiles this file once per set, so that the sets
// compile in parallel; the kernels themselves are in kvq_decode_impl.h.
#include "kvq_decode_impl.h"

#if !defined(KVQ_D) || !defined(KVQ_BK) || !defined(KVQ_PAGED) || !defined(KVQ_INST)
#error "KVQ_D, KVQ_BK, KVQ_PAGED and KVQ_INST must be defined by the build"
#endif

namespace kvq {

hipError_t KVQ_INST(const DecodeLaunch& L, int op, int cus, int* workers, hipStream_t st) {
  return dispatch_bv<KVQ_D, KVQ_BK, KVQ_PAGED != 0>(L, op, cus, workers, st);
}

}  // namespace kvq
