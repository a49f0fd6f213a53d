// Chunked-prefill kernels for INT4 group-32 keys (every value format and head
// dim, plain or Walsh-Hadamard rotated keys).
#include "kvq_prefill.h"

namespace kvq {

hipError_t prefill_keys_int4(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s) {
  return prefill_for_keys<F_INT4>(fv, D, rot, a, s);
}

}  // namespace kvq
