// Chunked-prefill kernels for KIVI keys (every value format and head dim,
// plain or Walsh-Hadamard rotated keys).
#include "kvq_prefill.h"

namespace kvq {

hipError_t prefill_keys_kivi(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s) {
  return prefill_for_keys<F_KIVI>(fv, D, rot, a, s);
}

}  // namespace kvq
