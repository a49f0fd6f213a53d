// Chunked-prefill kernels for E5M2 keys (every value format and head dim,
// plain or Walsh-Hadamard rotated keys).
#include "kvq_prefill.h"

namespace kvq {

hipError_t prefill_keys_e5m2(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s) {
  return prefill_for_keys<F_E5M2>(fv, D, rot, a, s);
}

}  // namespace kvq
