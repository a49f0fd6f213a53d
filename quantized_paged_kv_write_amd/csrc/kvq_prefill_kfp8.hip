// Chunked-prefill kernels for FP8 keys (every value format and head dim,
// plain or Walsh-Hadamard rotated keys).
#include "kvq_prefill.h"

namespace kvq {

hipError_t prefill_keys_fp8(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s) {
  return prefill_for_keys<F_FP8>(fv, D, rot, a, s);
}

}  // namespace kvq
