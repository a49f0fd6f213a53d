// Decode kernels for KIVI-style INT4 keys (every value format and head dim).
#include "kvq_decode.h"

namespace kvq {

hipError_t decode_keys_kivi(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  return decode_for_keys<F_KIVI, false>(fv, D, a, s);
}

}  // namespace kvq
