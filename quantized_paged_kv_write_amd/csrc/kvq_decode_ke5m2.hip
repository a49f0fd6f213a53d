// Decode kernels for FP8 E5M2 keys (every value format and head dim).
#include "kvq_decode.h"

namespace kvq {

hipError_t decode_keys_e5m2(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  return decode_for_keys<F_E5M2, false>(fv, D, a, s);
}

}  // namespace kvq
