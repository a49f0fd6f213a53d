// Decode kernels for FP8 E4M3FN keys (every value format and head dim).
#include "kvq_decode.h"

namespace kvq {

hipError_t decode_keys_fp8(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  return decode_for_keys<F_FP8, false>(fv, D, a, s);
}

}  // namespace kvq
