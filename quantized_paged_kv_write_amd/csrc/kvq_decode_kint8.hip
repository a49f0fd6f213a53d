// Decode kernels for INT8 keys (every value format and head dim).
#include "kvq_decode.h"

namespace kvq {

hipError_t decode_keys_int8(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  return decode_for_keys<F_INT8, false>(fv, D, a, s);
}

}  // namespace kvq
