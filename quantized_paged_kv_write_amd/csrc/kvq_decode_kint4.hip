// Decode kernels for INT4 group-32 keys (every value format and head dim).
#include "kvq_decode.h"

namespace kvq {

hipError_t decode_keys_int4(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  return decode_for_keys<F_INT4, false>(fv, D, a, s);
}

}  // namespace kvq
