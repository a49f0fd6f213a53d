// Decode kernels for Walsh-Hadamard rotated INT4 group-32 keys (every value
// format and head dim): the query operand is the rotated query, fp16 hi + lo.
#include "kvq_decode.h"

namespace kvq {

hipError_t decode_keys_int4_rot(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  return decode_for_keys<F_INT4, true>(fv, D, a, s);
}

}  // namespace kvq
