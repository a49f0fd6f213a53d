// Decode kernels for Walsh-Hadamard rotated FP8 E5M2 keys (every value format
// and head dim): the query operand is the rotated query, fp16 hi + lo.
#include "kvq_decode.h"

namespace kvq {

hipError_t decode_keys_e5m2_rot(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  return decode_for_keys<F_E5M2, true>(fv, D, a, s);
}

}  // namespace kvq
