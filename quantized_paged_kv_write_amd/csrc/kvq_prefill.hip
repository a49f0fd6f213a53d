// Chunked-prefill attention (gfx950): dispatch to the per-key-format
// translation units (kvq_prefill_k*.hip); the kernel is in kvq_prefill.h.
#include "kvq_internal.h"

namespace kvq {

hipError_t launch_prefill(const kvq_cache& c, const PrefillArgs& a, hipStream_t s) {
  const bool rot = a.rot_k != 0;
  if (rot) {
    const hipError_t e = launch_rotate_query(a.q, const_cast<uint16_t*>(a.qrot), (size_t)a.Tq * a.Hq, c.head_dim,
                                             a.rot_signs, s);
    if (e != hipSuccess) return e;
  }
  switch (c.k_dtype) {
    case KVQ_INT8: return prefill_keys_int8(c.v_dtype, c.head_dim, rot, a, s);
    case KVQ_FP8_E4M3FN: return prefill_keys_fp8(c.v_dtype, c.head_dim, rot, a, s);
    case KVQ_INT4_KIVI: return prefill_keys_kivi(c.v_dtype, c.head_dim, rot, a, s);
    case KVQ_FP8_E5M2: return prefill_keys_e5m2(c.v_dtype, c.head_dim, rot, a, s);
    case KVQ_INT4_G32: return prefill_keys_int4(c.v_dtype, c.head_dim, rot, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
