// Dequantizing paged decode attention (gfx950): host-side partition and
// dispatch.  The kernels are in kvq_decode.h; each key format's kernels are
// compiled in a translation unit of their own (kvq_decode_k*.hip) so the
// build runs in parallel.
#include <algorithm>

#include "kvq_decode.h"

namespace kvq {

int32_t heads_per_wave_log2(const kvq_cache& c, int32_t G) {
  int32_t l = 0;
  while (l < 2 && ((2 << l) * G) <= 16 && c.n_kv_heads % (2 << l) == 0) ++l;
  return l;
}

bool plan_decode(const kvq_cache& c, int32_t batch, int32_t n_q_heads, int32_t max_blocks, int32_t split_tokens,
                 DecodePlan* p) {
  if (n_q_heads <= 0 || n_q_heads % c.n_kv_heads != 0) return false;
  const int32_t hp_log2 = heads_per_wave_log2(c, n_q_heads / c.n_kv_heads);
  const int32_t tile_tokens = TILE >> hp_log2;
  const int32_t groups = c.n_kv_heads >> hp_log2;  // waves per share
  const int64_t max_tok = (int64_t)max_blocks * c.block_size;  // tokens one block-table row addresses
  if (max_tok >= (1ll << 30)) return false;
  const int64_t bound = (int64_t)batch * ((max_tok + tile_tokens - 1) / tile_tokens);  // tiles of the call, at most
  if (bound >= (1ll << 30)) return false;
  int64_t shares;
  if (split_tokens > 0) {
    const int64_t S = ((int64_t)split_tokens + tile_tokens - 1) / tile_tokens;
    shares = (bound + S - 1) / S;
    p->share_tiles = (int32_t)S;
  } else {
    shares = std::min<int64_t>((AUTO_MAX_WAVES + groups - 1) / groups, (bound + AUTO_MIN_TILES - 1) / AUTO_MIN_TILES);
    p->share_tiles = 0;
  }
  if (shares < 1) shares = 1;
  if (shares > (1 << 24)) return false;
  p->max_shares = (int32_t)shares;
  const size_t ints = 2 + (size_t)batch + (size_t)shares;
  p->plan_bytes = (ints * sizeof(int32_t) + 255) / 256 * 256;
  p->records = (size_t)shares + batch;
  p->bytes = p->plan_bytes + p->records * n_q_heads * ((size_t)c.head_dim + 2) * sizeof(float);
  return true;
}

hipError_t launch_decode(const kvq_cache& c, const DecodeArgs& a, hipStream_t s) {
  switch (c.k_dtype) {
    case F_INT8: return decode_keys_int8(c.v_dtype, c.head_dim, a, s);
    case F_FP8: return decode_keys_fp8(c.v_dtype, c.head_dim, a, s);
    case F_KIVI: return decode_keys_kivi(c.v_dtype, c.head_dim, a, s);
    case F_E5M2: return decode_keys_e5m2(c.v_dtype, c.head_dim, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
