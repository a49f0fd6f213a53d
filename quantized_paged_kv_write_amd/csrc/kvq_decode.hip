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
  const size_t end = p->plan_bytes + p->records * n_q_heads * ((size_t)c.head_dim + 2) * sizeof(float);
  p->qrot_offset = (end + 255) / 256 * 256;
  // rotated keys: the rotated query, fp16 hi and lo (B, Hq, D) each
  p->bytes = (c.flags & KVQ_ROTATE_K) ? p->qrot_offset + 2 * (size_t)batch * n_q_heads * c.head_dim * 2 : end;
  return true;
}

namespace {

// The rotated query of rotated keys ("Quantized KV caches in production",
// Numerical Formats: Walsh-Hadamard rotation): q' = H (sigma q) / D for every
// row (a query head of a sequence or of a chunk position), written as fp16
// hi = RN(q') and lo = RN(q' - hi).  One wave per row; lane l holds channels
// l CPL .. l CPL + CPL - 1.  The transform runs in float64 and is exact (sums
// of at most 256 fp16 values); 1/D is a power of two.
struct RotQArgs {
  const uint16_t* q;
  uint16_t* qrot;
  size_t rows;
  uint32_t signs[8];
};

template <int D>
__global__ __launch_bounds__(256) void rotate_q_kernel(RotQArgs a) {
  constexpr int CPL = D / 64;
  const int lane = (int)threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;  // uniform over the wave
  const uint16_t* qr = a.q + row * D;
  double y[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane * CPL + i;
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) w = (c >> 5) == k ? a.signs[k] : w;
    const double x = (double)h2f(qr[c]);
    y[i] = ((w >> (c & 31)) & 1) ? -x : x;
  }
#pragma unroll
  for (int s = 1; s < CPL; s <<= 1) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      if (i & s) continue;
      const double u = y[i], v = y[i + s];
      y[i] = u + v;
      y[i + s] = u - v;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const double p = __shfl_xor(y[i], m);
      y[i] = (lane & m) ? p - y[i] : y[i] + p;
    }
  }
  uint16_t* hi = a.qrot + row * D;
  uint16_t* lo = a.qrot + a.rows * D + row * D;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const double qp = y[i] * (1.0 / D);
    const uint32_t h = f2h_bits((float)qp);
    hi[lane * CPL + i] = (uint16_t)h;
    lo[lane * CPL + i] = (uint16_t)f2h_bits((float)(qp - (double)h2f(h)));
  }
}

}  // namespace

hipError_t launch_rotate_query(const uint16_t* q, uint16_t* qrot, size_t rows, int D, const uint32_t* signs,
                               hipStream_t s) {
  RotQArgs a{q, qrot, rows, {}};
  for (int i = 0; i < 8; ++i) a.signs[i] = signs[i];
  if (rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  switch (D) {
    case 64: hipLaunchKernelGGL(rotate_q_kernel<64>, dim3(blocks), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(rotate_q_kernel<128>, dim3(blocks), dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(rotate_q_kernel<256>, dim3(blocks), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const kvq_cache& c, const DecodeArgs& a, hipStream_t s) {
  if (a.rot_k) {
    const hipError_t e = launch_rotate_query(a.q, a.qrot, (size_t)a.B * a.Hq, c.head_dim, a.rot_signs, s);
    if (e != hipSuccess) return e;
    switch (c.k_dtype) {
      case F_INT8: return decode_keys_int8_rot(c.v_dtype, c.head_dim, a, s);
      case F_FP8: return decode_keys_fp8_rot(c.v_dtype, c.head_dim, a, s);
      case F_E5M2: return decode_keys_e5m2_rot(c.v_dtype, c.head_dim, a, s);
      case F_INT4: return decode_keys_int4_rot(c.v_dtype, c.head_dim, a, s);
    }
    return hipErrorInvalidValue;
  }
  switch (c.k_dtype) {
    case F_INT8: return decode_keys_int8(c.v_dtype, c.head_dim, a, s);
    case F_FP8: return decode_keys_fp8(c.v_dtype, c.head_dim, a, s);
    case F_KIVI: return decode_keys_kivi(c.v_dtype, c.head_dim, a, s);
    case F_E5M2: return decode_keys_e5m2(c.v_dtype, c.head_dim, a, s);
    case F_INT4: return decode_keys_int4(c.v_dtype, c.head_dim, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
