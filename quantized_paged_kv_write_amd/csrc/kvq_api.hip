// C-ABI entry points: host-side validation, then launches on the caller's
// stream.  Nothing here allocates device memory, and only the diagnostics
// call synchronizes.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kvq_internal.h"

// Per-device error word (kvq_device_error bits; [0] accumulates, [1] receives
// the value taken by kvq_get_device_error).  Each device holds its own copy;
// host code uses the address hipGetSymbolAddress returns on that device.
__device__ __align__(16) uint32_t kvq_error_word[2];

// Decode workspace of kvq_decode_attn_noalloc: one fixed array per device,
// held from the library's load until the process ends.  Host code must not
// pass this name to a kernel (on the host it is only a stand-in): it uses the
// device address looked up per device below.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_WORKSPACE_BYTES];

namespace {

using namespace kvq;

// Device addresses of this library's file-scope device symbols, looked up
// once per device with that device current.
constexpr int kMaxDevices = 64;
struct DeviceSymbols {
  uint32_t* err = nullptr;
  uint8_t* scratch = nullptr;
};
std::atomic<bool> g_sym_ready[kMaxDevices];
DeviceSymbols g_sym[kMaxDevices];
std::mutex g_sym_mutex;

int device_symbols(DeviceSymbols* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KVQ_ERR_NO_DEVICE;
  if (dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  if (!g_sym_ready[dev].load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_sym_mutex);
    if (!g_sym_ready[dev].load(std::memory_order_relaxed)) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(kvq_error_word)) != hipSuccess || !p) return KVQ_ERR_HIP;
      void* ps = nullptr;
      if (hipGetSymbolAddress(&ps, HIP_SYMBOL(scratch)) != hipSuccess || !ps) return KVQ_ERR_HIP;
      g_sym[dev].err = static_cast<uint32_t*>(p);
      g_sym[dev].scratch = static_cast<uint8_t*>(ps);
      g_sym_ready[dev].store(true, std::memory_order_release);
    }
  }
  *out = g_sym[dev];
  return KVQ_OK;
}

// w[1] = the accumulated bits, w[0] = 0, in one atomic exchange.
__global__ void take_errors_kernel(uint32_t* w) {
  if (threadIdx.x == 0) w[1] = __hip_atomic_exchange(&w[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

bool sym_fmt(int32_t f) {
  return f == KVQ_INT8 || f == KVQ_FP8_E4M3FN || f == KVQ_INT4_G32 || f == KVQ_FP8_E5M2;
}

int check_cache(const kvq_cache* c) {
  if (!c) return KVQ_ERR_INVALID_ARG;
  if (c->num_blocks <= 0 || c->block_size <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0)
    return KVQ_ERR_INVALID_ARG;
  if (!(c->k_dtype >= KVQ_INT8 && c->k_dtype <= KVQ_FP8_E5M2)) return KVQ_ERR_INVALID_ARG;
  if (!sym_fmt(c->v_dtype)) {
    return (c->v_dtype == KVQ_INT4_KIVI) ? KVQ_ERR_UNSUPPORTED : KVQ_ERR_INVALID_ARG;
  }
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (!is_pow2(c->block_size) || c->block_size < 8 || c->block_size > 128) return KVQ_ERR_UNSUPPORTED;
  if ((int64_t)c->num_blocks * c->block_size * c->n_kv_heads >= (1ll << 31)) return KVQ_ERR_SHAPE;
  if (!c->k_codes || !c->v_codes || !c->k_scales || !c->v_scales) return KVQ_ERR_INVALID_ARG;
  if (c->k_dtype == KVQ_INT4_KIVI) {
    if (c->block_size != 32) return KVQ_ERR_SHAPE;
    if (c->max_seqs <= 0) return KVQ_ERR_SHAPE;
    if (!c->k_zeros || !c->k_tail || !c->v_tail) return KVQ_ERR_INVALID_ARG;
  }
  if (c->flags & ~(uint32_t)(KVQ_ROTATE_K | KVQ_ROTATE_V)) return KVQ_ERR_INVALID_ARG;
  if ((c->flags & KVQ_ROTATE_K) && c->k_dtype == KVQ_INT4_KIVI) return KVQ_ERR_UNSUPPORTED;  // per-channel keys
  return KVQ_OK;
}

int device_present() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return KVQ_ERR_NO_DEVICE;
  return KVQ_OK;
}

}  // namespace

extern "C" {

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument (NULL pointer, non-positive size or unknown enum)";
    case KVQ_ERR_UNSUPPORTED: return "unsupported format, head_dim or block_size";
    case KVQ_ERR_SHAPE: return "shape rule broken (KIVI needs block_size 32 and max_seqs > 0; sizes too large; "
                               "n_q_heads not a multiple of n_kv_heads)";
    case KVQ_ERR_WORKSPACE: return "decode workspace missing, too small or not 16-byte aligned";
    case KVQ_ERR_NO_DEVICE: return "no HIP device available";
    case KVQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown kvq status";
}

namespace {

// kvq_write and kvq_write_static: k_static / v_static are NULL for the
// dynamic per-token scale.
int write_impl(const kvq_cache* cache, const void* k, const void* v, const int64_t* slot_mapping,
               const int32_t* seq_idx, int64_t num_tokens, const void* k_static, const void* v_static,
               void* stream) {
  int rc = check_cache(cache);
  if (rc != KVQ_OK) return rc;
  if (k_static && cache->k_dtype == KVQ_INT4_KIVI) return KVQ_ERR_UNSUPPORTED;  // KIVI keys are dynamic
  if (num_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (num_tokens == 0) return KVQ_OK;
  if (!k || !v || !slot_mapping) return KVQ_ERR_INVALID_ARG;
  if (cache->k_dtype == KVQ_INT4_KIVI && !seq_idx) return KVQ_ERR_INVALID_ARG;
  if (num_tokens * (int64_t)cache->n_kv_heads >= (1ll << 31)) return KVQ_ERR_SHAPE;
  rc = device_present();
  if (rc != KVQ_OK) return rc;
  DeviceSymbols sym;
  rc = device_symbols(&sym);
  if (rc != KVQ_OK) return rc;
  WriteArgs a{};
  a.err = sym.err;
  a.k_static = static_cast<const uint16_t*>(k_static);
  a.v_static = static_cast<const uint16_t*>(v_static);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.slots = slot_mapping;
  a.seq_idx = seq_idx;
  a.T = num_tokens;
  a.H = cache->n_kv_heads;
  a.bs = cache->block_size;
  a.capacity = (int64_t)cache->num_blocks * cache->block_size;
  a.div_h = make_fastdiv((uint32_t)cache->n_kv_heads);
  a.k_codes = static_cast<uint8_t*>(cache->k_codes);
  a.k_scales = static_cast<uint16_t*>(cache->k_scales);
  a.k_zeros = static_cast<uint16_t*>(cache->k_zeros);
  a.v_codes = static_cast<uint8_t*>(cache->v_codes);
  a.v_scales = static_cast<uint16_t*>(cache->v_scales);
  a.k_tail = static_cast<uint16_t*>(cache->k_tail);
  a.v_tail = static_cast<uint16_t*>(cache->v_tail);
  a.max_seqs = cache->max_seqs;
  a.rot_k = (cache->flags & KVQ_ROTATE_K) ? 1 : 0;
  a.rot_v = (cache->flags & KVQ_ROTATE_V) ? 1 : 0;
  for (int i = 0; i < 8; ++i) a.rot_signs[i] = cache->rot_signs[i];
  // One launch takes at most 2^24 (token, head) rows, so that its grid stays
  // far below the 2^32 work-items of a dispatch.  Larger calls run as
  // consecutive calls on the same stream over consecutive token ranges:
  // tokens are independent, and a KIVI page split between two ranges is
  // completed by the second from the tail the first wrote, as across calls.
  const int64_t rows_per_launch = 1ll << 24;
  const int64_t step = std::max<int64_t>(1, rows_per_launch / cache->n_kv_heads);
  const size_t row_elems = (size_t)cache->n_kv_heads * cache->head_dim;
  for (int64_t t0 = 0; t0 < num_tokens; t0 += step) {
    const int64_t n = std::min(step, num_tokens - t0);
    a.k = static_cast<const uint16_t*>(k) + (size_t)t0 * row_elems;
    a.v = static_cast<const uint16_t*>(v) + (size_t)t0 * row_elems;
    a.slots = slot_mapping + t0;
    a.seq_idx = seq_idx ? seq_idx + t0 : nullptr;
    a.T = n;
    // KIVI seal waves: one per call token for small calls (decode steps),
    // one per 32 tokens otherwise
    a.seal_chunk = n <= 2048 ? 1 : 32;
    if (launch_write(*cache, a, static_cast<hipStream_t>(stream)) != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

}  // namespace

int kvq_write(const kvq_cache* cache, const void* k, const void* v, const int64_t* slot_mapping,
              const int32_t* seq_idx, int64_t num_tokens, void* stream) {
  return write_impl(cache, k, v, slot_mapping, seq_idx, num_tokens, nullptr, nullptr, stream);
}

int kvq_write_static(const kvq_cache* cache, const void* k, const void* v, const int64_t* slot_mapping,
                     int64_t num_tokens, const void* k_scale, const void* v_scale, void* stream) {
  if (!k_scale || !v_scale) return KVQ_ERR_INVALID_ARG;
  return write_impl(cache, k, v, slot_mapping, nullptr, num_tokens, k_scale, v_scale, stream);
}

int kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t n_q_heads,
                               int32_t max_blocks_per_seq, int32_t split_tokens, size_t* bytes) {
  int rc = check_cache(cache);
  if (rc != KVQ_OK) return rc;
  if (!bytes || batch < 0 || n_q_heads <= 0 || max_blocks_per_seq <= 0 || split_tokens < 0)
    return KVQ_ERR_INVALID_ARG;
  DecodePlan p;
  if (!plan_decode(*cache, batch, n_q_heads, max_blocks_per_seq, split_tokens, &p)) return KVQ_ERR_SHAPE;
  *bytes = p.bytes;
  return KVQ_OK;
}

namespace {

// kvq_decode_attn and kvq_decode_attn_noalloc; for the latter `workspace` is
// NULL and the per-device scratch array serves as the workspace.
int decode_impl(const kvq_cache* cache, const void* q, const int32_t* block_table, int32_t max_blocks_per_seq,
                const int32_t* ctx_lens, int32_t batch, int32_t n_q_heads, float sm_scale, int32_t split_tokens,
                void* out, void* workspace, size_t workspace_bytes, bool use_scratch, void* stream) {
  int rc = check_cache(cache);
  if (rc != KVQ_OK) return rc;
  if (batch < 0 || n_q_heads <= 0 || max_blocks_per_seq <= 0 || split_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return KVQ_ERR_SHAPE;
  const int32_t G = n_q_heads / cache->n_kv_heads;
  if (G > 16) return KVQ_ERR_UNSUPPORTED;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return KVQ_ERR_INVALID_ARG;
  if (batch == 0) return KVQ_OK;
  if (cache->k_dtype == KVQ_INT4_KIVI && batch > cache->max_seqs) return KVQ_ERR_SHAPE;  // tail row per sequence
  if (!q || !block_table || !ctx_lens || !out) return KVQ_ERR_INVALID_ARG;
  DecodePlan p;
  if (!plan_decode(*cache, batch, n_q_heads, max_blocks_per_seq, split_tokens, &p)) return KVQ_ERR_SHAPE;
  if (use_scratch) {
    if (p.bytes > KVQ_NOALLOC_WORKSPACE_BYTES) return KVQ_ERR_WORKSPACE;
  } else {
    if (!workspace || workspace_bytes < p.bytes) return KVQ_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0) return KVQ_ERR_WORKSPACE;
  }
  rc = device_present();
  if (rc != KVQ_OK) return rc;
  DeviceSymbols sym;
  rc = device_symbols(&sym);
  if (rc != KVQ_OK) return rc;
  if (use_scratch) workspace = sym.scratch;  // this device's copy of the array
  DecodeArgs a{};
  a.err = sym.err;
  a.q = static_cast<const uint16_t*>(q);
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.max_blocks = max_blocks_per_seq;
  a.B = batch;
  a.Hq = n_q_heads;
  a.H = cache->n_kv_heads;
  a.G = G;
  a.bs = cache->block_size;
  a.log2_bs = 0;
  while ((1 << a.log2_bs) < cache->block_size) ++a.log2_bs;
  a.nb = cache->num_blocks;
  const float scale = sm_scale == 0.0f ? 1.0f / sqrtf((float)cache->head_dim) : sm_scale;
  a.qscale = scale * 1.4426950408889634f;  // log2(e): the softmax runs on exp2
  a.k_codes = static_cast<const uint8_t*>(cache->k_codes);
  a.k_scales = static_cast<const uint16_t*>(cache->k_scales);
  a.k_zeros = static_cast<const uint16_t*>(cache->k_zeros);
  a.v_codes = static_cast<const uint8_t*>(cache->v_codes);
  a.v_scales = static_cast<const uint16_t*>(cache->v_scales);
  a.k_tail = static_cast<const uint16_t*>(cache->k_tail);
  a.v_tail = static_cast<const uint16_t*>(cache->v_tail);
  a.max_seqs = cache->max_seqs;
  a.hp_log2 = heads_per_wave_log2(*cache, G);
  a.share_tiles = p.share_tiles;
  a.max_shares = p.max_shares;
  a.num_shares = p.max_shares;  // the launcher may use fewer
  a.plan = static_cast<int32_t*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + p.plan_bytes);
  a.out = static_cast<uint16_t*>(out);
  a.rot_k = (cache->flags & KVQ_ROTATE_K) ? 1 : 0;
  a.rot_v = (cache->flags & KVQ_ROTATE_V) ? 1 : 0;
  for (int i = 0; i < 8; ++i) a.rot_signs[i] = cache->rot_signs[i];
  a.qrot = a.rot_k ? reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + p.qrot_offset) : nullptr;
  return launch_decode(*cache, a, static_cast<hipStream_t>(stream)) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

int kvq_decode_attn(const kvq_cache* cache, const void* q, const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* ctx_lens, int32_t batch, int32_t n_q_heads, float sm_scale,
                    int32_t split_tokens, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(cache, q, block_table, max_blocks_per_seq, ctx_lens, batch, n_q_heads, sm_scale, split_tokens,
                     out, workspace, workspace_bytes, false, stream);
}

int kvq_decode_attn_noalloc(const kvq_cache* cache, const void* q, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* ctx_lens, int32_t batch, int32_t n_q_heads,
                            float sm_scale, int32_t split_tokens, void* out, void* stream) {
  return decode_impl(cache, q, block_table, max_blocks_per_seq, ctx_lens, batch, n_q_heads, sm_scale, split_tokens,
                     out, nullptr, 0, true, stream);
}

int kvq_prefill_workspace_bytes(const kvq_cache* cache, int64_t total_q, int32_t n_q_heads, size_t* bytes) {
  int rc = check_cache(cache);
  if (rc != KVQ_OK) return rc;
  if (!bytes || total_q < 0 || n_q_heads <= 0) return KVQ_ERR_INVALID_ARG;
  if (total_q * n_q_heads * (int64_t)cache->head_dim >= (1ll << 31)) return KVQ_ERR_SHAPE;
  *bytes = (cache->flags & KVQ_ROTATE_K) ? 2 * (size_t)total_q * n_q_heads * cache->head_dim * 2 : 0;
  return KVQ_OK;
}

int kvq_prefill_attn(const kvq_cache* cache, const void* q, const int32_t* q_start, const int32_t* block_table,
                     int32_t max_blocks_per_seq, const int32_t* ctx_lens, int32_t batch, int64_t total_q,
                     int32_t n_q_heads, int32_t max_q_len, float sm_scale, void* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int rc = check_cache(cache);
  if (rc != KVQ_OK) return rc;
  if (batch < 0 || total_q < 0 || n_q_heads <= 0 || max_blocks_per_seq <= 0 || max_q_len < 0)
    return KVQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return KVQ_ERR_SHAPE;
  if (!(sm_scale >= 0.0f) || isinf(sm_scale)) return KVQ_ERR_INVALID_ARG;
  const int32_t G = n_q_heads / cache->n_kv_heads;
  if (total_q * n_q_heads * (int64_t)cache->head_dim >= (1ll << 31)) return KVQ_ERR_SHAPE;
  if ((int64_t)max_q_len * G >= (1ll << 30)) return KVQ_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * cache->block_size >= (1ll << 30)) return KVQ_ERR_SHAPE;
  if (batch == 0 || total_q == 0 || max_q_len == 0) return KVQ_OK;
  if (cache->k_dtype == KVQ_INT4_KIVI && batch > cache->max_seqs) return KVQ_ERR_SHAPE;  // tail row per sequence
  if (!q || !q_start || !block_table || !ctx_lens || !out) return KVQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(out) & 15) != 0 || (reinterpret_cast<uintptr_t>(q) & 15) != 0)
    return KVQ_ERR_INVALID_ARG;
  size_t need = 0;
  rc = kvq_prefill_workspace_bytes(cache, total_q, n_q_heads, &need);
  if (rc != KVQ_OK) return rc;
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15) != 0))
    return KVQ_ERR_WORKSPACE;
  // query tiles of one (sequence, KV head): rows of 128 (head_dim <= 128) or 64
  const int32_t rows_per_tile = cache->head_dim <= 128 ? 128 : 64;
  const int64_t n_qtiles = ((int64_t)max_q_len * G + rows_per_tile - 1) / rows_per_tile;
  const int64_t n_wg = (int64_t)batch * cache->n_kv_heads * n_qtiles;
  if (n_wg >= (1ll << 31) - 8) return KVQ_ERR_SHAPE;
  rc = device_present();
  if (rc != KVQ_OK) return rc;
  DeviceSymbols sym;
  rc = device_symbols(&sym);
  if (rc != KVQ_OK) return rc;
  PrefillArgs a{};
  a.err = sym.err;
  a.q = static_cast<const uint16_t*>(q);
  a.qrot = need > 0 ? static_cast<const uint16_t*>(workspace) : nullptr;
  a.q_start = q_start;
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.Tq = total_q;
  a.max_blocks = max_blocks_per_seq;
  a.B = batch;
  a.Hq = n_q_heads;
  a.H = cache->n_kv_heads;
  a.G = G;
  a.bs = cache->block_size;
  a.log2_bs = 0;
  while ((1 << a.log2_bs) < cache->block_size) ++a.log2_bs;
  a.nb = cache->num_blocks;
  a.max_q_len = max_q_len;
  a.n_qtiles = (int32_t)n_qtiles;
  a.n_wg = (int32_t)n_wg;
  const float scale = sm_scale == 0.0f ? 1.0f / sqrtf((float)cache->head_dim) : sm_scale;
  a.qscale = scale * 1.4426950408889634f;  // log2(e): the softmax runs on exp2
  a.k_codes = static_cast<const uint8_t*>(cache->k_codes);
  a.k_scales = static_cast<const uint16_t*>(cache->k_scales);
  a.k_zeros = static_cast<const uint16_t*>(cache->k_zeros);
  a.v_codes = static_cast<const uint8_t*>(cache->v_codes);
  a.v_scales = static_cast<const uint16_t*>(cache->v_scales);
  a.k_tail = static_cast<const uint16_t*>(cache->k_tail);
  a.v_tail = static_cast<const uint16_t*>(cache->v_tail);
  a.max_seqs = cache->max_seqs;
  a.out = static_cast<uint16_t*>(out);
  a.rot_k = (cache->flags & KVQ_ROTATE_K) ? 1 : 0;
  a.rot_v = (cache->flags & KVQ_ROTATE_V) ? 1 : 0;
  for (int i = 0; i < 8; ++i) a.rot_signs[i] = cache->rot_signs[i];
  return launch_prefill(*cache, a, static_cast<hipStream_t>(stream)) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_get_device_error(void* stream) {
  int rc = device_present();
  if (rc != KVQ_OK) return rc;
  DeviceSymbols sym;
  rc = device_symbols(&sym);
  if (rc != KVQ_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(take_errors_kernel, dim3(1), dim3(64), 0, st, sym.err);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  uint32_t bits = 0;
  if (hipMemcpyAsync(&bits, sym.err + 1, sizeof(bits), hipMemcpyDeviceToHost, st) != hipSuccess) return KVQ_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return KVQ_ERR_HIP;
  return (int)(bits & 0x7FFFFFFFu);
}

}  // extern "C"
