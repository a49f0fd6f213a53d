// Moving whole quantized pages between two caches of the same geometry, such
// as the device cache and a pool of pages in pinned host memory ("Use Less
// Memory: Quantization and Offloading", section 4 "Pipelining and Latency
// Overlap": quantized blocks offloaded to CPU RAM and prefetched for the
// next step by asynchronous DMA into a second set of GPU buffers, while the
// current step computes).
//
// A page of a cache is one contiguous run of bytes in each of its paged
// buffers (codes, scales, KIVI zero points), so a batch of pages becomes a
// few hipMemcpyAsync calls: runs of consecutive source and destination ids
// are merged into one copy per buffer.  The copies go to the DMA engines,
// so they overlap kernels on other streams without taking compute units.
#include <algorithm>
#include <vector>

#include "kvq_internal.h"

namespace {

using namespace kvq;

struct PagedBuffer {
  char* src;
  char* dst;
  size_t page_bytes;
};

int code_bytes(int32_t fmt, int32_t D) { return (fmt == KVQ_INT4_G32 || fmt == KVQ_INT4_KIVI) ? D / 2 : D; }

// Bytes per page of each paged buffer, or an error for unusable caches.
int paged_buffers(const kvq_cache* s, const kvq_cache* d, std::vector<PagedBuffer>* out) {
  if (!s || !d) return KVQ_ERR_INVALID_ARG;
  if (s->block_size != d->block_size || s->n_kv_heads != d->n_kv_heads || s->head_dim != d->head_dim ||
      s->k_dtype != d->k_dtype || s->v_dtype != d->v_dtype)
    return KVQ_ERR_SHAPE;
  const int32_t bs = s->block_size, H = s->n_kv_heads, D = s->head_dim;
  if (s->num_blocks <= 0 || d->num_blocks <= 0 || bs <= 0 || H <= 0 || D <= 0) return KVQ_ERR_INVALID_ARG;
  if (!(s->k_dtype >= KVQ_INT8 && s->k_dtype <= KVQ_FP8_E5M2) || !(s->v_dtype >= KVQ_INT8 && s->v_dtype <= KVQ_FP8_E5M2) ||
      s->v_dtype == KVQ_INT4_KIVI)
    return KVQ_ERR_INVALID_ARG;
  const bool kivi = s->k_dtype == KVQ_INT4_KIVI;
  auto scale_bytes = [&](int32_t f) -> size_t {
    if (f == KVQ_INT4_KIVI) return (size_t)H * D * 2;             // (H, D) fp16 per page
    if (f == KVQ_INT4_G32) return (size_t)bs * H * (D / 32) * 2;  // (bs, H, D/32)
    return (size_t)bs * H * 2;                                    // (bs, H)
  };
  const void* sp[5] = {s->k_codes, s->v_codes, s->k_scales, s->v_scales, s->k_zeros};
  const void* dp[5] = {d->k_codes, d->v_codes, d->k_scales, d->v_scales, d->k_zeros};
  const size_t pb[5] = {(size_t)bs * H * code_bytes(s->k_dtype, D), (size_t)bs * H * code_bytes(s->v_dtype, D),
                        scale_bytes(s->k_dtype), scale_bytes(s->v_dtype), (size_t)H * D * 2};
  const int nbuf = kivi ? 5 : 4;
  out->clear();
  for (int i = 0; i < nbuf; ++i) {
    if (!sp[i] || !dp[i]) return KVQ_ERR_INVALID_ARG;
    out->push_back(PagedBuffer{static_cast<char*>(const_cast<void*>(sp[i])), static_cast<char*>(const_cast<void*>(dp[i])),
                               pb[i]});
  }
  return KVQ_OK;
}

}  // namespace

extern "C" int kvq_copy_blocks(const kvq_cache* src, const kvq_cache* dst, const int32_t* src_blocks,
                               const int32_t* dst_blocks, int32_t n, void* stream) {
  std::vector<PagedBuffer> bufs;
  int rc = paged_buffers(src, dst, &bufs);
  if (rc != KVQ_OK) return rc;
  if (n < 0) return KVQ_ERR_INVALID_ARG;
  if (n == 0) return KVQ_OK;
  if (!src_blocks || !dst_blocks) return KVQ_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (src_blocks[i] < 0 || src_blocks[i] >= src->num_blocks || dst_blocks[i] < 0 || dst_blocks[i] >= dst->num_blocks)
      return KVQ_ERR_INVALID_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return KVQ_ERR_NO_DEVICE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // runs [i, j) with consecutive source and destination ids, in list order.
  // (One hipMemcpyAsync per run and buffer: the batched copy call is newer
  // than the HIP runtime that PyTorch-ROCm processes load.)
  int32_t i = 0;
  while (i < n) {
    int32_t j = i + 1;
    while (j < n && src_blocks[j] == src_blocks[j - 1] + 1 && dst_blocks[j] == dst_blocks[j - 1] + 1) ++j;
    const size_t pages = (size_t)(j - i);
    for (const PagedBuffer& b : bufs) {
      if (hipMemcpyAsync(b.dst + (size_t)dst_blocks[i] * b.page_bytes, b.src + (size_t)src_blocks[i] * b.page_bytes,
                         pages * b.page_bytes, hipMemcpyDefault, st) != hipSuccess)
        return KVQ_ERR_HIP;
    }
    i = j;
  }
  return KVQ_OK;
}
