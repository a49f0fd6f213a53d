// Moving whole quantized pages between two caches of the same geometry, such
// as the device cache and a pool of pages in pinned host memory ("Use Less
// Memory: Quantization and Offloading", section 4 "Pipelining and Latency
// Overlap": quantized blocks offloaded to CPU RAM and prefetched for the
// next step by asynchronous DMA into a second set of GPU buffers, while the
// current step computes).
//
// A page of a cache is one contiguous run of bytes in each of its paged
// buffers (codes, scales, KIVI zero points).  Two engines move them: a copy
// kernel (one launch for the whole list, reading and writing pinned host
// memory through its device mapping), or the DMA engines (one hipMemcpyAsync
// per run of consecutive ids and buffer; no compute units, but each call
// costs host time in the runtime).
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

// The copy kernel: workgroup w moves pages w, w + grid, ... of the batch
// (one page per workgroup by default, a few workgroups looping over the pages
// for the narrow engine), each lane moving 16-byte chunks of every paged
// buffer of a page, four in flight.  Pinned host memory is read and written
// directly through its device mapping, so one launch serves any list of
// pages.  The kernel holds few registers and no LDS.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxRuns = 160;
struct CopyRun {
  int32_t src, dst, count;
};
struct CopyArgs {
  const u32x4* src[5];
  u32x4* dst[5];
  uint32_t chunks[5];  // 16-byte chunks per page of each buffer
  int32_t nbuf, nruns;
  int32_t run_start[kMaxRuns + 1];  // first page (of the batch) of each run
  CopyRun runs[kMaxRuns];
};

__global__ __launch_bounds__(256) void copy_pages_kernel(CopyArgs a) {
  const int pages = a.run_start[a.nruns];
  int r = 0;
  for (int p = (int)blockIdx.x; p < pages; p += (int)gridDim.x) {  // page of the batch
    while (r + 1 < a.nruns && a.run_start[r + 1] <= p) ++r;  // uniform scan over at most kMaxRuns runs
    const int k = p - a.run_start[r];
    const size_t sp = (size_t)(a.runs[r].src + k), dp = (size_t)(a.runs[r].dst + k);
    for (int b = 0; b < a.nbuf; ++b) {
      const uint32_t c = a.chunks[b];
      const u32x4* s = a.src[b] + sp * c;
      u32x4* d = a.dst[b] + dp * c;
      uint32_t i = threadIdx.x;
      for (; i + 768 < c; i += 1024) {
        const u32x4 v0 = __builtin_nontemporal_load(s + i);
        const u32x4 v1 = __builtin_nontemporal_load(s + i + 256);
        const u32x4 v2 = __builtin_nontemporal_load(s + i + 512);
        const u32x4 v3 = __builtin_nontemporal_load(s + i + 768);
        __builtin_nontemporal_store(v0, d + i);
        __builtin_nontemporal_store(v1, d + i + 256);
        __builtin_nontemporal_store(v2, d + i + 512);
        __builtin_nontemporal_store(v3, d + i + 768);
      }
      for (; i < c; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
    }
  }
}

}  // namespace

extern "C" int kvq_copy_blocks(const kvq_cache* src, const kvq_cache* dst, const int32_t* src_blocks,
                               const int32_t* dst_blocks, int32_t n, int32_t engine, void* stream) {
  std::vector<PagedBuffer> bufs;
  int rc = paged_buffers(src, dst, &bufs);
  if (rc != KVQ_OK) return rc;
  if (n < 0) return KVQ_ERR_INVALID_ARG;
  if (n == 0) return KVQ_OK;
  if (!src_blocks || !dst_blocks) return KVQ_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (src_blocks[i] < 0 || src_blocks[i] >= src->num_blocks || dst_blocks[i] < 0 || dst_blocks[i] >= dst->num_blocks)
      return KVQ_ERR_INVALID_ARG;
  if (engine != KVQ_COPY_KERNEL && engine != KVQ_COPY_DMA && engine != KVQ_COPY_KERNEL_NARROW)
    return KVQ_ERR_INVALID_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return KVQ_ERR_NO_DEVICE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (engine == KVQ_COPY_KERNEL || engine == KVQ_COPY_KERNEL_NARROW) {
    for (const PagedBuffer& b : bufs)
      if ((b.page_bytes & 15) || (reinterpret_cast<uintptr_t>(b.src) & 15) || (reinterpret_cast<uintptr_t>(b.dst) & 15))
        return KVQ_ERR_INVALID_ARG;
    CopyArgs a{};
    a.nbuf = (int32_t)bufs.size();
    for (int b = 0; b < a.nbuf; ++b) {
      a.src[b] = reinterpret_cast<const u32x4*>(bufs[b].src);
      a.dst[b] = reinterpret_cast<u32x4*>(bufs[b].dst);
      a.chunks[b] = (uint32_t)(bufs[b].page_bytes / 16);
    }
    // runs of consecutive ids, launched kMaxRuns at a time
    int32_t i = 0;
    while (i < n) {
      a.nruns = 0;
      int32_t pages = 0;
      while (i < n && a.nruns < kMaxRuns) {
        int32_t j = i + 1;
        while (j < n && src_blocks[j] == src_blocks[j - 1] + 1 && dst_blocks[j] == dst_blocks[j - 1] + 1) ++j;
        a.run_start[a.nruns] = pages;
        a.runs[a.nruns] = CopyRun{src_blocks[i], dst_blocks[i], j - i};
        ++a.nruns;
        pages += j - i;
        i = j;
      }
      a.run_start[a.nruns] = pages;
      const int32_t grid = engine == KVQ_COPY_KERNEL_NARROW ? std::min(pages, (int32_t)KVQ_COPY_NARROW_WORKGROUPS) : pages;
      hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)grid), dim3(256), 0, st, a);
      if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
    }
    return KVQ_OK;
  }
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
