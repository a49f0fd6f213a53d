// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

// Unsigned division by a run-time constant d >= 1 with a precomputed
// multiplier (round-up method of Granlund and Montgomery, "Division by
// Invariant Integers using Multiplication", 1994): for n < 2^32,
// n / d == (umulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.s);
}

struct WriteArgs {
  const uint16_t* k;  // fp16 (T, H, D)
  const uint16_t* v;
  const int64_t* slots;
  const int32_t* seq_idx;
  int64_t T;
  int32_t H;
  int32_t bs;
  int64_t capacity;  // num_blocks * block_size
  FastDiv div_h;
  uint8_t* k_codes;
  uint16_t* k_scales;
  uint16_t* k_zeros;
  uint8_t* v_codes;
  uint16_t* v_scales;
  uint16_t* k_tail;
  uint16_t* v_tail;
  int32_t max_seqs;
};

struct DecodeArgs {
  const uint16_t* q;  // fp16 (B, Hq, D)
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int32_t max_blocks;
  int32_t B, Hq, H, G, bs, log2_bs, nb;
  float qscale;  // sm_scale * log2(e)
  const uint8_t* k_codes;
  const uint16_t* k_scales;
  const uint16_t* k_zeros;
  const uint8_t* v_codes;
  const uint16_t* v_scales;
  const uint16_t* k_tail;
  const uint16_t* v_tail;
  int32_t max_seqs;
  int32_t pages_per_split;
  int32_t num_splits;   // partial states per (sequence, query head), incl. the KIVI tail split
  int32_t quant_splits;  // splits over quantized pages
  float* part;  // (B, Hq, num_splits, D + 2) fp32: m, l, acc[D]
  uint16_t* out;  // fp16 (B, Hq, D)
};

// Launchers (return hipError_t of the launch).
hipError_t launch_write(const kvq_cache& c, const WriteArgs& a, hipStream_t s);
hipError_t launch_decode(const kvq_cache& c, const DecodeArgs& a, hipStream_t s);

// Context split used by decode for given sizes (shared by the workspace query).
int32_t choose_pages_per_split(const kvq_cache& c, int32_t batch, int32_t max_blocks, int32_t requested);

}  // namespace kvq
