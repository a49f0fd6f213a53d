// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"
#include "kvq_fastdiv.h"

namespace kvq {

// n / f.d on the device (see kvq_fastdiv.h)
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
  int32_t seal_chunk;  // KIVI: call tokens per seal wave (32, or 1 for small calls)
  // Calibrated scales, fp16 per KV head, used instead of max|x| / q_max
  // (kvq_write_static); NULL for the dynamic per-token scale.
  const uint16_t* k_static;
  const uint16_t* v_static;
  uint32_t* err;  // per-device kvq_device_error word
  // Walsh-Hadamard rotation of keys / values (kvq_cache_flags) and its signs
  int32_t rot_k, rot_v;
  uint32_t rot_signs[8];
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
  // A wave handles HP = 2^hp_log2 consecutive KV heads; a tile is 32 rows,
  // (token, head) pairs: 32 / HP tokens of those HP heads.
  int32_t hp_log2;
  // Work partition.  The tiles of all sequences are numbered sequence by
  // sequence; share i covers tiles [i S, (i + 1) S) and is processed by
  // n_kv_heads / HP waves, one per group of HP KV heads.
  int32_t share_tiles;  // S requested by the caller; 0 = balanced over num_shares
  int32_t inline_plan;  // B <= 64: the kernels derive the plan from ctx_lens themselves
  int32_t num_shares;   // shares launched (<= max_shares)
  int32_t max_shares;   // shares the workspace was laid out for
  // Workspace: plan ints, then the partial softmax records.
  //   plan[0]              S used by this call
  //   plan[1 + b]          first tile of sequence b (b = 0..B; plan[1 + B] = all tiles)
  //   plan[2 + B + i]      sequence holding the first tile of share i
  int32_t* plan;
  // Record r, query head hq: part[(r Hq + hq) (D + 2) ...] = m, l, acc[D] (fp32).
  // Records: share i's piece of sequence b -> i + b.
  float* part;
  uint16_t* out;  // fp16 (B, Hq, D)
  uint32_t* err;  // per-device kvq_device_error word (checked by the merge kernel)
  // Walsh-Hadamard rotation (kvq_cache_flags): rotated keys are scored
  // against the rotated query q' = H (sigma q) / D, held in the workspace as
  // fp16 hi (B, Hq, D) then lo (B, Hq, D) with hi + lo = q' (to fp32
  // accuracy); rotated values are rotated back by the merge.
  int32_t rot_k, rot_v;
  uint32_t rot_signs[8];
  uint16_t* qrot;
};

struct PrefillArgs {
  const uint16_t* q;        // fp16 (Tq, Hq, D): the chunks of all sequences
  const uint16_t* qrot;     // rotated keys: q' as fp16 hi (Tq, Hq, D) then lo
  const int32_t* q_start;   // (B + 1): sequence b's queries are rows q_start[b] .. q_start[b + 1] - 1
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int64_t Tq;               // rows of q and out
  int32_t max_blocks;
  int32_t B, Hq, H, G, bs, log2_bs, nb;
  int32_t max_q_len;        // largest chunk the grid covers
  int32_t n_qtiles;         // query tiles per (sequence, KV head)
  int32_t n_wg;             // workgroups with work: B H n_qtiles
  float qscale;             // sm_scale * log2(e)
  const uint8_t* k_codes;
  const uint16_t* k_scales;
  const uint16_t* k_zeros;
  const uint8_t* v_codes;
  const uint16_t* v_scales;
  const uint16_t* k_tail;
  const uint16_t* v_tail;
  int32_t max_seqs;
  uint16_t* out;            // fp16 (Tq, Hq, D)
  uint32_t* err;            // per-device kvq_device_error word
  int32_t rot_k, rot_v;
  uint32_t rot_signs[8];
};

// Workspace layout of one decode call (host side, no device needed).
struct DecodePlan {
  int32_t share_tiles;   // requested S (0 = balanced)
  int32_t max_shares;    // upper bound on the shares any launch of this call uses
  size_t plan_bytes;     // plan ints, rounded up to 256 bytes
  size_t records;        // partial records
  size_t qrot_offset;    // rotated query (rotated keys only), 256-byte aligned
  size_t bytes;          // total workspace
};
// Returns false if the sizes overflow the ranges the kernels index with.
bool plan_decode(const kvq_cache& c, int32_t batch, int32_t n_q_heads, int32_t max_blocks, int32_t split_tokens,
                 DecodePlan* plan);

// log2 of the KV heads one decode wave handles for G query heads per KV head.
int32_t heads_per_wave_log2(const kvq_cache& c, int32_t G);

// Launchers (return hipError_t of the launch).
hipError_t launch_write(const kvq_cache& c, const WriteArgs& a, hipStream_t s);
hipError_t launch_decode(const kvq_cache& c, const DecodeArgs& a, hipStream_t s);
// Per key format (kvq_decode_k*.hip): fv value format, D head dim.
hipError_t decode_keys_int8(int fv, int D, const DecodeArgs& a, hipStream_t s);
hipError_t decode_keys_fp8(int fv, int D, const DecodeArgs& a, hipStream_t s);
hipError_t decode_keys_kivi(int fv, int D, const DecodeArgs& a, hipStream_t s);
hipError_t decode_keys_e5m2(int fv, int D, const DecodeArgs& a, hipStream_t s);
hipError_t decode_keys_int4(int fv, int D, const DecodeArgs& a, hipStream_t s);
// rotated keys (the query operand is the rotated query, fp16 hi + lo)
hipError_t decode_keys_int8_rot(int fv, int D, const DecodeArgs& a, hipStream_t s);
hipError_t decode_keys_fp8_rot(int fv, int D, const DecodeArgs& a, hipStream_t s);
hipError_t decode_keys_e5m2_rot(int fv, int D, const DecodeArgs& a, hipStream_t s);
hipError_t decode_keys_int4_rot(int fv, int D, const DecodeArgs& a, hipStream_t s);

// The rotated query q' = H (sigma q) / D of `rows` fp16 rows of head_dim D,
// written as fp16 hi (rows, D) at qrot and lo (rows, D) right after it.
hipError_t launch_rotate_query(const uint16_t* q, uint16_t* qrot, size_t rows, int D, const uint32_t* signs,
                               hipStream_t s);

// Chunked-prefill attention (kvq_prefill*.hip).
hipError_t launch_prefill(const kvq_cache& c, const PrefillArgs& a, hipStream_t s);
hipError_t prefill_keys_int8(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s);
hipError_t prefill_keys_fp8(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s);
hipError_t prefill_keys_kivi(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s);
hipError_t prefill_keys_e5m2(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s);
hipError_t prefill_keys_int4(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s);


}  // namespace kvq
