/*
 * kvq: quantize-on-write into a paged KV cache and dequantizing paged decode
 * attention, for AMD Instinct MI355X (gfx950).
 *
 * The library stores keys and values of a transformer's KV cache as low-bit
 * codes plus fp16 scales in fixed-size pages, and runs single-query (decode)
 * attention and causal chunked-prefill attention that read those pages
 * through a block table and dequantize them in registers.  Sources, cited by page title and section:
 *   [P1] "Use Less Memory: Quantization and Offloading", section 2.1
 *        (symmetric quantization: s = max|x| / q_max, x_q = clip(round(x/s),
 *        -q_max, q_max), x_hat = x_q * s; q_max 127 for INT8, 7 for INT4),
 *        section 2.2 (per-token / per-head granularity), section 2.3 (FP8
 *        E4M3 and E5M2 layouts and ranges).
 *   [P2] "12 KV Cache Quantization", section 5: "Where the scales live"
 *        (k_cache (num_blocks, block_size, n_kv_heads, head_dim) in
 *        FP8/INT8/INT4, k_scale (num_blocks, block_size, n_kv_heads) in FP16;
 *        INT4 with one FP16 scale per 32 channels), "K is more sensitive than
 *        V" (softmax(q.k^T/sqrt(d)), sum_i p_i v_i; per-channel K, per-token V),
 *        "The kernel side" (the attention kernel dequantizes while reading).
 *   [P3] "Quantized KV caches in production: FP8 vs INT8 vs INT4", Numerical
 *        Formats (E4M3 1-4-3 and E5M2 1-5-2 layouts; KIVI per-channel keys /
 *        per-token values), Kernel Backends (dequantization on load; paged
 *        block allocator keeping scale metadata beside the page tables) and
 *        Implementation Best Practices (calibrated scaling factors).
 *   [P4] "KV Cache Quantization" glossary: asymmetric quantization (min and
 *        max onto the full integer range), PagedAttention, GQA.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them beyond the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it asynchronously; no entry point synchronizes
 *     except the diagnostics call kvq_get_device_error.
 *   - Return value: KVQ_OK (0) or a negative kvq_status.  Arguments are
 *     validated on the host before anything is launched; on error nothing is
 *     enqueued.  No C++ exception crosses this interface.
 *   - Device-side ids are bounds-checked by the kernels: a slot outside
 *     [0, num_blocks * block_size) is skipped by kvq_write, and a page whose
 *     block id is outside [0, num_blocks) contributes nothing to attention.
 *     Such ids (other than the negative slots that mean "skip") are also
 *     recorded in a per-device error word that kvq_get_device_error reads.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1,  /* NULL pointer, non-positive size, bad enum   */
  KVQ_ERR_UNSUPPORTED = -2,  /* format or head_dim not implemented          */
  KVQ_ERR_SHAPE = -3,        /* shape rule broken (see kvq_cache)           */
  KVQ_ERR_WORKSPACE = -4,    /* decode workspace NULL, too small, unaligned */
  KVQ_ERR_NO_DEVICE = -5,    /* no HIP device visible                       */
  KVQ_ERR_HIP = -6           /* a HIP runtime call or launch failed         */
} kvq_status;

/* Device-side data errors: bits of the word kvq_get_device_error returns.
 * The kernels still finish normally; the offending id is handled as stated. */
typedef enum kvq_device_error {
  KVQ_DEVERR_SLOT = 1,  /* kvq_write / kvq_write_static: a slot at or past
                           num_blocks * block_size (the token is skipped)   */
  KVQ_DEVERR_SEQ = 2,   /* kvq_write, KIVI keys: a seq_idx outside
                           [0, max_seqs) for a token with a valid slot (its
                           key is dropped: no tail row, no page completed)  */
  KVQ_DEVERR_BLOCK = 4, /* kvq_decode_attn: a block id outside
                           [0, num_blocks) on a page within the context (the
                           page contributes nothing)                        */
  KVQ_DEVERR_CTX = 8,   /* kvq_decode_attn / kvq_prefill_attn: a ctx_len
                           below 0 or above max_blocks_per_seq * block_size
                           (clamped)                                        */
  KVQ_DEVERR_QLEN = 16  /* kvq_prefill_attn: a chunk with q_start[b] < 0,
                           q_start[b + 1] > total_q, or a length below 0 or
                           above max_q_len (the sequence is skipped: its
                           output rows are not written)                     */
} kvq_device_error;

/* Storage formats of a cache tensor.
 * KVQ_INT8       symmetric, one fp16 scale per (token, head), q_max 127
 *                ([P1] 2.1, [P2] 5).  Codes int8 in [-127, 127].
 * KVQ_FP8_E4M3FN symmetric, one fp16 scale per (token, head); codes are OCP
 *                E4M3FN bytes (bias 7, max 448, no infinities), q_max 448,
 *                round-to-nearest-even, saturating.  ([P1] 2.3 prints +-240,
 *                the maximum of the FNUZ variant; gfx950 uses OCP E4M3FN.)
 * KVQ_INT4_G32   symmetric, one fp16 scale per 32 consecutive channels of a
 *                (token, head) row, q_max 7; two codes per byte, even channel
 *                in the low nibble, two's complement ([P2] 5).  Keys or
 *                values.
 * KVQ_INT4_KIVI  keys only: asymmetric per channel over the 32 tokens of a
 *                page ([P2] 5, [P3], [P4]); requires block_size == 32.  Per
 *                (page, head, channel): scale = fp16(fl32(max-min)/15), zero =
 *                min (fp16), codes 0..15 unsigned nibbles (even channel low).
 *                A page is quantized when its last row is written; until then
 *                its rows (keys AND values) are kept in fp16 in the
 *                sequence's tail.
 * KVQ_FP8_E5M2   symmetric, one fp16 scale per (token, head); codes are OCP
 *                E5M2 bytes (bias 15, max 57344; [P1] 2.3 table), q_max
 *                57344, round-to-nearest-even, saturating (never an infinity
 *                code).  The fp16 scale max|x|/57344 is an fp16 subnormal
 *                below max|x| = 3.5 and 0 below about 1.7e-3 (codes 0).
 * Every quotient x/s is the IEEE binary32 quotient by the STORED fp16 scale;
 * an fp16 scale of 0 stores all-zero codes. */
typedef enum kvq_dtype {
  KVQ_INT8 = 1,
  KVQ_FP8_E4M3FN = 2,
  KVQ_INT4_G32 = 3,
  KVQ_INT4_KIVI = 4,
  KVQ_FP8_E5M2 = 5
} kvq_dtype;

/* A paged, quantized KV cache for one attention layer.  All buffers are
 * caller-allocated device memory, contiguous, in these layouts (nb =
 * num_blocks, bs = block_size, H = n_kv_heads, D = head_dim):
 *   k_codes / v_codes  uint8 (nb, bs, H, D)    INT8, FP8 (E4M3FN, E5M2)
 *                      uint8 (nb, bs, H, D/2)  INT4_G32, INT4_KIVI
 *   k_scales/v_scales  fp16  (nb, bs, H)       INT8, FP8 (E4M3FN, E5M2)
 *                      fp16  (nb, bs, H, D/32) INT4_G32
 *                      fp16  (nb, H, D)        INT4_KIVI (k only)
 *   k_zeros            fp16  (nb, H, D)        INT4_KIVI only, else NULL
 *   k_tail / v_tail    fp16  (max_seqs, bs, H, D)  INT4_KIVI only, else NULL;
 *                      row r of a sequence's tail holds the fp16 key/value
 *                      of its not-yet-quantized page at offset r.
 * Token slot s (= block * bs + offset) of a page lives at [s / bs, s % bs].
 * Shape rules: head_dim in {64, 128, 256}; INT4_KIVI only for keys, with
 * block_size 32 and max_seqs > 0; values use INT8, FP8_E4M3FN, FP8_E5M2 or
 * INT4_G32. */
typedef struct kvq_cache {
  int32_t num_blocks;
  int32_t block_size;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t k_dtype; /* kvq_dtype */
  int32_t v_dtype; /* kvq_dtype */
  int32_t max_seqs;
  uint32_t flags;  /* kvq_cache_flags */
  void* k_codes;
  void* v_codes;
  void* k_scales;
  void* v_scales;
  void* k_zeros;
  void* k_tail;
  void* v_tail;
  /* Random signs of the Walsh-Hadamard rotation (KVQ_ROTATE_K / _V): bit c
   * (bit c % 32 of word c / 32) set means channel c is negated.  The same
   * signs serve keys and values; unused without a rotation flag. */
  uint32_t rot_signs[8];
} kvq_cache;

/* kvq_cache.flags.  Walsh-Hadamard rotation ([P3] Numerical Formats: QuaRot's
 * randomized orthogonal Walsh-Hadamard transforms spread outlier channels
 * before 4-bit quantization; Accuracy, Latency, and Serving Economics: INT4
 * after rotation stays close to unquantized quality).  A rotated tensor stores,
 * for each (token, head) row x, the row y = H (sigma * x) -- H the Sylvester
 * Hadamard matrix of order head_dim (entries +-1), sigma the signs of
 * rot_signs -- with every entry computed exactly and rounded once to fp32,
 * then quantized like an ordinary row (its scale absorbs the factor
 * sqrt(head_dim)).  Decode attends to x_hat = sigma * (H y_hat) / head_dim:
 * for rotated keys it scores the rotated query H (sigma * q) / head_dim
 * against the stored rows; for rotated values it rotates the weighted sum
 * back.  Symmetric formats only (KIVI keys: KVQ_ERR_UNSUPPORTED); KIVI fp16
 * tails keep the original rows. */
typedef enum kvq_cache_flags {
  KVQ_ROTATE_K = 1,
  KVQ_ROTATE_V = 2
} kvq_cache_flags;

/* Quantize-on-write ([P1] 2.1-2.2, [P2] 5 "Where the scales live").
 *   k, v          fp16 (num_tokens, H, D), row-major; read only.
 *   slot_mapping  int64 (num_tokens): destination slot of each token;
 *                 negative = skip the token.
 *   seq_idx       int32 (num_tokens): tail row (sequence) of each token;
 *                 required when k_dtype == KVQ_INT4_KIVI, else ignored.
 * For KVQ_INT4_KIVI the rows of one page must appear in the call in slot
 * order and consecutively (as a prefill chunk or one token per decode step
 * does); a page is quantized when the call holds its last row, taking its
 * earlier rows from this call or from the tail written by earlier calls.
 * num_tokens == 0 is a no-op; num_tokens * n_kv_heads must be below 2^31
 * (else KVQ_ERR_SHAPE).  Calls beyond 2^24 (token, head) rows are run as
 * consecutive launches over token ranges, with the same result as one. */
int kvq_write(const kvq_cache* cache, const void* k, const void* v,
              const int64_t* slot_mapping, const int32_t* seq_idx,
              int64_t num_tokens, void* stream);

/* Quantize-on-write with calibrated scales ([P3] Implementation Best
 * Practices: static per-head scaling factors computed before deployment;
 * [P4] static calibration): like kvq_write, but row (token, head h) is quantized with
 * the given scale instead of max|x| / q_max.
 *   k_scale, v_scale  fp16 (n_kv_heads) device arrays, caller-owned, read
 *                     only; a per-tensor scale is the same value H times.
 *                     Each scale must be positive and finite, or 0 (codes 0).
 * Quotients x / s beyond +-q_max saturate at +-q_max (the largest code of
 * the format).  Every written row stores its head's scale in its ordinary
 * scale slot (each group slot for INT4_G32), so kvq_decode_attn reads the
 * cache unchanged.  Symmetric formats only: KVQ_INT4_KIVI keys return
 * KVQ_ERR_UNSUPPORTED; NULL k_scale or v_scale returns KVQ_ERR_INVALID_ARG.
 * Other arguments, errors and asynchrony as for kvq_write. */
int kvq_write_static(const kvq_cache* cache, const void* k, const void* v,
                     const int64_t* slot_mapping, int64_t num_tokens,
                     const void* k_scale, const void* v_scale, void* stream);

/* Bytes of device workspace kvq_decode_attn needs for these sizes and this
 * split_tokens (see below): the work partition and the partial softmax
 * states of the pieces the context is cut into.  Depends only on the
 * arguments, not on the device or on ctx_lens.  KVQ_ERR_SHAPE if
 * max_blocks_per_seq * block_size reaches 2^30 tokens or the call's tile
 * count (batch x that / (32 / HP)) reaches 2^30, or n_q_heads is not a
 * multiple of n_kv_heads. */
int kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t batch,
                               int32_t n_q_heads, int32_t max_blocks_per_seq,
                               int32_t split_tokens, size_t* bytes);

/* Decode attention over the quantized pages ([P2] 5 "The kernel side";
 * "K is more sensitive than V": o = softmax(q k^T * sm_scale) V).
 *   q            fp16 (batch, n_q_heads, D)
 *   block_table  int32 (batch, max_blocks_per_seq): physical block of each
 *                page of each sequence; entries past the sequence's pages are
 *                never read.
 *   ctx_lens     int32 (batch): tokens of each sequence in the cache (0 gives
 *                an all-zero output row; values above max_blocks_per_seq *
 *                block_size are clamped to it).  For KVQ_INT4_KIVI keys the
 *                last ctx_len % 32 tokens are read from tail row b (the batch
 *                row).
 *   sm_scale     softmax scale; 0 means 1/sqrt(head_dim).
 *   split_tokens work partition.  One wave reads HP consecutive KV heads
 *                (HP = 4, 2 or 1: the most with HP x n_q_heads/n_kv_heads
 *                <= 16 that divides n_kv_heads), in
 *                tiles of 32 (token, head) rows = 32 / HP tokens.  The tiles
 *                of all sequences are numbered sequence after sequence and
 *                cut into equal shares, each read by n_kv_heads / HP waves
 *                (a share may end in one sequence and go on in the next).
 *                0 = automatic: as many shares as fill the GPU's resident
 *                waves once (at least 4 tiles each); > 0 = shares of
 *                ceil(split_tokens / (32 / HP)) tiles.
 *   out          fp16 (batch, n_q_heads, D), written.
 *   workspace    device scratch of at least kvq_decode_workspace_bytes()
 *                for the same arguments, 16-byte aligned; its contents on
 *                entry do not matter.
 * Query head hq reads KV head hq / (n_q_heads / n_kv_heads) ([P4] GQA).
 * Scores and the softmax are accumulated in fp32; the result is rounded to
 * fp16 once, to nearest-even.  The result does not depend on the partition
 * except through fp32 rounding, and a given partition gives bitwise the same
 * result on every call. */
int kvq_decode_attn(const kvq_cache* cache, const void* q,
                    const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* ctx_lens, int32_t batch, int32_t n_q_heads,
                    float sm_scale, int32_t split_tokens, void* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Decode attention with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * kvq_decode_attn without `workspace` / `workspace_bytes`: the workspace is a
 * fixed per-device array of KVQ_NOALLOC_WORKSPACE_BYTES inside the library,
 * which every GPU the library runs on holds from the library's load until the
 * process ends.  This call allocates and frees nothing.
 * KVQ_ERR_WORKSPACE if kvq_decode_workspace_bytes() for these arguments
 * exceeds KVQ_NOALLOC_WORKSPACE_BYTES (use a larger split_tokens, or
 * kvq_decode_attn).  The array is shared by every call on the device and
 * keeps the last call's contents (which the kernels never read before they
 * write them): calls that overlap on one GPU, on different streams or from
 * different threads, race and must not be issued. */
#define KVQ_NOALLOC_WORKSPACE_BYTES (64u << 20)
int kvq_decode_attn_noalloc(const kvq_cache* cache, const void* q,
                            const int32_t* block_table,
                            int32_t max_blocks_per_seq,
                            const int32_t* ctx_lens, int32_t batch,
                            int32_t n_q_heads, float sm_scale,
                            int32_t split_tokens, void* out, void* stream);

/* Workspace bytes of kvq_prefill_attn for a chunk batch of total_q query
 * rows: 0 unless the cache stores rotated keys (KVQ_ROTATE_K), which need the
 * rotated queries, 2 x total_q x n_q_heads x head_dim fp16 values. */
int kvq_prefill_workspace_bytes(const kvq_cache* cache, int64_t total_q,
                                int32_t n_q_heads, size_t* bytes);

/* Causal chunked-prefill attention over the quantized pages ("Use Less
 * Memory: Quantization and Offloading", What Comes Next: a long prompt is
 * processed in scheduled pieces; "12 KV Cache Quantization", Interaction
 * with prefix caching: the pieces attend to quantized blocks already cached).
 * Each sequence b brings a chunk of n_b = q_start[b + 1] - q_start[b]
 * queries, its last n_b positions: their keys and values must already be in
 * the cache (kvq_write before this call).  Query i of the chunk sits at
 * position p = L_b - n_b + i and attends to tokens 0..p,
 * o = softmax(q k_hat^T * sm_scale) V_hat, where L_b is ctx_lens[b] taken
 * into [0, max_blocks_per_seq * block_size].  A query at p < 0 (a chunk
 * longer than the context) gets an all-zero row.
 *   q            fp16 (total_q, n_q_heads, D): the chunks one after another
 *   q_start      int32 (batch + 1), non-decreasing, q_start[0] >= 0,
 *                q_start[batch] <= total_q
 *   block_table, max_blocks_per_seq, ctx_lens, sm_scale: as kvq_decode_attn
 *                (KVQ_INT4_KIVI keys: sequence b's last L_b % 32 tokens are
 *                read from tail row b)
 *   max_q_len    an upper bound on every n_b (it sizes the grid); a longer
 *                chunk is skipped and recorded as KVQ_DEVERR_QLEN
 *   out          fp16 (total_q, n_q_heads, D), 16-byte aligned: rows of the
 *                chunks are written, other rows are left as they are
 *   workspace    at least kvq_prefill_workspace_bytes() (may be NULL when
 *                that is 0), 16-byte aligned
 * Query head hq reads KV head hq / (n_q_heads / n_kv_heads) ([P4] GQA).
 * Scores and the softmax are accumulated in fp32 and the result is rounded
 * to fp16 once; a given call gives bitwise the same result every time.
 * KVQ_ERR_SHAPE when total_q x n_q_heads x head_dim reaches 2^31 or
 * max_q_len x n_q_heads / n_kv_heads reaches 2^30. */
int kvq_prefill_attn(const kvq_cache* cache, const void* q,
                     const int32_t* q_start, const int32_t* block_table,
                     int32_t max_blocks_per_seq, const int32_t* ctx_lens,
                     int32_t batch, int64_t total_q, int32_t n_q_heads,
                     int32_t max_q_len, float sm_scale, void* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Copy whole pages between two caches of the same geometry and formats
 * (block_size, n_kv_heads, head_dim, k_dtype, v_dtype; num_blocks may
 * differ): page dst_blocks[i] of `dst` becomes a byte copy of page
 * src_blocks[i] of `src`, for i < n ("Use Less Memory: Quantization and
 * Offloading", section 4: quantized blocks offloaded to CPU RAM and
 * prefetched into a second set of GPU buffers for the next step while the
 * current one computes).  Either cache may live in device memory or in
 * pinned host memory (hipHostMalloc; the per-page layout is the same), so
 * the call offloads (device -> host), prefetches (host -> device) or moves
 * pages on the device.  A page is its codes, scales and (KIVI keys) zero
 * points; the per-sequence KIVI tails are not paged and are not copied.
 *   src_blocks, dst_blocks  int32 HOST arrays of n block ids, read during the
 *                           call only; ids outside [0, num_blocks) of their
 *                           cache give KVQ_ERR_INVALID_ARG before any copy.
 * The copies are enqueued on `stream` by the chosen engine (below); runs of
 * consecutive source and destination ids are merged.  The copy kernel needs
 * pinned (device-mapped) host memory and 16-byte aligned buffers
 * (KVQ_ERR_INVALID_ARG otherwise); with DMA, pageable host memory is
 * correct but not asynchronous.
 * Destination pages listed twice, or pages that are both read and written by
 * the call, give an unspecified result.  KVQ_ERR_SHAPE if the geometries or
 * formats differ; KVQ_ERR_INVALID_ARG for a NULL buffer the formats need. */
typedef enum kvq_copy_engine {
  KVQ_COPY_KERNEL = 0,        /* one copy-kernel launch for the whole list
                                 (pinned host memory through its device
                                 mapping), one workgroup of 256 lanes per page */
  KVQ_COPY_DMA = 1,           /* hipMemcpyAsync per run of consecutive ids and
                                 buffer: no compute units, more host time per
                                 call */
  KVQ_COPY_KERNEL_NARROW = 2  /* the copy kernel on at most
                                 KVQ_COPY_NARROW_WORKGROUPS workgroups of 256
                                 lanes, each looping over pages: it holds at
                                 most 4 x that many wave slots, so a decode
                                 launched beside it with that many slots left
                                 free (split_tokens) runs concurrently; a few
                                 workgroups already saturate the host link */
} kvq_copy_engine;
#define KVQ_COPY_NARROW_WORKGROUPS 16
int kvq_copy_blocks(const kvq_cache* src, const kvq_cache* dst,
                    const int32_t* src_blocks, const int32_t* dst_blocks,
                    int32_t n, int32_t engine, void* stream);

/* Static description of a status code (never NULL). */
const char* kvq_status_string(int status);

/* Diagnostics (the failure-detection side of the boundary): returns the
 * kvq_device_error bits recorded on the current device since the previous
 * call (0 if none), and clears them.  The read is ordered after the work
 * already enqueued on `stream` (NULL = the default stream), and this call
 * synchronizes that stream: it is meant for tests and debugging, not for the
 * hot loop.  Kernels on other streams record into the same per-device word;
 * calls that overlap with them may report their bits here or in the next
 * call.  Negative kvq_status on failure (KVQ_ERR_NO_DEVICE, KVQ_ERR_HIP). */
int kvq_get_device_error(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
