// Dequantizing paged decode attention (gfx950).
//
// What is computed ("12 KV Cache Quantization", section 5, "K is more
// sensitive than V" and "The kernel side"): for each sequence b and query head
// hq, o = softmax(q k_hat^T * sm_scale) V_hat over the ctx_lens[b] cached
// tokens, where k_hat, v_hat are dequantized from the pages while they are
// read, and query head hq reads KV head hq / G (KV Cache Quantization
// glossary, GQA).
//
// How (MI355X design, not the pages' Hopper kernels):
//  * Split-K over the context: a workgroup owns (context split, up to 8 KV
//    heads, sequence); wave w handles one KV head and all G query heads that
//    read it.  Splits are whole pages, so ragged batches stay balanced; a
//    second kernel merges the per-split softmax states.
//  * Tiles of 32 tokens.  Scores S^T = K Q^T run on the matrix cores
//    (v_mfma_f32_16x16x32_f16): the 8-bit/4-bit key codes become exact fp16
//    operands (q is fp16 already), so the products are exact and only the
//    fp32 accumulation rounds; the per-token key scale is applied to the
//    fp32 score afterwards (q.k_hat = s_k (q.codes)).
//  * Values: the tile's value pages are staged in LDS and read back with the
//    8-bit transpose read (ds_read_b64_tr_b8), which hands each lane one
//    channel (INT8/FP8) or one channel pair (INT4) of 8 tokens, the layout
//    the matrix core wants for P V.  Value codes become exact bf16 operands;
//    the probabilities times the per-token value scale are split into two
//    bf16 terms (hi + lo, relative error <= 2^-18), so P V costs two MFMAs per
//    16 channels and keeps fp32-level accuracy.
//  * Online softmax in the log2 domain (q pre-multiplied by sm_scale*log2 e),
//    fp32 throughout; each split stores (m, l, acc[D]).
#include <math.h>

#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef int i2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i2 lds_i2;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int TILE = 32;      // tokens per tile
constexpr int MAX_WAVES = 8;  // KV heads per workgroup
constexpr int MAX_PPS = 256;  // pages per split (block-table slice in LDS)

template <int FK, int D>
struct KShape {
  static constexpr int RB = FK == F_KIVI ? D / 2 : D;  // key row bytes
  static constexpr int LB = RB / 4;                    // bytes per lane (quarter row)
  static constexpr int NW = LB / 4;                    // dwords per lane
  static constexpr int KB = D / 32;                    // MFMA k-blocks
};

template <int FV, int D>
struct VShape {
  static constexpr int RB = FV == F_INT4 ? D / 2 : D;  // value row bytes
  static constexpr int RBP = RB + 16;                  // LDS row pitch
  static constexpr int CH = RB / 16;                   // 16-byte chunks per row
  static constexpr int NL = TILE * CH / 64;            // chunks staged per lane
  static constexpr int NG = FV == F_INT4 ? D / 32 : 1; // scales per row
  static constexpr int NPV = D / 16;                   // P.V MFMAs (16 channels each)
};

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// ---- key operands: 8 exact fp16 values of the k-block's 8 channels ----------
// INT8: (1024 + (c + 128)) - 1152 = c, exactly, in fp16.
__device__ __forceinline__ void int8_to_h4(uint32_t d, uint32_t& lo, uint32_t& hi) {
  d ^= 0x80808080u;
  // v_perm_b32: bytes [c0, 0x64, c1, 0x64] and [c2, 0x64, c3, 0x64]
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, d, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, d, 0x04030402u);
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = h2_bits(as_h2(a) - bias);
  hi = h2_bits(as_h2(b) - bias);
}
// FP8 E4M3FN -> fp16, two codes per instruction (exact: every E4M3FN value
// is an fp16 value; the scale operand 1.0 leaves the values unchanged).
__device__ __forceinline__ void fp8_to_h4(uint32_t d, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true));
}

template <int FK>
__device__ __forceinline__ h8 key_operand(const uint32_t* w, int kb) {
  u4 r;
  if constexpr (FK == F_KIVI) {
    // 8 unsigned nibbles of one dword; pair i = channels (i, i + 4):
    // (1024 + n) - 1024 = n exactly.
    const uint32_t d = w[kb];
    const h2 bias = {(_Float16)1024.0f, (_Float16)1024.0f};
    r.x = h2_bits(as_h2((d & 0x000F000Fu) | 0x64006400u) - bias);
    r.y = h2_bits(as_h2(((d >> 4) & 0x000F000Fu) | 0x64006400u) - bias);
    r.z = h2_bits(as_h2(((d >> 8) & 0x000F000Fu) | 0x64006400u) - bias);
    r.w = h2_bits(as_h2(((d >> 12) & 0x000F000Fu) | 0x64006400u) - bias);
  } else {
    uint32_t x0, x1, x2, x3;
    if constexpr (FK == F_FP8) {
      fp8_to_h4(w[2 * kb], x0, x1);
      fp8_to_h4(w[2 * kb + 1], x2, x3);
    } else {
      int8_to_h4(w[2 * kb], x0, x1);
      int8_to_h4(w[2 * kb + 1], x2, x3);
    }
    r = u4{x0, x1, x2, x3};
  }
  return __builtin_bit_cast(h8, r);
}

// Channel held in k-slot e of k-block kb by lane group j (the key operand
// order; the query operand is laid out to match).
template <int FK, int D>
__device__ __forceinline__ int key_channel(int j, int kb, int e) {
  const int base = j * (D / 4) + 8 * kb;
  if constexpr (FK == F_KIVI) return base + ((e & 1) ? 4 + (e >> 1) : (e >> 1));
  return base + e;
}

// ---- value operands: 8 exact bf16 values, 8 tokens of one channel ----------
// INT8: bf16(c + 128) (exact, <= 255); the +128 is removed afterwards with
// the sum of the probabilities.  FP8: exact.  INT4: 128 + (n + 8) (exact).
__device__ __forceinline__ uint32_t bf16_pair_hi(float a, float b) {
  // upper halves of a (low word) and b (high word): one v_perm_b32
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x07060302u);
}

template <int FV>
__device__ __forceinline__ b8 value_operand_8bit(i2 t) {
  const uint32_t d0 = (uint32_t)t.x, d1 = (uint32_t)t.y;
  u4 r;
  if constexpr (FV == F_FP8) {
    // FP8 E4M3FN -> bf16, two codes per instruction (exact)
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
  } else {
    const uint32_t e0 = d0 ^ 0x80808080u, e1 = d1 ^ 0x80808080u;
    // (float)((x >> 8k) & 0xFF) is one v_cvt_f32_ubyte{k}
    r.x = bf16_pair_hi((float)(e0 & 0xFFu), (float)((e0 >> 8) & 0xFFu));
    r.y = bf16_pair_hi((float)((e0 >> 16) & 0xFFu), (float)(e0 >> 24));
    r.z = bf16_pair_hi((float)(e1 & 0xFFu), (float)((e1 >> 8) & 0xFFu));
    r.w = bf16_pair_hi((float)((e1 >> 16) & 0xFFu), (float)(e1 >> 24));
  }
  return __builtin_bit_cast(b8, r);
}

// INT4: 8 bytes = 8 tokens of a channel pair; element order of both operands
// is tokens [0, 2, 1, 3, 4, 6, 5, 7].
__device__ __forceinline__ void value_operand_int4(i2 t, b8& even, b8& odd) {
  const uint32_t d0 = (uint32_t)t.x ^ 0x88888888u, d1 = (uint32_t)t.y ^ 0x88888888u;
  const uint32_t m = 0x000F000Fu, o = 0x43004300u;
  u4 e, od;
  e.x = (d0 & m) | o;
  e.y = ((d0 >> 8) & m) | o;
  e.z = (d1 & m) | o;
  e.w = ((d1 >> 8) & m) | o;
  od.x = ((d0 >> 4) & m) | o;
  od.y = ((d0 >> 12) & m) | o;
  od.z = ((d1 >> 4) & m) | o;
  od.w = ((d1 >> 12) & m) | o;
  even = __builtin_bit_cast(b8, e);
  odd = __builtin_bit_cast(b8, od);
}

// x = hi + lo with hi = bf16_rne(x), lo = bf16_rne(x - hi), two values at a
// time (v_cvt_pk_bf16_f32); `used` is what the operands hold, hi + lo.
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16x2(f2 x, uint32_t& hi, uint32_t& lo, f2& used) {
  const bf2 h = __builtin_convertvector(x, bf2);
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const f2 fh = {__builtin_bit_cast(float, hb << 16), __builtin_bit_cast(float, hb & 0xFFFF0000u)};
  const bf2 l = __builtin_convertvector(x - fh, bf2);
  const uint32_t lb = __builtin_bit_cast(uint32_t, l);
  hi = hb;
  lo = lb;
  used = fh + f2{__builtin_bit_cast(float, lb << 16), __builtin_bit_cast(float, lb & 0xFFFF0000u)};
}

// Flat row index (slot * H + h) of token t0 + t and whether it is live: in the
// context and on a page whose block id is valid.  The block id comes from
// the split's block-table slice in LDS (s_blk[page - p0]).
__device__ __forceinline__ uint32_t tile_row(const DecodeArgs& a, const int32_t* s_blk, int p0, int t, int t0,
                                             int tok_end, int h, bool& live) {
  const int tt = t0 + t;
  const int lbs = a.log2_bs;
  const int pg = tt >> lbs;
  const bool in = tt < tok_end;
  const int bid = in ? s_blk[pg - p0] : 0;
  live = in && bid >= 0 && bid < a.nb;
  const uint32_t blk = live ? (uint32_t)bid : 0u;
  return ((blk << lbs) + (uint32_t)(tt & ((1 << lbs) - 1))) * (uint32_t)a.H + (uint32_t)h;
}

// ---- asynchronous copies global -> LDS ----------------------------------
// global_load_lds_dword{,x4}: lane l of the instruction writes its 4 (16)
// bytes at LDS address m0 + 4 l (16 l).  The loop below issues every global
// read of a tile this way, so nothing it waits on lives in registers; the
// compiler does not track these transfers, so the loop waits for them with
// explicit s_waitcnt vmcnt(N) (loads complete in issue order).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds_addr), "v"(src) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" : : "s"(lds_addr), "v"(src) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Swizzles of the 16-byte chunks of a tile row in LDS: chunk (row, col)
// sits in slot row * CH + (col ^ swz(row)), so the rows one read instruction
// touches fall in distinct bank groups.  Values are read with the 8-bit
// transpose read (rows T_j), keys with 16-byte reads (16 consecutive rows).
template <int CH>
__device__ __forceinline__ int vswz(int row) {
  return ((row & 3) | (((row >> 4) & 1) << 2)) & (CH - 1);
}
template <int CH>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (CH >= 8) return row & 7;
  else if constexpr (CH == 4) return (row >> 1) & 3;
  else return (row >> 2) & 1;
}

template <int FK, int FV, int D>
struct Stage {
  using KS = KShape<FK, D>;
  using VS = VShape<FV, D>;
  static constexpr int KT = TILE * KS::RB;          // key tile bytes
  static constexpr int VT = TILE * VS::RB;          // value tile bytes
  static constexpr int NLK = KT / 1024;             // 16-byte key chunks per lane (>= 1)
  static constexpr int NLV = VT / 1024;
  static constexpr int NGD = VS::NG > 1 ? VS::NG / 2 : 1;  // value-scale dwords per token
  static constexpr int KIVI_BYTES = FK == F_KIVI ? 2 * D * 2 : 0;  // page scale + zero (fp16)
  // byte offsets inside a stage
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = KT;
  static constexpr int OFF_S = KT + VT;              // raw scale dwords (see issue_tile)
  static constexpr int OFF_M = OFF_S + 4 * TILE * (1 + NGD);
  static constexpr int BYTES = OFF_M + KIVI_BYTES;
  // DMA instructions per tile: keys, values, scales, KIVI page metadata
  static constexpr int NDMA = NLK + NLV + NGD + (FK == F_KIVI ? 1 : 0);
};

// Start the copy of one tile (keys, values, per-token scale dwords; KIVI
// page scale/zero) into LDS stage `st`; returns the live-token mask (bit t
// and t + 32: token t0 + t is in the context on a valid page).  Masked rows
// copy from the start of the buffer; those bytes are never used unmasked.
template <int FK, int FV, int D>
__device__ __forceinline__ uint64_t issue_tile(const DecodeArgs& a, const int32_t* s_blk, int p0, int t0, int tok_end,
                                               int h, uint8_t* st) {
  using S = Stage<FK, FV, D>;
  using KS = KShape<FK, D>;
  using VS = VShape<FV, D>;
  constexpr int CHK = KS::RB / 16 > 0 ? KS::RB / 16 : 1;
  const int lane = (int)threadIdx.x;
  const uint32_t base = lds_addr(st);
  // row index of token `lane & 31`, or ~0 when masked; shared with shuffles
  bool live;
  const uint32_t r_own = tile_row(a, s_blk, p0, lane & 31, t0, tok_end, h, live);
  const uint64_t live_mask = __ballot(live);
  const uint32_t rl = live ? r_own : ~0u;
#pragma unroll
  for (int i = 0; i < S::NLK; ++i) {
    const int p = 64 * i + lane;  // LDS slot of this lane
    const int row = p / CHK;
    const int col = (p % CHK) ^ kswz<CHK>(row);
    const uint32_t r = (uint32_t)__shfl((int)rl, row);
    dma16(a.k_codes + (r != ~0u ? (size_t)r * KS::RB + col * 16 : 0), base + S::OFF_K + 1024 * i);
  }
#pragma unroll
  for (int i = 0; i < S::NLV; ++i) {
    const int p = 64 * i + lane;
    const int row = p / VS::CH;
    const int col = (p % VS::CH) ^ vswz<VS::CH>(row);
    const uint32_t r = (uint32_t)__shfl((int)rl, row);
    dma16(a.v_codes + (r != ~0u ? (size_t)r * VS::RB + col * 16 : 0), base + S::OFF_V + 1024 * i);
  }
  // scale dwords (LDS dword index): [t] the dword holding token t's key
  // scale, [32 + t] the first value-scale dword of token t, [32 + 32 k + t]
  // its value-scale dword k >= 1 (INT4 groups)
  {
    const uint16_t* src;
    if (lane < 32) src = FK == F_KIVI ? a.v_scales : a.k_scales + (live ? (r_own & ~1u) : 0);
    else src = a.v_scales + (live ? ((size_t)r_own * VS::NG & ~(size_t)1) : 0);
    dma4(src, base + S::OFF_S);
  }
#pragma unroll
  for (int g = 1; g < S::NGD; ++g) {
    if (lane < 32) dma4(a.v_scales + (live ? (size_t)r_own * VS::NG + 2 * g : 0), base + S::OFF_S + 128 + 128 * g);
  }
  if constexpr (FK == F_KIVI) {
    // the tile is one page (block_size 32): its D scales and D zeros
    constexpr int CH = D * 2 / 16;
    const uint32_t r0 = (uint32_t)__shfl((int)rl, 0);
    const bool ok = r0 != ~0u;
    const size_t mrow = ((size_t)(r0 / (32u * (uint32_t)a.H)) * a.H + h) * D;
    if (lane < 2 * CH) {
      const uint16_t* src = (lane < CH ? a.k_scales : a.k_zeros) + (ok ? mrow + 8 * (lane % CH) : 0);
      dma16(src, base + S::OFF_M);
    }
  }
  return live_mask;
}

template <int FK, int FV, int D>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using KS = KShape<FK, D>;
  using VS = VShape<FV, D>;
  using ST = Stage<FK, FV, D>;
  constexpr int CHK = KS::RB / 16 > 0 ? KS::RB / 16 : 1;
  constexpr int NCS = FV == F_INT4 ? VS::NG : 1;  // bias-correction sums kept per value group
  __shared__ int32_t s_blk[MAX_PPS];
  // three stages: tile i is computed while tiles i+1 and i+2 are in flight
  __shared__ __attribute__((aligned(16))) uint8_t s_st[3][ST::BYTES];
  // this tile's scales as fp32: key scale x sm_scale x log2 e, value scales
  __shared__ __attribute__((aligned(16))) float s_fk[TILE];
  __shared__ __attribute__((aligned(16))) float s_fv[TILE * VS::NG];

  // Work unit (sequence, split, KV head); the KV heads of one (sequence,
  // split) are consecutive workgroups of one XCD (workgroups are dealt to the
  // 8 XCDs round robin), so they share the L2 lines of the page scales.
  const uint32_t wg = blockIdx.x;
  const uint32_t kk = wg >> 3;
  const int h = (int)(kk % (uint32_t)a.H);
  const uint32_t unit = (kk / (uint32_t)a.H) * 8 + (wg & 7);
  if (unit >= (uint32_t)(a.B * a.quant_splits)) return;
  const int b = (int)(unit / (uint32_t)a.quant_splits), split = (int)(unit % (uint32_t)a.quant_splits);

  const int lane = (int)threadIdx.x;
  const int j = lane >> 4, n = lane & 15;
  const int bs = 1 << a.log2_bs;
  // ctx_len is clamped to what the block-table row can address
  const int L = min(max(a.ctx_lens[b], 0), a.max_blocks * bs);
  const int Lq = FK == F_KIVI ? (L & ~31) : L;  // tokens held in quantized pages
  const int npages = (Lq + bs - 1) >> a.log2_bs;
  const int p0 = split * a.pages_per_split;
  const int p1 = min(npages, p0 + a.pages_per_split);
  for (int i = lane; i < p1 - p0; i += 64) s_blk[i] = a.block_table[(size_t)b * a.max_blocks + p0 + i];

  const int G = a.G;
  const int hq0 = h * G;
  f4 acc[VS::NPV];
#pragma unroll
  for (int m = 0; m < VS::NPV; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  float cs_run[NCS];  // sum of the probability operands (hi + lo) of query head n, per value group
#pragma unroll
  for (int g = 0; g < NCS; ++g) cs_run[g] = 0.f;

  // Query operand (B of S^T = K Q^T): lane (j, n) holds query head n's
  // channels of k-slots 8j..8j+7 in the key operand's channel order.
  const uint16_t* qrow = a.q + ((size_t)b * a.Hq + hq0 + (n < G ? n : 0)) * D;
  h8 qop[KS::KB];
#pragma unroll
  for (int kb = 0; kb < KS::KB; ++kb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t bits = qrow[key_channel<FK, D>(j, kb, e)];
      qop[kb][e] = __builtin_bit_cast(_Float16, (uint16_t)(n < G ? bits : 0));
    }
  }
  // the half of a scale dword holding this (token, head)'s scale is
  // (row index) & 1: h & 1 for an even head count, (t + h) & 1 otherwise
  const bool h_odd = (a.H & 1) != 0;

  // Value transpose reads: lane (j, i) points at row T_j[i / 2] of the value
  // tile, byte 8 (i % 2) of the chunk, where T_j[e] = 16 (e / 4) + 4 j + e % 4
  // is the token of k-slot e of lane group j.
  const int trow = 16 * ((n >> 1) >> 2) + 4 * j + ((n >> 1) & 3);
  const int tbase = ST::OFF_V + trow * VS::RB + 8 * (n & 1);
  const int tswz = vswz<VS::CH>(trow);

  const int tok_begin = p0 * bs, tok_end = min(Lq, p1 * bs);
  const int ntiles = tok_end > tok_begin ? (tok_end - tok_begin + TILE - 1) / TILE : 0;
  __syncthreads();  // s_blk written before it is read below
  uint64_t live[3] = {0, 0, 0};
  if (ntiles > 0) live[0] = issue_tile<FK, FV, D>(a, s_blk, p0, tok_begin, tok_end, h, s_st[0]);
  if (ntiles > 1) live[1] = issue_tile<FK, FV, D>(a, s_blk, p0, tok_begin + TILE, tok_end, h, s_st[1]);

  int it = 0;
  // One tile; S is the LDS stage holding it.
  auto step = [&](auto stage) -> bool {
    constexpr int S = decltype(stage)::value;
    if (it >= ntiles) return false;
    const int t0 = tok_begin + it * TILE;
    uint8_t* cur = s_st[S];
    // ---- wait for this tile's copies (the next tile's may stay in flight)
    if (it + 1 < ntiles) wait_vmcnt<ST::NDMA>();
    else wait_vmcnt<0>();
    const uint64_t live_mask = live[S];
    // ---- start the tile after next -----------------------------------------
    if (it + 2 < ntiles)
      live[(S + 2) % 3] = issue_tile<FK, FV, D>(a, s_blk, p0, t0 + 2 * TILE, tok_end, h, s_st[(S + 2) % 3]);

    // ---- scales -> fp32 (0 for masked tokens); FP8 codes of masked value
    //      rows zeroed (a garbage byte may be a NaN code)
    {
      const uint32_t* sdw = reinterpret_cast<const uint32_t*>(cur + ST::OFF_S);
      const int t = lane & 31;
      const bool lv = (live_mask >> t) & 1;
      const bool hi_half = h_odd ? ((t + h) & 1) : (h & 1);
      if (lane < 32) {
        if constexpr (FK != F_KIVI) {
          const uint32_t d = sdw[t];
          s_fk[t] = lv ? h2f(hi_half ? d >> 16 : d & 0xFFFFu) * a.qscale : 0.f;
        }
      }
      if constexpr (VS::NG == 1) {
        if (lane >= 32) {
          const uint32_t d = sdw[32 + t];
          s_fv[t] = lv ? h2f(hi_half ? d >> 16 : d & 0xFFFFu) : 0.f;
        }
      } else {
        // value scales of (token t, group g): dword g/2 of the token, half g&1
        // lanes 0..31 take the even dwords of token t, lanes 32..63 the odd ones
#pragma unroll
        for (int gd = 0; gd < VS::NG / 2; ++gd) {
          if ((lane >> 5) == (gd & 1)) {
            const uint32_t d = sdw[32 + 32 * gd + t];
            s_fv[t * VS::NG + 2 * gd] = lv ? h2f(d & 0xFFFFu) : 0.f;
            s_fv[t * VS::NG + 2 * gd + 1] = lv ? h2f(d >> 16) : 0.f;
          }
        }
      }
      if constexpr (FV == F_FP8) {
        if (live_mask != ~0ull) {
#pragma unroll
          for (int i = 0; i < ST::NLV; ++i) {
            const int p = 64 * i + lane;
            if (!((live_mask >> (p / VS::CH)) & 1)) *reinterpret_cast<u4*>(cur + ST::OFF_V + 16 * p) = u4{0u, 0u, 0u, 0u};
          }
        }
      }
    }

    // ---- keys: lane (j, n) reads its quarter rows of tokens n, 16 + n --------
    uint32_t kw[2][KS::NW];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 16 * u + n;
      if constexpr (KS::LB >= 16) {
#pragma unroll
        for (int q = 0; q < KS::LB / 16; ++q) {
          const int col = (j * KS::LB / 16 + q) ^ kswz<CHK>(row);
          const u4 v = *reinterpret_cast<const u4*>(cur + ST::OFF_K + (row * CHK + col) * 16);
          kw[u][4 * q] = v.x; kw[u][4 * q + 1] = v.y; kw[u][4 * q + 2] = v.z; kw[u][4 * q + 3] = v.w;
        }
      } else {  // 8 bytes per lane (KIVI, head_dim 64)
        const int col = ((j * KS::LB) / 16) ^ kswz<CHK>(row);
        const u2 v = *reinterpret_cast<const u2*>(cur + ST::OFF_K + (row * CHK + col) * 16 + (j * KS::LB) % 16);
        kw[u][0] = v.x; kw[u][1] = v.y;
      }
    }

    // ---- KIVI: this page's query operand q * s (fp16 hi + lo) and q . z ----
    h8 qhi[KS::KB], qlo[KS::KB];
    float qz = 0.f;
    if constexpr (FK == F_KIVI) {
#pragma unroll
      for (int kb = 0; kb < KS::KB; ++kb) {
        const int cb = j * (D / 4) + 8 * kb;
        const u4 sw = *reinterpret_cast<const u4*>(cur + ST::OFF_M + 2 * cb);
        const u4 zw = *reinterpret_cast<const u4*>(cur + ST::OFF_M + 2 * D + 2 * cb);
        float s8[8], z8[8];
        unpack8(uint4{sw.x, sw.y, sw.z, sw.w}, s8);
        unpack8(uint4{zw.x, zw.y, zw.z, zw.w}, z8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ch = key_channel<FK, D>(j, kb, e) - cb;
          const float qv = (float)qop[kb][e];
          const float qs = qv * s8[ch];
          const _Float16 hi = (_Float16)qs;
          qhi[kb][e] = hi;
          qlo[kb][e] = (_Float16)(qs - (float)hi);
          qz = __builtin_fmaf(qv, z8[ch], qz);
        }
      }
      qz += __shfl_xor(qz, 16);
      qz += __shfl_xor(qz, 32);
      qz *= a.qscale;
    }

    // ---- scores S^T[t][g] on the matrix cores ------------------------------
    f4 sc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sc[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KS::KB; ++kb) {
        const h8 kop = key_operand<FK>(kw[u], kb);
        if constexpr (FK == F_KIVI) {
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qhi[kb], sc[u], 0, 0, 0);
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qlo[kb], sc[u], 0, 0, 0);
        } else {
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[kb], sc[u], 0, 0, 0);
        }
      }
    }
    // lane (j, n): sc[u][r] = raw score of token 16u + 4j + r, query head n.
    float s[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f4 ks4 = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (FK != F_KIVI) ks4 = *reinterpret_cast<const f4*>(&s_fk[16 * u + 4 * j]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 16 * u + 4 * j + r;
        float v;
        if constexpr (FK == F_KIVI) v = __builtin_fmaf(sc[u][r], a.qscale, qz);
        else v = sc[u][r] * ks4[r];
        // a masked row's key codes may be anything: select, don't multiply
        v = ((live_mask >> tr) & 1) ? v : -INFINITY;
        s[4 * u + r] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    // Rescale only when some head's running max moved (rare after the first
    // tiles): alpha = 2^(m_old - m_new).
    if (__ballot(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 0 on the first live tile
      l_run *= alpha;
#pragma unroll
      for (int g = 0; g < NCS; ++g) cs_run[g] *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * j + r);
#pragma unroll
        for (int m = 0; m < VS::NPV; ++m) acc[m][r] *= ar;
      }
      m_run = m_new;
    }
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(s[e] - m_use);  // exp2(-inf) = 0 for masked rows
      l_run += p[e];
    }

    // ---- P V on the matrix cores -------------------------------------------
    // Probability operand of lane (j, n): 8 k-slots (tokens T_j[e]) of query
    // head n times the value scale, as bf16 hi + lo.  Value operands hold
    // exact codes, biased to non-negative for INT8/INT4; the bias times the
    // probability sum is removed once, after the last tile (cs_run).
    if constexpr (FV == F_INT4) {
      // element order [0, 2, 1, 3, 4, 6, 5, 7] (see value_operand_int4)
#pragma unroll
      for (int grp = 0; grp < VS::NG; ++grp) {
        uint32_t ah[4], al[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // pair q: slots (0,2) (1,3) (4,6) (5,7)
          const int s0 = (q >> 1) * 4 + (q & 1), s1 = s0 + 2;
          const int t0_ = 16 * (s0 >> 2) + 4 * j + (s0 & 3), t1_ = 16 * (s1 >> 2) + 4 * j + (s1 & 3);
          f2 used;
          split_bf16x2(f2{p[s0] * s_fv[t0_ * VS::NG + grp], p[s1] * s_fv[t1_ * VS::NG + grp]}, ah[q], al[q], used);
          cs_run[grp] += used.x + used.y;
        }
        const b8 A_hi = __builtin_bit_cast(b8, u4{ah[0], ah[1], ah[2], ah[3]});
        const b8 A_lo = __builtin_bit_cast(b8, u4{al[0], al[1], al[2], al[3]});
        const i2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(cur + tbase + ((grp ^ tswz) << 4)));
        b8 ve, vo;
        value_operand_int4(raw, ve, vo);
        acc[2 * grp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, ve, acc[2 * grp], 0, 0, 0);
        acc[2 * grp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, ve, acc[2 * grp], 0, 0, 0);
        acc[2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, vo, acc[2 * grp + 1], 0, 0, 0);
        acc[2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, vo, acc[2 * grp + 1], 0, 0, 0);
      }
    } else {
      f4 vs4[2];
      vs4[0] = *reinterpret_cast<const f4*>(&s_fv[4 * j]);
      vs4[1] = *reinterpret_cast<const f4*>(&s_fv[16 + 4 * j]);
      uint32_t ah[4], al[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // pair q: slots 2q, 2q + 1
        const int u = q >> 1, r0 = 2 * (q & 1);
        f2 used;
        split_bf16x2(f2{p[2 * q] * vs4[u][r0], p[2 * q + 1] * vs4[u][r0 + 1]}, ah[q], al[q], used);
        if constexpr (FV == F_INT8) cs_run[0] += used.x + used.y;
      }
      const b8 A_hi = __builtin_bit_cast(b8, u4{ah[0], ah[1], ah[2], ah[3]});
      const b8 A_lo = __builtin_bit_cast(b8, u4{al[0], al[1], al[2], al[3]});
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m) {
        const i2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(cur + tbase + ((m ^ tswz) << 4)));
        const b8 vop = value_operand_8bit<FV>(raw);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, vop, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, vop, acc[m], 0, 0, 0);
      }
    }
    ++it;
    return true;
  };
  for (;;) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
    if (!step(std::integral_constant<int, 2>{})) break;
  }

  // ---- remove the value-operand bias: acc[g][ch] -= bias * sum of the
  //      probability operands of query head g (INT8 +128, INT4 +136) -------
  if constexpr (FV != F_FP8) {
    constexpr float bias = FV == F_INT8 ? 128.f : 136.f;
#pragma unroll
    for (int g = 0; g < NCS; ++g) {
      float cs = cs_run[g];
      cs += __shfl_xor(cs, 16);
      cs += __shfl_xor(cs, 32);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float corr = bias * __shfl(cs, 4 * j + r);
        if constexpr (FV == F_INT8) {
#pragma unroll
          for (int m = 0; m < VS::NPV; ++m) acc[m][r] -= corr;
        } else {
          acc[2 * g][r] -= corr;
          acc[2 * g + 1][r] -= corr;
        }
      }
    }
  }

  // ---- write this split's softmax state ------------------------------------
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const size_t stride = (size_t)D + 2;
  float* pbase = a.part + (((size_t)b * a.Hq + hq0) * a.num_splits + split) * stride;
  const size_t hstride = (size_t)a.num_splits * stride;
  if (j == 0 && n < G) {
    pbase[n * hstride] = m_run;
    pbase[n * hstride + 1] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int g = 4 * j + r;
    if (g < G) {
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m) {
        const int ch = FV == F_INT4 ? 32 * (m >> 1) + 2 * n + (m & 1) : 16 * m + n;
        pbase[g * hstride + 2 + ch] = acc[m][r];
      }
    }
  }
}

// KIVI fp16 tail: the last ctx_len % 32 tokens of each sequence, keys and
// values in fp16, as one extra split (index num_splits - 1).  One wave per
// (sequence, KV head); plain fp32 arithmetic.
template <int D>
__global__ __launch_bounds__(64) void kivi_tail_kernel(DecodeArgs a) {
  const int b = (int)blockIdx.x, h = (int)blockIdx.y, lane = (int)threadIdx.x;
  const int L = min(max(a.ctx_lens[b], 0), a.max_blocks * 32);
  const int nt = b < a.max_seqs ? (L & 31) : 0;  // tail rows exist only for b < max_seqs
  const int split = a.num_splits - 1;
  const size_t stride = (size_t)D + 2;
  const size_t hstride = (size_t)a.num_splits * stride;
  float* pbase = a.part + (((size_t)b * a.Hq + h * a.G) * a.num_splits + split) * stride;
  constexpr int CPL = D / 64;  // channels per lane for the value accumulation
  for (int g = 0; g < a.G; ++g) {
    const uint16_t* qrow = a.q + ((size_t)b * a.Hq + h * a.G + g) * D;
    float sc = -INFINITY;
    if (lane < nt) {
      const uint16_t* krow = a.k_tail + (((size_t)b * 32 + lane) * a.H + h) * D;
      float dot = 0.f;
      for (int c = 0; c < D; ++c) dot = __builtin_fmaf(h2f(qrow[c]), h2f(krow[c]), dot);
      sc = dot * a.qscale;
    }
    float mx = sc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float mu = mx == -INFINITY ? 0.f : mx;
    const float pv = exp2f(sc - mu);
    float l = pv;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
    float accv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) accv[c] = 0.f;
    for (int t = 0; t < nt; ++t) {
      const float pt = __shfl(pv, t);
      const uint16_t* vrow = a.v_tail + (((size_t)b * 32 + t) * a.H + h) * D;
#pragma unroll
      for (int c = 0; c < CPL; ++c) accv[c] = __builtin_fmaf(pt, h2f(vrow[lane * CPL + c]), accv[c]);
    }
    float* dst = pbase + g * hstride;
    if (lane == 0) {
      dst[0] = mx;
      dst[1] = l;
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) dst[2 + lane * CPL + c] = accv[c];
  }
}

// Merge the splits of one (sequence, query head): M = max m_s,
// out = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), rounded to fp16.
// Four waves share the splits; lanes own channels.
constexpr int MERGE_WAVES = 4;

template <int D>
__global__ __launch_bounds__(MERGE_WAVES * 64) void merge_kernel(DecodeArgs a) {
  constexpr int CPL = D / 64;
  __shared__ float s_m[MERGE_WAVES];
  __shared__ float s_acc[MERGE_WAVES][D + 1];
  const int bh = (int)blockIdx.x, tid = (int)threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int S = a.num_splits;
  const size_t stride = (size_t)D + 2;
  const float* base = a.part + (size_t)bh * S * stride;
  float M = -INFINITY;
  for (int s = tid; s < S; s += MERGE_WAVES * 64) M = fmaxf(M, base[s * stride]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) s_m[w] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MERGE_WAVES; ++i) M = fmaxf(M, s_m[i]);
  float accv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) accv[c] = 0.f;
  float l = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = w; s < S; s += MERGE_WAVES) {
      const float* p = base + s * stride;
      const float ms = p[0];
      const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
      l = __builtin_fmaf(p[1], wgt, l);
#pragma unroll
      for (int c = 0; c < CPL; ++c) accv[c] = __builtin_fmaf(p[2 + lane * CPL + c], wgt, accv[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) s_acc[w][lane * CPL + c] = accv[c];
  if (lane == 0) s_acc[w][D] = l;
  __syncthreads();
  if (w != 0) return;
  float lt = 0.f;
#pragma unroll
  for (int i = 0; i < MERGE_WAVES; ++i) lt += s_acc[i][D];
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  uint16_t* o = a.out + (size_t)bh * D;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < MERGE_WAVES; ++i) v += s_acc[i][lane * CPL + c];
    o[lane * CPL + c] = (uint16_t)f2h_bits(v * inv);
  }
}

namespace {

template <int FK, int FV, int D>
hipError_t launch3(const DecodeArgs& a, hipStream_t st) {
  // one wave per (sequence, split, KV head); see decode_split_kernel for the order
  const uint32_t units = (uint32_t)(a.B * a.quant_splits);
  const uint32_t wgs = ((units + 7) / 8) * 8 * (uint32_t)a.H;
  hipLaunchKernelGGL((decode_split_kernel<FK, FV, D>), dim3(wgs), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (FK == F_KIVI) {
    hipLaunchKernelGGL((kivi_tail_kernel<D>), dim3((unsigned)a.B, (unsigned)a.H), dim3(64), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)(a.B * a.Hq)), dim3(MERGE_WAVES * 64), 0, st, a);
  return hipGetLastError();
}

template <int FK, int FV>
hipError_t by_dim(int D, const DecodeArgs& a, hipStream_t s) {
  switch (D) {
    case 64: return launch3<FK, FV, 64>(a, s);
    case 128: return launch3<FK, FV, 128>(a, s);
    case 256: return launch3<FK, FV, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int FK>
hipError_t by_v(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  switch (fv) {
    case F_INT8: return by_dim<FK, F_INT8>(D, a, s);
    case F_FP8: return by_dim<FK, F_FP8>(D, a, s);
    case F_INT4: return by_dim<FK, F_INT4>(D, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int32_t choose_pages_per_split(const kvq_cache& c, int32_t batch, int32_t max_blocks, int32_t requested) {
  // Tiles are 32 tokens, so a split is a whole number of tiles.
  const int32_t unit = c.block_size >= 32 ? 1 : 32 / c.block_size;
  int32_t pps = requested;
  if (pps <= 0) {
    // Enough workgroups to fill 256 CUs several times over, each holding
    // a few thousand tokens per KV head.
    const int64_t target_units = 1024;  // (sequence, split) pairs; each runs n_kv_heads waves
    int64_t per_seq = (target_units + batch - 1) / batch;
    if (per_seq < 1) per_seq = 1;
    pps = (int32_t)((max_blocks + per_seq - 1) / per_seq);
    const int32_t min_pps = (512 + c.block_size - 1) / c.block_size;  // >= 512 tokens per split
    if (pps < min_pps) pps = min_pps;
  }
  pps = ((pps + unit - 1) / unit) * unit;
  if (pps > MAX_PPS) pps = (MAX_PPS / unit) * unit;
  return pps;
}

hipError_t launch_decode(const kvq_cache& c, const DecodeArgs& a, hipStream_t s) {
  switch (c.k_dtype) {
    case F_INT8: return by_v<F_INT8>(c.v_dtype, c.head_dim, a, s);
    case F_FP8: return by_v<F_FP8>(c.v_dtype, c.head_dim, a, s);
    case F_KIVI: return by_v<F_KIVI>(c.v_dtype, c.head_dim, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
