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
//  * Work partition: the quantized 32-token tiles of all sequences are
//    numbered sequence after sequence and cut into equal shares (a small plan
//    kernel, or each wave itself, computes the cut on the device).  A share
//    is read by one wave per group of HP = 1, 2 or 4 KV heads, which handles
//    the G query heads of each; the waves of a share form one workgroup, so
//    they run on one compute unit.  By default as many waves run as fit at
//    once (two per SIMD up to head_dim 128), all with the same amount of
//    work, so no wave waits for a later round.  A wave writes one partial
//    softmax state per sequence piece it covers; a merge kernel combines them.
//  * Data path: a tile's key and value rows, scales and block ids are loaded
//    into registers several tiles ahead (the compiler tracks the loads, and
//    every step issues the same loads so its waits stay exact), then stored
//    into one LDS stage in a swizzled layout and read back as MFMA operands.
//  * Scores S^T = K Q^T run on the matrix cores (v_mfma_f32_16x16x32_f16):
//    the 8-bit/4-bit key codes become exact fp16 operands (q is fp16
//    already), so the products are exact and only the fp32 accumulation
//    rounds; the per-token key scale is applied to the fp32 score afterwards
//    (q.k_hat = s_k (q.codes)).
//  * Values are read back with the 8-bit transpose read (ds_read_b64_tr_b8),
//    which hands each lane one channel (INT8/FP8) or one channel pair (INT4)
//    of 8 tokens, the layout the matrix core wants for P V.  Value codes
//    become exact bf16 operands; the probabilities times the per-token value
//    scale are split into two bf16 terms (hi + lo, relative error <= 2^-18),
//    so P V costs two MFMAs per 16 channels and keeps fp32-level accuracy.
//  * Online softmax in the log2 domain (q pre-multiplied by sm_scale*log2 e),
//    fp32 throughout; each piece stores (m, l, acc[D]).
#pragma once

#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

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
// Balanced partition: at most this many waves, and at least this many tiles
// per share unless the caller asks for a size.
constexpr int AUTO_MAX_WAVES = 4096;
constexpr int AUTO_MIN_TILES = 4;

template <int FK, int D>
struct KShape {
  static constexpr int RB = FK == F_KIVI || FK == F_INT4 ? D / 2 : D;  // key row bytes
  static constexpr int LB = RB / 4;                    // bytes per lane (quarter row)
  static constexpr int NW = LB / 4;                    // dwords per lane
  static constexpr int KB = D / 32;                    // MFMA k-blocks
  // INT4 keys: one scale per 32 channels (k-block kb is scale group kb);
  // a row's scales fill NGKD whole dwords
  static constexpr int NGK = FK == F_INT4 ? D / 32 : 1;
  static constexpr int NGKD = FK == F_INT4 ? D / 64 : 1;
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

// E5M2 -> fp16: an E5M2 byte is the upper byte of the fp16 of the same value
// (one v_perm per two codes).
__device__ __forceinline__ void e5m2_to_h4(uint32_t d, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_amdgcn_perm(0u, d, 0x010C000Cu);  // [0, c0, 0, c1]
  hi = __builtin_amdgcn_perm(0u, d, 0x030C020Cu);  // [0, c2, 0, c3]
}

template <int FK>
__device__ __forceinline__ h8 key_operand(const uint32_t* w, int kb) {
  u4 r;
  if constexpr (FK == F_INT4) {
    // 8 two's-complement nibbles of one dword, channels 32 kb + 8 j .. + 7
    // (byte b: channel 2b low, 2b + 1 high); pair i = channels (i, i + 4).
    // (nibble ^ 8) under the fp16 exponent of 1024 is 1024 + c + 8, exactly;
    // one packed subtract of 1032 leaves c.  f(x, m, k) = (x & m) ^ k has the
    // truth table 0x6A (x = 0xF0, m = 0xCC, k = 0xAA).
    const uint32_t d = w[kb];
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    auto pair = [&](uint32_t x) __attribute__((always_inline)) {
      return h2_bits(as_h2(__builtin_amdgcn_bitop3_b32(x, 0x000F000Fu, 0x64086408u, 0x6A)) - bias);
    };
    r.x = pair(d);
    r.y = pair(d >> 4);
    r.z = pair(d >> 8);
    r.w = pair(d >> 12);
  } else if constexpr (FK == F_KIVI) {
    // 8 unsigned nibbles of one dword; pair i = channels (i, i + 4).  A
    // nibble in mantissa bits 0-3 of an fp16 is the subnormal n 2^-24, in
    // bits 4-7 it is 16 n 2^-24, both exact: even channels (x, z) give
    // n 2^-24, odd channels (y, w) 16 n 2^-24; the query operand of even
    // channels carries the factor 16 instead.
    const uint32_t d = w[kb], t = d >> 8;
    r.x = d & 0x000F000Fu;
    r.y = d & 0x00F000F0u;
    r.z = t & 0x000F000Fu;
    r.w = t & 0x00F000F0u;
  } else {
    uint32_t x0, x1, x2, x3;
    if constexpr (FK == F_FP8) {
      fp8_to_h4(w[2 * kb], x0, x1);
      fp8_to_h4(w[2 * kb + 1], x2, x3);
    } else if constexpr (FK == F_E5M2) {
      e5m2_to_h4(w[2 * kb], x0, x1);
      e5m2_to_h4(w[2 * kb + 1], x2, x3);
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
  if constexpr (FK == F_INT4) return 32 * kb + 8 * j + ((e & 1) ? 4 + (e >> 1) : (e >> 1));
  const int base = j * (D / 4) + 8 * kb;
  if constexpr (FK == F_KIVI) return base + ((e & 1) ? 4 + (e >> 1) : (e >> 1));
  return base + e;
}

// ---- value operands: 8 exact bf16 values, 8 tokens of one channel ----------
// FP8 (E4M3FN, E5M2): the exact value.  INT8 and INT4: the unsigned code u (c + 128, or
// c + 8 for INT4) as the bf16 bit pattern u, which is exactly u 2^-133 for
// every u < 256 (subnormal below 128; from 128 on the smallest exponent
// continues the same spacing).  The probability operand carries 2^60 so the
// products stay normal fp32; the offset times the probability sum is removed
// once per piece (cs_run), and the scale factors with it.

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
  } else if constexpr (FV == F_E5M2) {
    // FP8 E5M2 -> bf16, two codes per instruction (exact)
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, 1.0f, true));
  } else {
    // bytes c + 128 into zero-padded halves: [u0, 0, u1, 0] per dword
    const uint32_t e0 = d0 ^ 0x80808080u, e1 = d1 ^ 0x80808080u;
    r.x = __builtin_amdgcn_perm(0u, e0, 0x0C010C00u);
    r.y = __builtin_amdgcn_perm(0u, e0, 0x0C030C02u);
    r.z = __builtin_amdgcn_perm(0u, e1, 0x0C010C00u);
    r.w = __builtin_amdgcn_perm(0u, e1, 0x0C030C02u);
  }
  return __builtin_bit_cast(b8, r);
}

// INT4: 8 bytes = 8 tokens of a channel pair; element order of both operands
// is tokens [0, 2, 1, 3, 4, 6, 5, 7].  Each operand dword is one v_bitop3,
// (x ^ c) & m: the even channel's nibbles xor 8 (code + 8) stay in bits 0-3
// of each half (u 2^-133), the odd channel's in bits 4-7 (16 u 2^-133).
template <uint32_t M, uint32_t C>
__device__ __forceinline__ uint32_t int4_pair(uint32_t x) {
  // f(x, m, c) = m & (x ^ c) (truth table of x = 0xF0, m = 0xCC, c = 0xAA)
  return __builtin_amdgcn_bitop3_b32(x, M, C, 0x48);
}
__device__ __forceinline__ void value_operand_int4(i2 t, b8& even, b8& odd) {
  const uint32_t d0 = (uint32_t)t.x, d1 = (uint32_t)t.y, d0s = d0 >> 8, d1s = d1 >> 8;
  constexpr uint32_t ME = 0x000F000Fu, CE = 0x00080008u, MO = 0x00F000F0u, CO = 0x00800080u;
  u4 e, od;
  e.x = int4_pair<ME, CE>(d0);
  e.y = int4_pair<ME, CE>(d0s);
  e.z = int4_pair<ME, CE>(d1);
  e.w = int4_pair<ME, CE>(d1s);
  od.x = int4_pair<MO, CO>(d0);
  od.y = int4_pair<MO, CO>(d0s);
  od.z = int4_pair<MO, CO>(d1);
  od.w = int4_pair<MO, CO>(d1s);
  even = __builtin_bit_cast(b8, e);
  odd = __builtin_bit_cast(b8, od);
}

// x = hi + lo with hi = bf16_rne(x), lo = bf16_rne(x - hi), two values at a
// time (v_cvt_pk_bf16_f32).
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16x2(f2 x, uint32_t& hi, uint32_t& lo) {
  const bf2 h = __builtin_convertvector(x, bf2);
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const f2 fh = {__builtin_bit_cast(float, hb << 16), __builtin_bit_cast(float, hb & 0xFFFF0000u)};
  const bf2 l = __builtin_convertvector(x - fh, bf2);
  hi = hb;
  lo = __builtin_bit_cast(uint32_t, l);
}
// cs + the four bf16 values of a split pair (what the operands hold), with
// two v_dot2_f32_bf16 against (1, 1).  The accumulating dot product does not
// round like an IEEE add (measured on gfx950: a long chain of them drifts by
// several 1e-4 relative), so callers sum one tile's operands in a fresh chain
// and add that to the running sum with an fp32 add.
__device__ __forceinline__ float add_split(float cs, uint32_t hi, uint32_t lo) {
  const bf2 one = {(__bf16)1.0f, (__bf16)1.0f};
  cs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, hi), one, cs, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, lo), one, cs, false);
}

// Lanes l and l ^ 16 (or l ^ 32) without a trip through LDS: swapping x with
// itself by v_permlane16_swap (v_permlane32_swap) leaves, on every lane, the
// pair's lower-row (lower-half) value in one register and its upper one in
// the other.  Max and sum are symmetric, so the results equal those of a
// lane exchange bit for bit.
// (The results are copied out element by element before the bit cast: a bit
// cast of a vector element reference reads element 0 with this compiler.)
template <int X>
__device__ __forceinline__ f2 xor_pair(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = X == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t lo = r[0], hi = r[1];
  return f2{__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi)};
}
// reduction over the 4 lanes l ^ {0, 16, 32, 48}
__device__ __forceinline__ float sum_j(float x) {
  f2 p = xor_pair<16>(x);
  p = xor_pair<32>(p.x + p.y);
  return p.x + p.y;
}
__device__ __forceinline__ float max_j(float x) {
  f2 p = xor_pair<16>(x);
  p = xor_pair<32>(fmaxf(p.x, p.y));
  return fmaxf(p.x, p.y);
}

// Tile row rho (0..31) is token t0 + rho / HP of the sequence, KV head
// h0 + rho % HP (HP = 2^hp_log2 heads per wave).  Returns its flat row index
// (slot * H + head) and whether it is live: in the context and on a page
// whose block id (bid) is valid.
__device__ __forceinline__ uint32_t tile_row(const DecodeArgs& a, int bid, int rho, int t0, int tok_end, int h0,
                                             bool& live) {
  const int tt = t0 + (rho >> a.hp_log2);
  const int lbs = a.log2_bs;
  live = tt < tok_end && bid >= 0 && bid < a.nb;
  const uint32_t blk = live ? (uint32_t)bid : 0u;
  const uint32_t head = (uint32_t)(h0 + (rho & ((1 << a.hp_log2) - 1)));
  return ((blk << lbs) + (uint32_t)(tt & ((1 << lbs) - 1))) * (uint32_t)a.H + head;
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
  // KIVI: the page's scales, then its zeros, of up to 4 KV heads (fp16)
  static constexpr int KIVI_BYTES = FK == F_KIVI ? 4 * 2 * D * 2 : 0;
  // byte offsets inside a stage
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = KT;
  static constexpr int OFF_S = KT + VT;              // raw scale dwords (see load_tile)
  static constexpr int OFF_M = OFF_S + 4 * TILE * (KS::NGKD + NGD);
  static constexpr int BYTES = OFF_M + KIVI_BYTES;
  // one wave's LDS: the stage, then this tile's key scales (TILE NGK fp32)
  // and value scales (TILE NG fp32)
  static constexpr int WAVE_LDS = (BYTES + 4 * TILE * KS::NGK + 4 * TILE * VS::NG + 15) / 16 * 16;
  // Waves per SIMD and register slots for tiles.  Head dims up to 128 run
  // two waves per SIMD (each within 256 registers), so one wave's compute
  // hides the other's waits; a wave then holds NS = 2 tiles (one in flight
  // while one is stored to LDS and computed).  Head dim 256 runs one wave per
  // SIMD with up to 4 tiles held, within about 136 registers.
  static constexpr int WPE = D <= 128 ? 2 : 1;
  static constexpr int TILE_REGS = 4 * (NLK + NLV) + NGD + KS::NGKD + (FK == F_KIVI ? 4 * (D / 64) : 0);
  static constexpr int NS_FIT = 136 / TILE_REGS;
  static constexpr int NS = WPE == 2 ? 2 : (NS_FIT < 2 ? 2 : (NS_FIT > 4 ? 4 : NS_FIT));
};

// One tile's global data in registers: the 16-byte chunks of its key and
// value rows, its scale dwords and (KIVI) its page's scales and zeros for the
// wave's HPC heads.  Each lane holds exactly what it later stores into the
// LDS stage.
template <int FK, int FV, int D, int HPC>
struct TileRegs {
  using S = Stage<FK, FV, D>;
  using VS = VShape<FV, D>;
  static constexpr int MCH = FK == F_KIVI ? HPC * D / 4 : 0;  // 16-byte chunks of page metadata
  static constexpr int KM = (MCH + 63) / 64;                  // per lane
  static constexpr int NR = HPC >= 2 ? 2 * (4 / HPC) : 1;     // score rows per lane
  static constexpr int VSB = 2 * VS::NG;                      // value-scale bytes per row
  static constexpr int VW = VSB >= 4 ? VSB / 4 : 1;           // ... in registers
  u4 k[S::NLK];
  u4 v[S::NLV];
  uint32_t s[S::NGD];
  uint32_t sk[KShape<FK, D>::NGKD > 1 ? KShape<FK, D>::NGKD - 1 : 1];  // INT4 keys: key-scale dwords 1..
  uint32_t par;  // bit rho: row rho's 16-bit scale is the high half of its dword
  // direct scales (one page per tile, two or four heads per wave): the raw
  // fp16 key scale and value scales of the lane's score rows
  uint32_t fk[NR];
  uint32_t fv[NR][VW];
  u4 m[KM > 0 ? KM : 1];
};

// Direct scales: with one page per tile and two or four KV heads per wave,
// each lane loads the scales of its own score rows (two or four rows, see
// score_row) straight into registers; otherwise every row's scales are
// loaded once and passed on through LDS.
template <int HPC, bool OP>
constexpr bool direct_scales() {
  return OP && HPC >= 2;
}

// Score row i (i = u (4 / HPC) + ii) of lane group j whose column's KV head
// is hn: tile row 16 u + 4 j + r, r = hn + HPC ii.
template <int HPC>
__device__ __forceinline__ int score_row(int j, int hn, int i) {
  constexpr int NU = 4 / HPC;
  const int u = i / NU, ii = i % NU;
  return 16 * u + 4 * j + (HPC == 1 ? ii : hn + HPC * ii);
}

// Raw buffer resource over `base` (word 3: 32-bit data format, so untyped
// loads are valid); offsets stay within one page by construction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
constexpr int BUF_NT = 2;  // cache policy of a streaming load (nt)
template <int BYTES, int AUX = 0>
__device__ __forceinline__ void buf_load(uint32_t* dst, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (BYTES == 16) {
    const u4 x = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
    dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
  } else if constexpr (BYTES == 8) {
    const u2 x = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX));
    dst[0] = x.x; dst[1] = x.y;
  } else if constexpr (BYTES == 4) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX);
  } else {
    dst[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, AUX);
  }
}

// Load one tile (keys, values, per-token scale dwords; KIVI page scales and
// zeros) into registers; bid is the block id of token lane % 32's page.
// Returns the live-token mask (bit t and t + 32: token t0 + t is in the
// context on a valid page).  Every load is issued by every lane, so each
// tile costs the same number of loads: masked rows read flat row 0 (every
// cache has at least one block) and idle lanes the start of the buffer;
// those bytes are never used unmasked.
//
// OP (one page): the tile's 32 / HPC tokens lie in one page (block_size is
// a multiple of them; tiles start at multiples of them), so bid is the same
// on every lane and tile row rho is flat row row0 + (rho / HPC) H + rho % HPC:
// a uniform page base plus a per-lane constant, with no row exchange between
// lanes.  Rows past the context are read from the same page (page 0 when bid
// is out of range), so every address stays inside the cache; they are masked.
template <int FK, int FV, int D, int HPC, bool OP>
__device__ __forceinline__ uint64_t load_tile(const DecodeArgs& a, int bid, int t0, int tok_end, int h0,
                                              const uint32_t* sro, TileRegs<FK, FV, D, HPC>& r) {
  using S = Stage<FK, FV, D>;
  using KS = KShape<FK, D>;
  using VS = VShape<FV, D>;
  constexpr int CHK = KS::RB / 16 > 0 ? KS::RB / 16 : 1;
  const int lane = (int)threadIdx.x & 63;
  if constexpr (OP) {
    constexpr int hp = HPC == 4 ? 2 : HPC == 2 ? 1 : 0;
    const int bu = __builtin_amdgcn_readfirstlane(bid);
    const bool bok = bu >= 0 && bu < a.nb;
    const uint32_t blk = bok ? (uint32_t)bu : 0u;
    const uint32_t row0 = ((blk << a.log2_bs) + (uint32_t)(t0 & (a.bs - 1))) * (uint32_t)a.H + (uint32_t)h0;
    // flat-row offset of tile row rho from row0
    auto ro = [&](int rho) __attribute__((always_inline)) {
      return (uint32_t)((rho >> hp) * a.H + (rho & (HPC - 1)));
    };
    const int t = lane & 31;
    const bool live = bok && t0 + (t >> hp) < tok_end;
    const uint64_t live_mask = __ballot(live);
    const uint32_t r_own = row0 + ro(t);
    // buffer loads from the page base (scalar) at per-lane constant offsets
    const auto rk = buf_rsrc(a.k_codes + (size_t)row0 * KS::RB);
    const auto rv = buf_rsrc(a.v_codes + (size_t)row0 * VS::RB);
#pragma unroll
    for (int i = 0; i < S::NLK; ++i) {
      const int p = 64 * i + lane;
      const int row = p / CHK;
      const int col = (p % CHK) ^ kswz<CHK>(row);
      buf_load<16, BUF_NT>(reinterpret_cast<uint32_t*>(&r.k[i]), rk, ro(row) * KS::RB + col * 16);
    }
#pragma unroll
    for (int i = 0; i < S::NLV; ++i) {
      const int p = 64 * i + lane;
      const int row = p / VS::CH;
      const int col = (p % VS::CH) ^ vswz<VS::CH>(row);
      buf_load<16, BUF_NT>(reinterpret_cast<uint32_t*>(&r.v[i]), rv, ro(row) * VS::RB + col * 16);
    }
    if constexpr (direct_scales<HPC, OP>()) {
      // the lane's score rows (flat-row offsets sro from row0)
      using TR = TileRegs<FK, FV, D, HPC>;
      const auto rks = buf_rsrc(a.k_scales + row0);
      const auto rvs = buf_rsrc(a.v_scales + (size_t)row0 * VS::NG);
#pragma unroll
      for (int i = 0; i < TR::NR; ++i) {
        if constexpr (FK != F_KIVI) buf_load<2>(&r.fk[i], rks, sro[i] * 2);
        buf_load<TR::VSB>(r.fv[i], rvs, sro[i] * TR::VSB);
      }
    } else {
      {
        const uint16_t* src;
        if (lane < 32) src = FK == F_KIVI ? a.v_scales : a.k_scales + (r_own & ~1u);
        else src = a.v_scales + ((size_t)r_own * VS::NG & ~(size_t)1);
        r.s[0] = *reinterpret_cast<const uint32_t*>(src);
        r.par = (uint32_t)__ballot(live && (r_own & 1u));
      }
#pragma unroll
      for (int g = 1; g < S::NGD; ++g)
        r.s[g] = *reinterpret_cast<const uint32_t*>(a.v_scales + (lane < 32 ? (size_t)r_own * VS::NG + 2 * g : 0));
    }
    if constexpr (FK == F_KIVI) {
      using TR = TileRegs<FK, FV, D, HPC>;
      constexpr int HALF = HPC * D / 8;
      const size_t mrow = ((size_t)blk * a.H + h0) * D;
#pragma unroll
      for (int k = 0; k < TR::KM; ++k) {
        const int c = 64 * k + lane;
        const bool use = c < TR::MCH;
        const uint16_t* src = (c < HALF ? a.k_scales : a.k_zeros) + (use ? mrow + 8 * (c < HALF ? c : c - HALF) : 0);
        r.m[k] = *reinterpret_cast<const u4*>(src);
      }
    }
    return live_mask;
  }
  // row index of token `lane & 31`, or ~0 when masked; shared with shuffles
  bool live;
  const uint32_t r_own = tile_row(a, bid, lane & 31, t0, tok_end, h0, live);
  const uint64_t live_mask = __ballot(live);
  const uint32_t rl = live ? r_own : 0u;
#pragma unroll
  for (int i = 0; i < S::NLK; ++i) {
    const int p = 64 * i + lane;  // LDS chunk slot this lane stores
    const int row = p / CHK;
    const int col = (p % CHK) ^ kswz<CHK>(row);
    const uint32_t rr = (uint32_t)__shfl((int)rl, row);
    r.k[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u4*>(a.k_codes + (size_t)rr * KS::RB + col * 16));
  }
#pragma unroll
  for (int i = 0; i < S::NLV; ++i) {
    const int p = 64 * i + lane;
    const int row = p / VS::CH;
    const int col = (p % VS::CH) ^ vswz<VS::CH>(row);
    const uint32_t rr = (uint32_t)__shfl((int)rl, row);
    r.v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u4*>(a.v_codes + (size_t)rr * VS::RB + col * 16));
  }
  // scale dwords (LDS dword index): [rho] the dword holding row rho's key
  // scale, [32 + rho] the first value-scale dword of row rho, [32 + 32 k +
  // rho] its value-scale dword k >= 1 (INT4 groups; lanes < 32).  A lone
  // fp16 scale sits in half (flat row & 1) of its dword (par).  INT4 keys:
  // [rho] is the first of row rho's key-scale dwords (groups 0, 1), and
  // [32 (1 + NGD) + 32 (k - 1) + rho] its key-scale dword k >= 1.
  {
    const uint16_t* src;
    if (lane < 32) {
      if constexpr (FK == F_KIVI) src = a.v_scales;
      else if constexpr (FK == F_INT4) src = a.k_scales + (live ? (size_t)r_own * KS::NGK : 0);
      else src = a.k_scales + (live ? (r_own & ~1u) : 0);
    } else {
      src = a.v_scales + (live ? ((size_t)r_own * VS::NG & ~(size_t)1) : 0);
    }
    r.s[0] = *reinterpret_cast<const uint32_t*>(src);
    r.par = (uint32_t)__ballot(live && (r_own & 1u));
  }
#pragma unroll
  for (int g = 1; g < S::NGD; ++g)
    r.s[g] = *reinterpret_cast<const uint32_t*>(a.v_scales +
                                                (live && lane < 32 ? (size_t)r_own * VS::NG + 2 * g : 0));
  if constexpr (FK == F_INT4) {
#pragma unroll
    for (int g = 1; g < KS::NGKD; ++g)
      r.sk[g - 1] = *reinterpret_cast<const uint32_t*>(a.k_scales +
                                                       (live && lane < 32 ? (size_t)r_own * KS::NGK + 2 * g : 0));
  }
  if constexpr (FK == F_KIVI) {
    // the tile lies in one page (block_size 32): the D scales of heads
    // h0 .. h0 + HPC - 1 (contiguous), then their D zeros; chunk c of 16 bytes
    using TR = TileRegs<FK, FV, D, HPC>;
    constexpr int HALF = HPC * D / 8;  // chunks of scales
    const uint32_t r0 = (uint32_t)__shfl((int)rl, 0);
    const size_t mrow = ((size_t)(r0 / (32u * (uint32_t)a.H)) * a.H + h0) * D;
#pragma unroll
    for (int k = 0; k < TR::KM; ++k) {
      const int c = 64 * k + lane;
      const bool use = c < TR::MCH;
      const uint16_t* src = (c < HALF ? a.k_scales : a.k_zeros) + (use ? mrow + 8 * (c < HALF ? c : c - HALF) : 0);
      r.m[k] = *reinterpret_cast<const u4*>(src);
    }
  }
  return live_mask;
}

// Store a loaded tile into the LDS stage `st` (layout of Stage).
template <int FK, int FV, int D, int HPC, bool OP>
__device__ __forceinline__ void store_tile(const TileRegs<FK, FV, D, HPC>& r, uint8_t* st) {
  using S = Stage<FK, FV, D>;
  const int lane = (int)threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < S::NLK; ++i) reinterpret_cast<u4*>(st + S::OFF_K)[64 * i + lane] = r.k[i];
#pragma unroll
  for (int i = 0; i < S::NLV; ++i) reinterpret_cast<u4*>(st + S::OFF_V)[64 * i + lane] = r.v[i];
  if constexpr (!direct_scales<HPC, OP>()) {
    uint32_t* sd = reinterpret_cast<uint32_t*>(st + S::OFF_S);
    sd[lane] = r.s[0];
#pragma unroll
    for (int g = 1; g < S::NGD; ++g)
      if (lane < 32) sd[32 + 32 * g + lane] = r.s[g];
    if constexpr (FK == F_INT4) {
#pragma unroll
      for (int g = 1; g < KShape<FK, D>::NGKD; ++g)
        if (lane < 32) sd[32 * (1 + S::NGD) + 32 * (g - 1) + lane] = r.sk[g - 1];
    }
  }
  if constexpr (FK == F_KIVI) {
    using TR = TileRegs<FK, FV, D, HPC>;
#pragma unroll
    for (int k = 0; k < TR::KM; ++k)
      if (64 * k + lane < TR::MCH) reinterpret_cast<u4*>(st + S::OFF_M)[64 * k + lane] = r.m[k];
  }
}

// Sequence b of the tile numbering owns tiles [lo, hi) and holds lq tokens in
// quantized pages.  Lane i of the window registers holds, for sequence
// wb + i, the end of its tile range (hi) and lq; a cursor reads them with
// readlane, so moving to the next sequence costs no memory access (a refill
// after 64 sequences does).
struct SeqCursor {
  int b, wb, lo, hi, lq;
  int win_hi, win_lq;  // per lane
};

template <int FK>
__device__ __forceinline__ int seq_tokens(const DecodeArgs& a, int b) {
  // ctx_len clamped to what the block-table row addresses; KIVI: whole pages
  const int L = min(max(a.ctx_lens[b], 0), a.max_blocks << a.log2_bs);
  return FK == F_KIVI ? (L & ~31) : L;
}

template <int FK>
__device__ __forceinline__ void fill_window(SeqCursor& c, const DecodeArgs& a, int wb) {
  const int lane = (int)threadIdx.x & 63, sb = wb + lane;
  c.wb = wb;
  c.win_hi = sb < a.B ? a.plan[2 + sb] : INT_MAX;
  c.win_lq = sb < a.B ? seq_tokens<FK>(a, sb) : 0;
}

__device__ __forceinline__ int rdlane(int v, int i) { return __builtin_amdgcn_readlane(v, i); }

// The plan of a batch of at most 64 sequences, computed by one wave: lane b
// holds sequence b's quantized tokens (lq), tiles (n) and first tile (excl);
// returns the tiles of the whole batch.
template <int FK>
__device__ __forceinline__ int wave_plan(const DecodeArgs& a, int& lq, int& n, int& excl) {
  const int lane = (int)threadIdx.x & 63;
  lq = lane < a.B ? seq_tokens<FK>(a, lane) : 0;
  const int tt = TILE >> a.hp_log2;
  n = (lq + tt - 1) / tt;
  int incl = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  excl = incl - n;
  return rdlane(incl, 63);
}

// Tiles per share: requested, or the balanced share of num_shares.
__device__ __forceinline__ int share_size(const DecodeArgs& a, int total) {
  return a.share_tiles > 0 ? a.share_tiles : max((total + a.num_shares - 1) / a.num_shares, AUTO_MIN_TILES);
}

// Move the cursor to the sequence holding tile x (x >= the current tile and
// x < the number of tiles, so the loop ends on a valid sequence).
template <int FK>
__device__ __forceinline__ void seek(SeqCursor& c, const DecodeArgs& a, int x) {
  if (x < c.hi) return;
  do {
    ++c.b;
    if (c.b - c.wb >= 64) fill_window<FK>(c, a, c.b);
    c.lo = c.hi;
    c.hi = rdlane(c.win_hi, c.b - c.wb);
  } while (x >= c.hi);
  c.lq = rdlane(c.win_lq, c.b - c.wb);
}

// Block id of the page of tile row lane % 32 of tile x of the cursor's
// sequence (entry 0 of its row past the sequence's end; those rows are masked).
// OP: every lane loads the page of the tile's first token (in the sequence).
template <bool OP>
__device__ __forceinline__ int load_ids(const DecodeArgs& a, const SeqCursor& c, int x) {
  if constexpr (OP) {
    const int tok0 = (TILE * (x - c.lo)) >> a.hp_log2;
    return a.block_table[(size_t)c.b * a.max_blocks + (tok0 >> a.log2_bs)];
  }
  const int tok = ((TILE * (x - c.lo)) >> a.hp_log2) + (((int)threadIdx.x & 31) >> a.hp_log2);
  const int pg = tok < c.lq ? tok >> a.log2_bs : 0;
  return a.block_table[(size_t)c.b * a.max_blocks + pg];
}

// HPC: KV heads per wave (a.hp_log2 == log2 HPC).  Lane (j, n) keeps only the
// scores of its column's head: rows 16 u + 4 j + r with r = hn (mod HPC).
// OP: every tile lies in one page (32 / HPC <= block_size), see load_tile.
//
// A workgroup holds NW = blockDim.x / 64 waves of one share: KV-head groups
// c NW .. c NW + NW - 1.  They run on one compute unit and read neighbouring
// segments of the same token rows at about the same time; each has its own
// LDS (dynamic, NW Stage::WAVE_LDS bytes) and they never synchronize.
//
// ROTQ (keys stored Walsh-Hadamard rotated): the query operand is the rotated
// query q' = H (sigma q) / D, which is not an fp16 value: it is read as fp16
// hi + lo (a pre-pass writes both to the workspace) and every key k-block
// takes two MFMAs, so the products stay exact and q' keeps fp32 accuracy.
template <int FK, int FV, int D, int HPC, bool OP, bool ROTQ>
__global__ __launch_bounds__((256 * Stage<FK, FV, D>::WPE))
__attribute__((amdgpu_waves_per_eu(Stage<FK, FV, D>::WPE, Stage<FK, FV, D>::WPE)))
void decode_split_kernel(DecodeArgs a) {
  using KS = KShape<FK, D>;
  using VS = VShape<FV, D>;
  using ST = Stage<FK, FV, D>;
  constexpr int CHK = KS::RB / 16 > 0 ? KS::RB / 16 : 1;
  constexpr int NCS = FV == F_INT4 ? VS::NG : 1;  // bias-correction sums kept per value group
  // value scales carry 2^60 for the INT8 / INT4 value operands (u 2^-133)
  constexpr bool VFP8 = FV == F_FP8 || FV == F_E5M2;  // value operands hold the exact value
  constexpr float VSC = VFP8 ? 1.f : 0x1p60f;
  // NS tiles held in registers: tile x is stored to LDS and computed while
  // tiles x + 1 .. x + P are in flight
  constexpr int NS = ST::NS, P = NS - 1;
  constexpr int L = NS > 2 ? 2 : 1;  // block ids are loaded L tiles ahead of their tile
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
  // wave of the workgroup (uniform: so are the head group and every address
  // derived from it, which then stay in scalar registers)
  const uint32_t wv = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint8_t* const s_st = s_dyn + wv * ST::WAVE_LDS;
  // this tile's scales as fp32: key scale x sm_scale x log2 e, value scales
  float* const s_fk = reinterpret_cast<float*>(s_st + ST::BYTES);
  float* const s_fv = s_fk + TILE * KS::NGK;

  // Wave (share, group of HP KV heads).  The workgroups of one share (when
  // a share needs more than one) are consecutive workgroups of one XCD
  // (workgroups are dealt to the 8 XCDs round robin), so they read the same
  // page-scale lines of its L2 at about the same time.
  const uint32_t wg = blockIdx.x;
  const uint32_t kk = wg >> 3;
  const uint32_t nw = blockDim.x >> 6;
  const uint32_t nwg = (uint32_t)(a.H >> a.hp_log2) / nw;  // workgroups per share
  const int h0 = (int)((kk % nwg) * nw + wv) << a.hp_log2;  // first KV head of the wave
  const int share = (int)((kk / nwg) * 8 + (wg & 7));
  if (share >= a.num_shares) return;
  SeqCursor cc;  // tile being computed
  int S, total;
  if (a.inline_plan) {
    // one window holds the whole batch
    int lq, nt, excl;
    total = wave_plan<FK>(a, lq, nt, excl);
    S = share_size(a, total);
    if (share * S >= total) return;
    const int lane = (int)threadIdx.x & 63;
    cc.wb = 0;
    cc.win_hi = lane < a.B ? excl + nt : INT_MAX;
    cc.win_lq = lq;
    // first sequence whose tiles end after the share's first tile
    cc.b = __popcll(__ballot(lane < a.B && excl + nt <= share * S));
    cc.lo = rdlane(excl, cc.b);
    cc.hi = rdlane(cc.win_hi, cc.b);
    cc.lq = rdlane(cc.win_lq, cc.b);
  } else {
    S = a.plan[0];
    total = a.plan[1 + a.B];
    if (share * S >= total) return;
    cc.b = a.plan[2 + a.B + share];
    cc.lo = a.plan[1 + cc.b];
    fill_window<FK>(cc, a, cc.b);
    cc.hi = rdlane(cc.win_hi, 0);
    cc.lq = rdlane(cc.win_lq, 0);
  }
  const int x_begin = share * S;
  const int x_end = min(x_begin + S, total);
  SeqCursor ci = cc, cd = cc;  // tile being issued, block ids being fetched

  const int lane = (int)threadIdx.x & 63;
  const int j = lane >> 4, n = lane & 15;
  // MFMA column n (query operand, scores, output rows) is query head
  // hq0 + n: KV head h0 + n / G, for n < NC = HP G (at most 16).
  const int G = a.G;
  const int NC = G << a.hp_log2;
  const int hq0 = h0 * G;
  // tile rows whose KV head is column n's (all rows when HP = 1)
  const int hp_mask = HPC - 1;
  const int hn = n < NC ? n / G : 0;  // column n's head within the wave
  uint32_t colmask = 0;
  if (n < NC) {
#pragma unroll
    for (int rho = 0; rho < 32; ++rho) colmask |= ((rho & hp_mask) == n / G ? 1u : 0u) << rho;
  }
  // direct scales: the lane's score rows and their flat-row offsets from the
  // tile's first row (one page per tile)
  constexpr bool DSC = direct_scales<HPC, OP>();
  constexpr int NR = TileRegs<FK, FV, D, HPC>::NR;
  uint32_t sro[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int rho = score_row<HPC>(j, hn, i);
    sro[i] = (uint32_t)((rho >> a.hp_log2) * a.H + (rho & hp_mask));
  }
  // v_perm selectors that place the bf16 probabilities of column n's rows
  // into the probability operand (slots of other heads' rows get 0): psel[q]
  // builds operand dword q from the packed pair of split_bf16x2.
  uint32_t psel[4] = {0u, 0u, 0u, 0u};
  {
    // move half `from` of a dword to half `to`, zero the other half
    auto half_sel = [](int from, bool to) __attribute__((always_inline)) {
      const uint32_t v = (uint32_t)((2 * from + 1) << 8 | 2 * from);
      return to ? v << 16 | 0x0C0Cu : 0x0C0C0000u | v;
    };
    if constexpr (HPC == 4) {
      // one row per u: row hn of u = q >> 1 sits in the dword q with
      // q & 1 == (INT4: hn & 1; 8-bit: hn >> 1), half (INT4: hn >> 1; 8-bit: hn & 1)
      const int dsel = FV == F_INT4 ? (hn & 1) : (hn >> 1);
      const bool hsel = FV == F_INT4 ? (hn >> 1) : (hn & 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) psel[q] = (q & 1) == dsel ? half_sel(q >> 1, hsel) : 0x0C0C0C0Cu;
    } else if constexpr (HPC == 2 && FV != F_INT4) {
      // rows hn + 2 i of u: dword 2 u + i, half hn (from half i of u's pair)
      psel[0] = half_sel(0, hn);
      psel[1] = half_sel(1, hn);
    }
  }
  f4 acc[VS::NPV];
#pragma unroll
  for (int m = 0; m < VS::NPV; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
  // l_run + l_err: probability sum of the lane's rows, kept with its rounding
  // error (two_sum_acc), one add per tile
  float m_run = -INFINITY, l_run = 0.f, l_err = 0.f;
  float cs_run[NCS];  // sum of the probability operands (hi + lo) of query head n, per value group
#pragma unroll
  for (int g = 0; g < NCS; ++g) cs_run[g] = 0.f;
  // Query operand (B of S^T = K Q^T), loaded at the start of each sequence's
  // piece: lane (j, n) holds query head n's channels of k-slots 8j..8j+7 in
  // the key operand's channel order.
  h8 qop[KS::KB];
  h8 qlo_r[ROTQ ? KS::KB : 1];  // rotated keys: the low half of the rotated query
  bool piece_start = true;
  // KIVI: q * s of the current page (fp16 hi + lo) and q . z, column n's head
  h8 qhi[FK == F_KIVI ? KS::KB : 1], qlo[FK == F_KIVI ? KS::KB : 1];
  float qz = 0.f, kmul = 0.f;  // score = raw kmul + qz

  // Value transpose reads: lane (j, i) points at row T_j[i / 2] of the value
  // tile, byte 8 (i % 2) of the chunk, where T_j[e] = 16 (e / 4) + 4 j + e % 4
  // is the token of k-slot e of lane group j.
  const int trow = 16 * ((n >> 1) >> 2) + 4 * j + ((n >> 1) & 3);
  const int tbase = ST::OFF_V + trow * VS::RB + 8 * (n & 1);
  const int tswz = vswz<VS::CH>(trow);

  // Loads are issued in groups, one per tile y: the block ids of tile y + L,
  // then tile y itself (with the ids loaded L groups earlier).  Every group
  // issues the same loads, tiles past the share's end reload its last tile,
  // so the compiler's load counters are exact and only wait for the tile
  // being stored.  Registers rotate over NS slots: slot (y - x_begin) % NS.
  TileRegs<FK, FV, D, HPC> regs[NS];
  uint64_t live[NS];
  int ids[NS];
  const int x_last = x_end - 1;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int y = min(x_begin + i, x_last);
    seek<FK>(cd, a, y);
    ids[i] = load_ids<OP>(a, cd, y);
  }
  auto load_group = [&](int y, int& ids_out, int ids_in, TileRegs<FK, FV, D, HPC>& r) __attribute__((always_inline)) {
    const int yi = min(y + L, x_last);
    seek<FK>(cd, a, yi);
    ids_out = load_ids<OP>(a, cd, yi);
    const int yc = min(y, x_last);
    seek<FK>(ci, a, yc);
    return load_tile<FK, FV, D, HPC, OP>(a, ids_in, (TILE * (yc - ci.lo)) >> a.hp_log2, ci.lq, h0, sro, r);
  };
#pragma unroll
  for (int i = 0; i < P; ++i) live[i] = load_group(x_begin + i, ids[(i + L) % NS], ids[i], regs[i]);

  // Write the softmax state of sequence b's piece (record share + b) and
  // reset it for the next piece.
  auto write_piece = [&](int b) __attribute__((always_inline)) {
    // remove the value-operand offset and scale factors: with P = 2^60 p s
    // and value operands u 2^-133 (u = c + 128) the true sum is
    // 2^73 acc - 2^-53 cs; INT4 (u = c + 8): even channels 2^73 acc - 2^-57 cs,
    // odd channels (16 u 2^-133) 2^69 acc - 2^-57 cs; cs = sum of the
    // probability operands of query head g
    if constexpr (!VFP8) {
#pragma unroll
      for (int g = 0; g < NCS; ++g) {
        float cs = cs_run[g];
        cs = sum_j(cs);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float csr = __shfl(cs, 4 * j + r);
          if constexpr (FV == F_INT8) {
            const float corr = csr * 0x1p-53f;
#pragma unroll
            for (int m = 0; m < VS::NPV; ++m) acc[m][r] = __builtin_fmaf(acc[m][r], 0x1p73f, -corr);
          } else {
            const float corr = csr * 0x1p-57f;
            acc[2 * g][r] = __builtin_fmaf(acc[2 * g][r], 0x1p73f, -corr);
            acc[2 * g + 1][r] = __builtin_fmaf(acc[2 * g + 1][r], 0x1p69f, -corr);
          }
        }
      }
    }
    float l = sum_j(l_run) + sum_j(l_err);
    const size_t stride = (size_t)D + 2;
    float* pbase = a.part + ((size_t)(share + b) * a.Hq + hq0) * stride;
    if (j == 0 && n < NC) {
      pbase[n * stride] = m_run;
      pbase[n * stride + 1] = l;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * j + r;
      if (g < NC) {
#pragma unroll
        for (int m = 0; m < VS::NPV; ++m) {
          const int ch = FV == F_INT4 ? 32 * (m >> 1) + 2 * n + (m & 1) : 16 * m + n;
          pbase[g * stride + 2 + ch] = acc[m][r];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < VS::NPV; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
    l_err = 0.f;
#pragma unroll
    for (int g = 0; g < NCS; ++g) cs_run[g] = 0.f;
    piece_start = true;
  };

  const int slot = (int)(__builtin_amdgcn_s_getreg((31 << 11) | 4) & 1);  // wave slot on the SIMD (HW_ID bit 0)
  int xr = x_begin;  // first tile of the current round
  // Step S_ of a round: tile x = xr + S_, held in register slot S_.
  auto step = [&](auto stage) __attribute__((always_inline)) {
    constexpr int S_ = decltype(stage)::value;
    const int x = xr + S_;
    // Alternate the issue priority of the SIMD's two wave slots every tile.
    // With equal priorities the older wave wins every issue conflict and
    // finishes its (equal) share about a quarter earlier; the younger one
    // then runs alone with nothing to hide its latencies.
    if ((S_ & 1) ^ slot) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    // ---- start tile x + P ---------------------------------------------------
    live[(S_ + P) % NS] = load_group(x + P, ids[(S_ + P + L) % NS], ids[(S_ + P) % NS], regs[(S_ + P) % NS]);
    if (x >= x_end) return;
    // ---- tile x into LDS ------------------------------------------------------
    uint8_t* cur = s_st;
    store_tile<FK, FV, D, HPC, OP>(regs[S_], cur);
    const uint64_t live_mask = live[S_];
    const uint32_t par = regs[S_].par;
    // ---- first tile of a sequence's piece: its query operand ---------------
    const bool new_piece = piece_start;
    if (piece_start) {
      const uint16_t* qrow = (ROTQ ? a.qrot : a.q) + ((size_t)cc.b * a.Hq + hq0 + (n < NC ? n : 0)) * D;
#pragma unroll
      for (int kb = 0; kb < KS::KB; ++kb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t bits = qrow[key_channel<FK, D>(j, kb, e)];
          qop[kb][e] = __builtin_bit_cast(_Float16, (uint16_t)(n < NC ? bits : 0));
        }
      }
      if constexpr (ROTQ) {
        const uint16_t* qlo = qrow + (size_t)a.B * a.Hq * D;
#pragma unroll
        for (int kb = 0; kb < KS::KB; ++kb) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint16_t bits = qlo[key_channel<FK, D>(j, kb, e)];
            qlo_r[kb][e] = __builtin_bit_cast(_Float16, (uint16_t)(n < NC ? bits : 0));
          }
        }
      }
      piece_start = false;
    }

    // ---- scales -> fp32 (0 for masked tokens); FP8 codes of masked value
    //      rows zeroed (a garbage byte may be a NaN or infinity code)
    // Direct scales: the score rows' scales are in registers (fkf: key scale
    // x sm_scale x log2 e; fvm: value-scale dwords, 0 for masked rows, so a
    // garbage scale never meets a zero probability).
    float fkf[NR];
    uint32_t fvm[NR][TileRegs<FK, FV, D, HPC>::VW];
    if constexpr (DSC) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const bool lv = (live_mask >> score_row<HPC>(j, hn, i)) & 1;
        if constexpr (FK != F_KIVI) fkf[i] = h2f(regs[S_].fk[i]) * a.qscale;
#pragma unroll
        for (int w = 0; w < TileRegs<FK, FV, D, HPC>::VW; ++w) fvm[i][w] = lv ? regs[S_].fv[i][w] : 0u;
      }
    }
    {
      const uint32_t* sdw = reinterpret_cast<const uint32_t*>(cur + ST::OFF_S);
      const int t = lane & 31;
      const bool lv = (live_mask >> t) & 1;
      const bool hi_half = (par >> t) & 1;
      if (!DSC && lane < 32) {
        if constexpr (FK == F_INT4) {
          // row t's key scales, group g at s_fk[t NGK + g]
#pragma unroll
          for (int g = 0; g < KS::NGKD; ++g) {
            const uint32_t d = g == 0 ? sdw[t] : sdw[32 * (1 + ST::NGD) + 32 * (g - 1) + t];
            s_fk[t * KS::NGK + 2 * g] = lv ? h2f(d & 0xFFFFu) * a.qscale : 0.f;
            s_fk[t * KS::NGK + 2 * g + 1] = lv ? h2f(d >> 16) * a.qscale : 0.f;
          }
        } else if constexpr (FK != F_KIVI) {
          const uint32_t d = sdw[t];
          s_fk[t] = lv ? h2f(hi_half ? d >> 16 : d & 0xFFFFu) * a.qscale : 0.f;
        }
      }
      if constexpr (DSC) {
      } else if constexpr (VS::NG == 1) {
        if (lane >= 32) {
          const uint32_t d = sdw[32 + t];
          s_fv[t] = lv ? h2f(hi_half ? d >> 16 : d & 0xFFFFu) * VSC : 0.f;
        }
      } else {
        // value scales of (token t, group g): dword g/2 of the token, half g&1
        // lanes 0..31 take the even dwords of token t, lanes 32..63 the odd ones
#pragma unroll
        for (int gd = 0; gd < VS::NG / 2; ++gd) {
          if ((lane >> 5) == (gd & 1)) {
            const uint32_t d = sdw[32 + 32 * gd + t];
            s_fv[t * VS::NG + 2 * gd] = lv ? h2f(d & 0xFFFFu) * VSC : 0.f;
            s_fv[t * VS::NG + 2 * gd + 1] = lv ? h2f(d >> 16) * VSC : 0.f;
          }
        }
      }
      if constexpr (VFP8) {
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
      if constexpr (FK == F_INT4) {
        // k-block kb is the row's 16-byte chunk kb (scale group kb); lane
        // group j takes its dword j (channels 32 kb + 8 j .. + 7)
#pragma unroll
        for (int kb = 0; kb < KS::KB; ++kb) {
          const int col = kb ^ kswz<CHK>(row);
          kw[u][kb] = *reinterpret_cast<const uint32_t*>(cur + ST::OFF_K + (row * CHK + col) * 16 + 4 * j);
        }
      } else if constexpr (KS::LB >= 16) {
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

    // ---- KIVI: the page's query operand q * s (fp16 hi + lo) and q . z for
    //      column n's head, once per page (a page is HPC tiles).  q * s is
    //      scaled by a power of two F (per column) so that its largest
    //      magnitude times 16 lies in [2^14, 2^15): the fp16 operands neither
    //      overflow nor lose digits to subnormals. --------------------------
    if constexpr (FK == F_KIVI) {
      if (new_piece || ((x - cc.lo) & (HPC - 1)) == 0) {
        qz = 0.f;
        float qs[KS::KB][8];
        float mx = 0.f;
#pragma unroll
        for (int kb = 0; kb < KS::KB; ++kb) {
          const int cb = j * (D / 4) + 8 * kb;
          // fp16 scales and zeros of 8 channels; the products take the fp16
          // operands directly (mixed-precision FMA, exact in fp32)
          const h8 s8 = *reinterpret_cast<const h8*>(cur + ST::OFF_M + 2 * (hn * D + cb));
          const h8 z8 = *reinterpret_cast<const h8*>(cur + ST::OFF_M + 2 * (HPC * D + hn * D + cb));
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ch = key_channel<FK, D>(j, kb, e) - cb;
            qs[kb][e] = __builtin_fmaf((float)qop[kb][e], (float)s8[ch], 0.f);
            mx = fmaxf(mx, fabsf(qs[kb][e]));
            qz = __builtin_fmaf((float)qop[kb][e], (float)z8[ch], qz);
          }
        }
        qz = sum_j(qz);
        qz *= a.qscale;
        mx = max_j(mx);
        // mx < 2^ex; F = 2^(11 - ex), so 16 F mx < 2^15
        const int ex = mx > 0.f ? min(max(__builtin_amdgcn_frexp_expf(mx), -100), 100) : 0;
        const float f_odd = __builtin_ldexpf(1.f, 11 - ex), f_even = 16.f * f_odd;
        // raw = 2^-24 16 F sum n q s
        kmul = a.qscale * __builtin_ldexpf(1.f, 20 - (11 - ex));
#pragma unroll
        for (int kb = 0; kb < KS::KB; ++kb) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // slots e = 2, 3, 6, 7 hold odd channels (16 n 2^-24 keys)
            const float xs = qs[kb][e] * ((e & 2) ? f_odd : f_even);
            const _Float16 hi = (_Float16)xs;
            qhi[kb][e] = hi;
            qlo[kb][e] = (_Float16)__builtin_fmaf((float)hi, -1.0f, xs);  // xs - hi exactly, then rounded
          }
        }
      }
    }

    // ---- scores S^T[t][g] on the matrix cores ------------------------------
    f4 sc[2];
    // INT4 keys: one product per k-block (scale group), scaled per row below
    f4 sck[FK == F_INT4 ? KS::KB : 1][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sc[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KS::KB; ++kb) {
        const h8 kop = key_operand<FK>(kw[u], kb);
        if constexpr (FK == F_INT4) {
          sck[kb][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[kb], f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          if constexpr (ROTQ) sck[kb][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qlo_r[kb], sck[kb][u], 0, 0, 0);
        } else if constexpr (FK == F_KIVI) {
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qhi[kb], sc[u], 0, 0, 0);
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qlo[kb], sc[u], 0, 0, 0);
        } else if constexpr (ROTQ) {
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[kb], sc[u], 0, 0, 0);
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qlo_r[kb], sc[u], 0, 0, 0);
        } else {
          sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[kb], sc[u], 0, 0, 0);
        }
      }
    }
    // lane (j, n): sc[u][r] = raw score of tile row 16u + 4j + r, column n;
    // only rows r = hn + HPC i (i < NU) hold column n's head.
    constexpr int NU = 4 / HPC;
    const uint32_t vmask = (uint32_t)live_mask & colmask;
    float s[2][NU];
    int rows[2][NU];
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int i = 0; i < NU; ++i) {
        const int r = HPC == 1 ? i : hn + HPC * i;
        const int tr = 16 * u + 4 * j + r;
        rows[u][i] = tr;
        auto pick = [&](const f4& x) __attribute__((always_inline)) {
          if constexpr (HPC == 1) return x[i];
          else if constexpr (HPC == 2) return hn ? x[2 * i + 1] : x[2 * i];
          else {
            const float r01 = (hn & 1) ? x[1] : x[0];
            const float r23 = (hn & 1) ? x[3] : x[2];
            return (hn & 2) ? r23 : r01;
          }
        };
        const float raw = FK == F_INT4 ? 0.f : pick(sc[u]);
        float v;
        if constexpr (FK == F_INT4) {
          v = 0.f;
#pragma unroll
          for (int kb = 0; kb < KS::KB; ++kb) v = __builtin_fmaf(pick(sck[kb][u]), s_fk[tr * KS::NGK + kb], v);
        } else if constexpr (FK == F_KIVI) v = __builtin_fmaf(raw, kmul, qz);
        else if constexpr (DSC) v = raw * fkf[u * NU + i];
        else v = raw * s_fk[tr];
        // a masked row's key codes may be anything, and a row of another KV
        // head than column n's does not belong to it: select, don't multiply
        v = ((vmask >> tr) & 1) ? v : -INFINITY;
        s[u][i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = max_j(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    // Rescale only when some head's running max moved (rare after the first
    // tiles): alpha = 2^(m_old - m_new).
    if (__ballot(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 0 on the first live tile
      l_run *= alpha;
      l_err *= alpha;
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
    float p[2][NU];
    float lt = 0.f;  // this tile's sum
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int i = 0; i < NU; ++i) {
        p[u][i] = __builtin_amdgcn_exp2f(s[u][i] - m_use);  // exp2(-inf) = 0 for masked rows
        lt += p[u][i];
      }
    }
    two_sum_acc(l_run, l_err, lt);

    // ---- P V on the matrix cores -------------------------------------------
    // Probability operand of lane (j, n): 8 k-slots (tile rows T_j[e]) of
    // column n times the value scale, as bf16 hi + lo; slots of rows of other
    // heads are 0.  Value operands hold exact codes, biased to non-negative
    // for INT8/INT4; the bias times the probability sum is removed once,
    // after the last tile (cs_run).
    auto place = [](uint32_t b, uint32_t sel) __attribute__((always_inline)) { return __builtin_amdgcn_perm(b, b, sel); };
    // p x value scale of score row (u, i), group grp (x 2^60 for the INT8 /
    // INT4 operands; 0 for masked rows), one rounding: with direct scales the
    // fp16 scale is an operand of a mixed-precision FMA
    float pv[2][NU];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < NU; ++i) pv[u][i] = p[u][i] * VSC;
    auto pvs = [&](int u, int i, int grp) __attribute__((always_inline)) {
      if constexpr (DSC) {
        const uint32_t d = fvm[u * NU + i][VS::NG == 1 ? 0 : grp >> 1];
        const uint16_t h = (uint16_t)((VS::NG > 1 && (grp & 1)) ? d >> 16 : d & 0xFFFFu);
        return __builtin_fmaf(pv[u][i], (float)__builtin_bit_cast(_Float16, h), 0.f);
      } else {
        return p[u][i] * s_fv[rows[u][i] * VS::NG + grp];
      }
    };
    if constexpr (FV == F_INT4) {
      // dword q holds slots (q >> 1) 4 + (q & 1) (rows r = q & 1, low half) and
      // that + 2 (r = (q & 1) + 2, high half) of u = q >> 1 (value_operand_int4)
#pragma unroll
      for (int grp = 0; grp < VS::NG; ++grp) {
        uint32_t ah[4], al[4];
        float cst = 0.f;  // this tile's operand sum (a short chain, see add_split)
        if constexpr (HPC == 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int u = q >> 1, r0 = q & 1;
            split_bf16x2(f2{p[u][r0] * s_fv[rows[u][r0] * VS::NG + grp],
                            p[u][r0 + 2] * s_fv[rows[u][r0 + 2] * VS::NG + grp]},
                         ah[q], al[q]);
            cst = add_split(cst, ah[q], al[q]);
          }
        } else if constexpr (HPC == 2) {
          // rows hn, hn + 2 of u share dword 2 u + hn
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            uint32_t h, l;
            split_bf16x2(f2{pvs(u, 0, grp), pvs(u, 1, grp)}, h, l);
            cst = add_split(cst, h, l);
            ah[2 * u] = hn ? 0u : h;
            ah[2 * u + 1] = hn ? h : 0u;
            al[2 * u] = hn ? 0u : l;
            al[2 * u + 1] = hn ? l : 0u;
          }
        } else {
          // row hn of u: dword 2 u + (hn & 1), half hn >> 1 (psel)
          uint32_t h, l;
          split_bf16x2(f2{pvs(0, 0, grp), pvs(1, 0, grp)}, h, l);
          cst = add_split(cst, h, l);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            ah[q] = place(h, psel[q]);
            al[q] = place(l, psel[q]);
          }
        }
        cs_run[grp] += cst;
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
      // dword q holds slots 2q, 2q + 1: rows r = 2 (q & 1), 2 (q & 1) + 1 of u = q >> 1
      uint32_t ah[4], al[4];
      float cst = 0.f;  // this tile's operand sum (a short chain, see add_split)
      if constexpr (HPC == 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = q >> 1, r0 = 2 * (q & 1);
          split_bf16x2(f2{p[u][r0] * s_fv[rows[u][r0]], p[u][r0 + 1] * s_fv[rows[u][r0 + 1]]}, ah[q], al[q]);
          if constexpr (FV == F_INT8) cst = add_split(cst, ah[q], al[q]);
        }
      } else if constexpr (HPC == 2) {
        // row hn + 2 i of u: dword 2 u + i, half hn
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t h, l;
          split_bf16x2(f2{pvs(u, 0, 0), pvs(u, 1, 0)}, h, l);
          if constexpr (FV == F_INT8) cst = add_split(cst, h, l);
          ah[2 * u] = place(h, psel[0]);
          ah[2 * u + 1] = place(h, psel[1]);
          al[2 * u] = place(l, psel[0]);
          al[2 * u + 1] = place(l, psel[1]);
        }
      } else {
        // row hn of u: dword 2 u + (hn >> 1), half hn & 1
        uint32_t h, l;
        split_bf16x2(f2{pvs(0, 0, 0), pvs(1, 0, 0)}, h, l);
        if constexpr (FV == F_INT8) cst = add_split(cst, h, l);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ah[q] = place(h, psel[q]);
          al[q] = place(l, psel[q]);
        }
      }
      if constexpr (FV == F_INT8) cs_run[0] += cst;
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
    // ---- last tile of the piece: write its softmax state ---------------------
    if (x + 1 == x_end || x + 1 == cc.hi) {
      write_piece(cc.b);
      if (x + 1 < x_end) seek<FK>(cc, a, x + 1);
    }
  };
  auto round = [&]<int... I>(std::integer_sequence<int, I...>) __attribute__((always_inline)) {
    (step(std::integral_constant<int, I>{}), ...);
  };
  for (; xr < x_end; xr += NS) round(std::make_integer_sequence<int, NS>{});
}

// Merge the pieces of one (sequence, query head): M = max m_r,
// out = sum_r acc_r 2^(m_r - M) / sum_r l_r 2^(m_r - M), rounded to fp16.
// Sequence b's tiles [P_b, P_b+1) lie in shares P_b / S .. (P_b+1 - 1) / S,
// whose pieces are records share + b.  For KIVI keys the last ctx_len % 32
// tokens (fp16 keys and values in tail row b) are one more piece, computed
// here by wave 0 in plain fp32.  MW waves share the records (16 when the
// grid is small, so a few long record lists still fill the GPU); lanes own
// channels.  One pass: each wave loads its records once and combines them
// against its own maximum; the waves' partial sums are then combined against
// the overall maximum (the same sums, grouped by wave).
template <int D, bool KIVI, int MERGE_WAVES>
__global__ __launch_bounds__(MERGE_WAVES * 64) void merge_kernel(DecodeArgs a) {
  constexpr int CPL = D / 64;
  __shared__ float s_m[MERGE_WAVES];
  __shared__ float s_acc[MERGE_WAVES][D + 1];
  __shared__ float s_tail[D + 2];  // KIVI tail piece: m, l, acc[D]
  const int bh = (int)blockIdx.x, tid = (int)threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int b = bh / a.Hq, hq = bh - b * a.Hq;
  // Data errors of sequence b: a context length outside [0, the tokens its
  // block-table row addresses] (clamped), or a block id outside
  // [0, num_blocks) on a page the split kernel reads (left out there).  The
  // Hq workgroups of the sequence check every Hq-th page each; the ids load
  // with the records and are reported at the end.
  bool bad_id = false, bad_ctx = false;
  {
    const int cap = a.max_blocks << a.log2_bs;
    const int raw = a.ctx_lens[b];
    const int L = min(max(raw, 0), cap);
    const int np = ((KIVI ? (L & ~31) : L) + a.bs - 1) >> a.log2_bs;
    for (int p = hq + a.Hq * tid; p < np; p += a.Hq * MERGE_WAVES * 64) {
      const int id = a.block_table[(size_t)b * a.max_blocks + p];
      bad_id |= id < 0 || id >= a.nb;
    }
    bad_ctx = hq == 0 && tid == 0 && (raw < 0 || raw > cap);
  }
  int S, t0, t1;
  if (a.inline_plan) {
    int lq, nt, excl;
    const int total = wave_plan<KIVI ? F_KIVI : F_INT8>(a, lq, nt, excl);
    S = share_size(a, total);
    t0 = rdlane(excl, b);
    t1 = t0 + rdlane(nt, b);
  } else {
    S = a.plan[0];
    t0 = a.plan[1 + b];
    t1 = a.plan[2 + b];
  }
  const int first = t1 > t0 ? t0 / S : 0;
  const int nrec = t1 > t0 ? (t1 - 1) / S - first + 1 : 0;
  const size_t stride = (size_t)D + 2;
  auto rec = [&](int i) -> const float* { return a.part + ((size_t)(first + i + b) * a.Hq + hq) * stride; };
  float tm = -INFINITY;  // the tail piece's max (KIVI)
  if constexpr (KIVI) {
    if (w == 0) {
      const int L = min(max(a.ctx_lens[b], 0), a.max_blocks * 32);
      const int nt = b < a.max_seqs ? (L & 31) : 0;  // tail rows exist only for b < max_seqs
      const int h = hq / a.G;
      const uint16_t* qrow = a.q + ((size_t)b * a.Hq + hq) * D;
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
      if (lane == 0) {
        s_tail[0] = mx;
        s_tail[1] = l;
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) s_tail[2 + lane * CPL + c] = accv[c];
    }
    __syncthreads();
    tm = s_tail[0];
  }
  float tailv[CPL];  // rotated values: the KIVI tail's weighted values (wave 0)
#pragma unroll
  for (int c = 0; c < CPL; ++c) tailv[c] = 0.f;
  // this wave's records (i = w, w + MW, ...), combined against their maximum
  // Mw (the KIVI tail joins wave 0's)
  constexpr int RB = 8;  // records loaded per batch
  float Mw = w == 0 ? tm : -INFINITY;
  float accv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) accv[c] = 0.f;
  float l = 0.f;
  for (int i0 = w; i0 < nrec; i0 += RB * MERGE_WAVES) {
    float ms[RB], ls[RB], av[RB][CPL];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int i = i0 + k * MERGE_WAVES;
      const float* p = rec(i < nrec ? i : 0);
      ms[k] = i < nrec ? p[0] : -INFINITY;
      ls[k] = p[1];
#pragma unroll
      for (int c = 0; c < CPL; ++c) av[k][c] = p[2 + lane * CPL + c];
    }
    float mb = Mw;
#pragma unroll
    for (int k = 0; k < RB; ++k) mb = fmaxf(mb, ms[k]);
    if (mb == -INFINITY) continue;
    // rescale what the wave holds to the new maximum
    const float r = Mw == -INFINITY ? 0.f : exp2f(Mw - mb);
    l *= r;
#pragma unroll
    for (int c = 0; c < CPL; ++c) accv[c] *= r;
    Mw = mb;
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const float wgt = ms[k] == -INFINITY ? 0.f : exp2f(ms[k] - mb);
      l = __builtin_fmaf(ls[k], wgt, l);
#pragma unroll
      for (int c = 0; c < CPL; ++c) accv[c] = __builtin_fmaf(av[k][c], wgt, accv[c]);
    }
  }
  if (lane == 0) s_m[w] = Mw;
#pragma unroll
  for (int c = 0; c < CPL; ++c) s_acc[w][lane * CPL + c] = accv[c];
  if (lane == 0) s_acc[w][D] = l;
  report_error(a.err, bad_id, KVQ_DEVERR_BLOCK);
  report_error(a.err, bad_ctx, KVQ_DEVERR_CTX);
  __syncthreads();
  if (w != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < MERGE_WAVES; ++i) M = fmaxf(M, s_m[i]);
  float wg[MERGE_WAVES];
  float lt = 0.f;
#pragma unroll
  for (int i = 0; i < MERGE_WAVES; ++i) {
    wg[i] = s_m[i] == -INFINITY ? 0.f : exp2f(s_m[i] - M);
    lt = __builtin_fmaf(s_acc[i][D], wg[i], lt);
  }
  float v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    v[c] = 0.f;
#pragma unroll
    for (int i = 0; i < MERGE_WAVES; ++i) v[c] = __builtin_fmaf(s_acc[i][lane * CPL + c], wg[i], v[c]);
  }
  if (KIVI && tm != -INFINITY) {
    const float wgt = exp2f(tm - M);
    lt = __builtin_fmaf(s_tail[1], wgt, lt);
    // the tail holds the original (unrotated) values: with rotated values
    // it joins after the pages' sum is rotated back
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float t = s_tail[2 + lane * CPL + c] * wgt;
      if (a.rot_v) tailv[c] = t;
      else v[c] += t;
    }
  }
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  uint16_t* o = a.out + (size_t)bh * D;
  if (a.rot_v) {
    // values stored rotated (y = H (sigma x)): the weighted sum of the stored
    // rows is rotated back, x = sigma (H y) / D, in fp32.  Channel c = lane
    // CPL + i: its low bits are inside the lane, the lane bits above them.
#pragma unroll
    for (int s = 1; s < CPL; s <<= 1) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        if (i & s) continue;
        const float x0 = v[i], x1 = v[i + s];
        v[i] = x0 + x1;
        v[i + s] = x0 - x1;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const float p = __shfl_xor(v[i], m);
        v[i] = (lane & m) ? p - v[i] : v[i] + p;
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane * CPL + i;
      uint32_t wd = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) wd = (c >> 5) == k ? a.rot_signs[k] : wd;
      v[i] = (((wd >> (c & 31)) & 1) ? -v[i] : v[i]) * (1.0f / D) + tailv[i];
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[lane * CPL + c] = (uint16_t)f2h_bits(v[c] * inv);
}

// The partition of one call: tiles per sequence, their prefix sums, the
// share size S and the sequence holding each share's first tile (plan
// layout in DecodeArgs).  One workgroup; sequences in chunks of 1024.
constexpr int PLAN_THREADS = 1024;

template <bool KIVI>
__device__ __forceinline__ int seq_tiles(const DecodeArgs& a, int b) {
  const int L = min(max(a.ctx_lens[b], 0), a.max_blocks << a.log2_bs);
  const int Lq = KIVI ? (L & ~31) : L;
  const int tt = TILE >> a.hp_log2;  // tokens per tile
  return (Lq + tt - 1) / tt;
}

// Exclusive prefix sum over the workgroup; returns the workgroup total.
__device__ __forceinline__ int block_scan(int v, int& excl, int* s_tot) {
  const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) s_tot[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < PLAN_THREADS / 64; ++i) {
    before += i < w ? s_tot[i] : 0;
    all += s_tot[i];
  }
  __syncthreads();  // s_tot is reused by the next chunk
  excl = before + incl - v;
  return all;
}

template <bool KIVI>
__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(DecodeArgs a) {
  __shared__ int s_tot[PLAN_THREADS / 64];
  const int tid = (int)threadIdx.x;
  int* pre = a.plan + 1;
  int carry = 0;
  for (int c = 0; c < a.B; c += PLAN_THREADS) {
    const int b = c + tid;
    const int n = b < a.B ? seq_tiles<KIVI>(a, b) : 0;
    int excl;
    const int all = block_scan(n, excl, s_tot);
    if (b < a.B) pre[b] = carry + excl;
    carry += all;
  }
  const int total = carry;
  int S = a.share_tiles;
  if (S <= 0) S = max((total + a.num_shares - 1) / a.num_shares, AUTO_MIN_TILES);
  if (tid == 0) {
    pre[a.B] = total;
    a.plan[0] = S;
  }
  // share i starts in the sequence whose tiles [P_b, P_b + n_b) hold i S
  int* first = a.plan + 2 + a.B;
  carry = 0;
  for (int c = 0; c < a.B; c += PLAN_THREADS) {
    const int b = c + tid;
    const int n = b < a.B ? seq_tiles<KIVI>(a, b) : 0;
    int excl;
    const int all = block_scan(n, excl, s_tot);
    const int p = carry + excl;
    if (n > 0) {
      const int i1 = min((p + n + S - 1) / S, a.num_shares);
      for (int i = (p + S - 1) / S; i < i1; ++i) first[i] = b;
    }
    carry += all;
  }
}

namespace {

// Waves of decode_split_kernel<FK, FV, D> to run at once on the current
// device in workgroups of nw waves: WPE per SIMD (4 WPE per compute unit),
// or the occupancy if lower.  Every wave gets the same work, so a SIMD
// holding more waves than the others would hold the whole launch back.
// Cached per device and nw.
template <int FK, int FV, int D, int HPC, bool OP, bool ROTQ>
int resident_waves(int nw) {
  constexpr int MAXW = 4 * Stage<FK, FV, D>::WPE;
  static std::atomic<int> cache[64][MAXW + 1];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || nw < 1 || nw > MAXW) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev][nw].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<FK, FV, D, HPC, OP, ROTQ>, 64 * nw,
                                                   (size_t)nw * Stage<FK, FV, D>::WAVE_LDS) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int w = std::min(per_cu * nw, MAXW) * cus;
  if (dev >= 0 && dev < 64 && w > 0) cache[dev][nw].store(w, std::memory_order_relaxed);
  return w;
}

template <int FK, int FV, int D, int HPC, bool OP, bool ROTQ>
hipError_t launch4(DecodeArgs a, hipStream_t st) {
  // Waves per workgroup: the largest divisor of the share's head groups that
  // fits on one compute unit (4 WPE waves).  Putting a share's head groups
  // on one compute unit measured 4.5% (FP8, 4 heads per wave) to 11% (INT8,
  // 2 heads per wave) faster than one wave per workgroup.
  const int groups = a.H >> a.hp_log2;
  int nw = std::min(groups, 4 * Stage<FK, FV, D>::WPE);
  while (groups % nw) --nw;
  if (a.share_tiles <= 0) {
    // balanced: all waves the same length, all resident at once
    const int w = resident_waves<FK, FV, D, HPC, OP, ROTQ>(nw);
    if (w <= 0) return hipErrorInvalidDevice;
    a.num_shares = min(a.max_shares, max(1, w / (a.H >> a.hp_log2)));
  } else {
    a.num_shares = a.max_shares;
  }
  // Up to 64 sequences, every wave derives the plan from ctx_lens itself.
  a.inline_plan = a.B <= 64 ? 1 : 0;
  hipError_t e;
  if (!a.inline_plan) {
    hipLaunchKernelGGL((plan_kernel<FK == F_KIVI>), dim3(1), dim3(PLAN_THREADS), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // one wave per (share, group of HP KV heads), nw waves per workgroup; see
  // decode_split_kernel for the order
  const uint32_t wgs = (((uint32_t)a.num_shares + 7) / 8) * 8 * (uint32_t)(groups / nw);
  const size_t lds = (size_t)nw * Stage<FK, FV, D>::WAVE_LDS;
  hipLaunchKernelGGL((decode_split_kernel<FK, FV, D, HPC, OP, ROTQ>), dim3(wgs), dim3(64 * nw), lds, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.B * a.Hq < 512)
    hipLaunchKernelGGL((merge_kernel<D, FK == F_KIVI, 16>), dim3((unsigned)(a.B * a.Hq)), dim3(16 * 64), 0, st, a);
  else
    hipLaunchKernelGGL((merge_kernel<D, FK == F_KIVI, 4>), dim3((unsigned)(a.B * a.Hq)), dim3(4 * 64), 0, st, a);
  return hipGetLastError();
}

template <int FK, int FV, int D, bool ROTQ>
hipError_t launch3(const DecodeArgs& a, hipStream_t st) {
  // (INT4 keys: the general path, whose scales pass through LDS)
  constexpr bool OP_PAYS = (FV == F_INT4 || FK == F_KIVI) && FK != F_INT4;
  switch (a.hp_log2) {
    // Tiles of 32 / HP tokens lie in one page when the page holds at least
    // that many (always for HP = 4: block_size >= 8).  The one-page address
    // path saves about a sixth of the VALU work per tile, which pays where
    // that work bounds the kernel (4-bit values, KIVI keys); with 8-bit keys
    // and values it measured 1-2% slower, so those keep the general path.
    case 0:
      return OP_PAYS && a.bs >= 32 ? launch4<FK, FV, D, 1, OP_PAYS, ROTQ>(a, st)
                                   : launch4<FK, FV, D, 1, false, ROTQ>(a, st);
    case 1:
      return OP_PAYS && a.bs >= 16 ? launch4<FK, FV, D, 2, OP_PAYS, ROTQ>(a, st)
                                   : launch4<FK, FV, D, 2, false, ROTQ>(a, st);
    case 2: return launch4<FK, FV, D, 4, OP_PAYS, ROTQ>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int FK, int FV, bool ROTQ>
hipError_t by_dim(int D, const DecodeArgs& a, hipStream_t s) {
  switch (D) {
    case 64: return launch3<FK, FV, 64, ROTQ>(a, s);
    case 128: return launch3<FK, FV, 128, ROTQ>(a, s);
    case 256: return launch3<FK, FV, 256, ROTQ>(a, s);
  }
  return hipErrorInvalidValue;
}

// Decode launch for key format FK and any value format (one instantiation
// per translation unit kvq_decode_k*.hip).
template <int FK, bool ROTQ>
hipError_t decode_for_keys(int fv, int D, const DecodeArgs& a, hipStream_t s) {
  switch (fv) {
    case F_INT8: return by_dim<FK, F_INT8, ROTQ>(D, a, s);
    case F_FP8: return by_dim<FK, F_FP8, ROTQ>(D, a, s);
    case F_INT4: return by_dim<FK, F_INT4, ROTQ>(D, a, s);
    case F_E5M2: return by_dim<FK, F_E5M2, ROTQ>(D, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

}  // namespace kvq
