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
constexpr int MAX_PPS = 512;  // pages per split (block-table slice in LDS)

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
  const uint32_t a = (d & 0xFFu) | ((d & 0xFF00u) << 8) | 0x64006400u;
  const uint32_t b = ((d >> 16) & 0xFFu) | ((d >> 8) & 0xFF0000u) | 0x64006400u;
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = h2_bits(as_h2(a) - bias);
  hi = h2_bits(as_h2(b) - bias);
}
// FP8 E4M3FN -> fp32 (exact) -> fp16 (exact: every E4M3FN value is an fp16
// value, so round-toward-zero packing is exact).
__device__ __forceinline__ void fp8_to_h4(uint32_t d, uint32_t& lo, uint32_t& hi) {
  const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, false);
  const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, true);
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f01[0], f01[1]));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f23[0], f23[1]));
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
  return (__builtin_bit_cast(uint32_t, a) >> 16) | (__builtin_bit_cast(uint32_t, b) & 0xFFFF0000u);
}

template <int FV>
__device__ __forceinline__ b8 value_operand_8bit(i2 t) {
  const uint32_t d0 = (uint32_t)t.x, d1 = (uint32_t)t.y;
  u4 r;
  if constexpr (FV == F_FP8) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)d0, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)d0, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)d1, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)d1, true);
    r.x = bf16_pair_hi(a[0], a[1]);
    r.y = bf16_pair_hi(b[0], b[1]);
    r.z = bf16_pair_hi(c[0], c[1]);
    r.w = bf16_pair_hi(d[0], d[1]);
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

// x = hi + lo with hi = bf16_rne(x), lo = bf16_rne(x - hi).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo, float& used) {
  hi = (__bf16)x;
  const float fh = (float)hi;
  lo = (__bf16)(x - fh);
  used = fh + (float)lo;
}

template <int FK, int FV, int D>
__global__ __launch_bounds__(MAX_WAVES * 64) void decode_split_kernel(DecodeArgs a) {
  using KS = KShape<FK, D>;
  using VS = VShape<FV, D>;
  __shared__ int32_t s_blk[MAX_PPS];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[MAX_WAVES][TILE * VS::RBP];
  __shared__ float s_sk[MAX_WAVES][TILE];
  __shared__ float s_sv[MAX_WAVES][TILE * VS::NG];

  const int split = (int)blockIdx.x, b = (int)blockIdx.z;
  const int nw = (int)(blockDim.x >> 6);
  const int w = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int h = (int)blockIdx.y * nw + w;
  const int j = lane >> 4, n = lane & 15;
  const int bs = a.bs;
  // ctx_len is clamped to what the block-table row can address
  const int L = min(max(a.ctx_lens[b], 0), a.max_blocks * bs);
  const int Lq = FK == F_KIVI ? (L & ~31) : L;  // tokens held in quantized pages
  const int npages = (Lq + bs - 1) / bs;
  const int p0 = split * a.pages_per_split;
  const int p1 = min(npages, p0 + a.pages_per_split);
  for (int i = (int)threadIdx.x; i < p1 - p0; i += (int)blockDim.x)
    s_blk[i] = a.block_table[(size_t)b * a.max_blocks + p0 + i];
  __syncthreads();
  if (h >= a.H) return;  // no barrier below this point

  const int G = a.G;
  const int hq0 = h * G;
  f4 acc[VS::NPV];
#pragma unroll
  for (int m = 0; m < VS::NPV; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Query operand (B of S^T = K Q^T): lane (j, n) holds query head n's
  // channels of k-slots 8j..8j+7 in the key operand's channel order.
  const uint16_t* qrow = a.q + ((size_t)b * a.Hq + hq0 + n) * D;
  h8 qop[KS::KB];
#pragma unroll
  for (int kb = 0; kb < KS::KB; ++kb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t bits = n < G ? qrow[key_channel<FK, D>(j, kb, e)] : (uint16_t)0;
      qop[kb][e] = __builtin_bit_cast(_Float16, bits);
    }
  }

  uint8_t* sv = s_v[w];
  const int tok_begin = p0 * bs, tok_end = min(Lq, p1 * bs);
  for (int t0 = tok_begin; t0 < tok_end; t0 += TILE) {
    // ---- keys of the tile: lane (j, n) reads a quarter row of tokens n, 16+n
    uint32_t kw[2][KS::NW];
    bool kvalid[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tt = t0 + 16 * u + n;
      const int pg = tt / bs;
      int blk = -1;
      if (tt < tok_end) blk = s_blk[pg - p0];
      kvalid[u] = blk >= 0 && blk < a.nb;
      const uint8_t* src = a.k_codes + (((size_t)(kvalid[u] ? blk : 0) * bs + (tt - pg * bs)) * a.H + h) * KS::RB +
                           j * KS::LB;
#pragma unroll
      for (int i = 0; i < KS::NW; i += 4) {
        if constexpr (KS::NW >= 4) {
          u4 v = kvalid[u] ? *reinterpret_cast<const u4*>(src + 4 * i) : u4{0u, 0u, 0u, 0u};
          kw[u][i] = v.x; kw[u][i + 1] = v.y; kw[u][i + 2] = v.z; kw[u][i + 3] = v.w;
        }
      }
      if constexpr (KS::NW == 2) {
        u2 v = kvalid[u] ? *reinterpret_cast<const u2*>(src) : u2{0u, 0u};
        kw[u][0] = v.x; kw[u][1] = v.y;
      }
    }
    // ---- values of the tile -> LDS (zeros for masked rows) ---------------
#pragma unroll
    for (int i = 0; i < VS::NL; ++i) {
      const int c = lane + 64 * i;
      const int r = c / VS::CH, col = c % VS::CH;
      const int tt = t0 + r;
      const int pg = tt / bs;
      int blk = -1;
      if (tt < tok_end) blk = s_blk[pg - p0];
      u4 v = {0u, 0u, 0u, 0u};
      if (blk >= 0 && blk < a.nb)
        v = *reinterpret_cast<const u4*>(a.v_codes + (((size_t)blk * bs + (tt - pg * bs)) * a.H + h) * VS::RB +
                                         col * 16);
      *reinterpret_cast<u4*>(sv + r * VS::RBP + col * 16) = v;
    }
    // ---- per-token scales -> LDS (0 for masked rows); live-token mask ----
    uint64_t live_mask;
    {
      const int r = lane & 31;
      const int tt = t0 + r;
      const int pg = tt / bs;
      int blk = -1;
      if (tt < tok_end) blk = s_blk[pg - p0];
      const bool ok = blk >= 0 && blk < a.nb;
      live_mask = __ballot(ok);  // bit r: token t0 + r is in the context and its block id is valid
      const size_t row = ((size_t)(ok ? blk : 0) * bs + (tt - pg * bs)) * a.H + h;
      if (lane < 32) {
        if constexpr (FK != F_KIVI) s_sk[w][r] = ok ? h2f(a.k_scales[row]) : 0.f;
      } else {
#pragma unroll
        for (int g = 0; g < VS::NG; ++g) s_sv[w][r * VS::NG + g] = ok ? h2f(a.v_scales[row * VS::NG + g]) : 0.f;
      }
    }

    // ---- KIVI: per-page query operand q * s (fp16 hi + lo) and q . z ------
    h8 qhi[KS::KB], qlo[KS::KB];
    float qz = 0.f;
    if constexpr (FK == F_KIVI) {
      const int blk = s_blk[t0 / bs - p0];  // one page per tile (bs == 32)
      const bool ok = blk >= 0 && blk < a.nb;
      const size_t mrow = ((size_t)(ok ? blk : 0) * a.H + h) * D;
#pragma unroll
      for (int kb = 0; kb < KS::KB; ++kb) {
        // scales and zeros of the k-block's 8 channels: one 16-byte load each
        const size_t cb = mrow + j * (D / 4) + 8 * kb;
        const u4 sw = ok ? *reinterpret_cast<const u4*>(a.k_scales + cb) : u4{0u, 0u, 0u, 0u};
        const u4 zw = ok ? *reinterpret_cast<const u4*>(a.k_zeros + cb) : u4{0u, 0u, 0u, 0u};
        float s8[8], z8[8];
        unpack8(uint4{sw.x, sw.y, sw.z, sw.w}, s8);
        unpack8(uint4{zw.x, zw.y, zw.z, zw.w}, z8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ch = key_channel<FK, D>(j, kb, e) - (j * (D / 4) + 8 * kb);
          const float qv = (float)qop[kb][e];
          const float s = s8[ch];
          const float z = z8[ch];
          const float qs = qv * s;
          const _Float16 hi = (_Float16)qs;
          qhi[kb][e] = hi;
          qlo[kb][e] = (_Float16)(qs - (float)hi);
          qz = __builtin_fmaf(qv, z, qz);
        }
      }
      qz += __shfl_xor(qz, 16);
      qz += __shfl_xor(qz, 32);
    }

    // ---- scores S^T[t][g] on the matrix cores ----------------------------
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
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 16 * u + 4 * j + r;
        const bool live = (live_mask >> tr) & 1;
        float v;
        if constexpr (FK == F_KIVI) v = (sc[u][r] + qz) * a.qscale;
        else v = sc[u][r] * s_sk[w][tr] * a.qscale;
        // a masked row's key codes may be anything: select, don't multiply
        v = live ? v : -INFINITY;
        s[4 * u + r] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);  // 0 on the first live tile
    m_run = m_new;
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(s[e] - m_use);
      psum += p[e];
    }
    l_run = l_run * alpha + psum;
    // rescale the accumulator: lane (j, n) holds query heads 4j + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * j + r);
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m) acc[m][r] *= ar;
    }

    // ---- P V on the matrix cores -----------------------------------------
    // Token of k-slot e for lane group j: T_j[e] = 16 (e / 4) + 4 j + e % 4.
    // tr8 addresses: lane (j, i) points at row T_j[i / 2], byte offset
    // c0 + 8 (i % 2); lane (j, n) then receives byte c0 + n of the 8 rows.
    const int trow = 16 * ((n >> 1) >> 2) + 4 * j + ((n >> 1) & 3);
    const lds_u8* vbase = (const lds_u8*)(sv + trow * VS::RBP + 8 * (n & 1));
    if constexpr (FV == F_INT4) {
#pragma unroll
      for (int grp = 0; grp < VS::NG; ++grp) {
        __bf16 ah[8], al[8];
        float cs = 0.f;
        constexpr int ord[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int slot = ord[e];
          const int tr = 16 * (slot >> 2) + 4 * j + (slot & 3);
          float used;
          split_bf16(p[slot] * s_sv[w][tr * VS::NG + grp], ah[e], al[e], used);
          cs += used;
        }
        b8 A_hi, A_lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) { A_hi[e] = ah[e]; A_lo[e] = al[e]; }
        const i2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(vbase + 16 * grp));
        b8 ve, vo;
        value_operand_int4(raw, ve, vo);
        // corr[g] = 136 * sum of the operand values of query head g
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
        acc[2 * grp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, ve, acc[2 * grp], 0, 0, 0);
        acc[2 * grp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, ve, acc[2 * grp], 0, 0, 0);
        acc[2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, vo, acc[2 * grp + 1], 0, 0, 0);
        acc[2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, vo, acc[2 * grp + 1], 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float corr = 136.f * __shfl(cs, 4 * j + r);
          acc[2 * grp][r] -= corr;
          acc[2 * grp + 1][r] -= corr;
        }
      }
    } else {
      b8 A_hi, A_lo;
      float cs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tr = 16 * (e >> 2) + 4 * j + (e & 3);
        __bf16 hi, lo;
        float used;
        split_bf16(p[e] * s_sv[w][tr], hi, lo, used);
        A_hi[e] = hi;
        A_lo[e] = lo;
        cs += used;
      }
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m) {
        const i2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(vbase + 16 * m));
        const b8 vop = value_operand_8bit<FV>(raw);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_hi, vop, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_lo, vop, acc[m], 0, 0, 0);
      }
      if constexpr (FV == F_INT8) {
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float corr = 128.f * __shfl(cs, 4 * j + r);
#pragma unroll
          for (int m = 0; m < VS::NPV; ++m) acc[m][r] -= corr;
        }
      }
    }
  }

  // ---- write this split's softmax state ----------------------------------
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
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(DecodeArgs a) {
  const int bh = (int)blockIdx.x, lane = (int)threadIdx.x;
  constexpr int CPL = D / 64;
  const size_t stride = (size_t)D + 2;
  const float* base = a.part + (size_t)bh * a.num_splits * stride;
  float M = -INFINITY;
  for (int s = 0; s < a.num_splits; ++s) M = fmaxf(M, base[s * stride]);
  float accv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) accv[c] = 0.f;
  float l = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.num_splits; ++s) {
      const float ms = base[s * stride];
      if (ms == -INFINITY) continue;
      const float wgt = exp2f(ms - M);
      l = __builtin_fmaf(base[s * stride + 1], wgt, l);
#pragma unroll
      for (int c = 0; c < CPL; ++c) accv[c] = __builtin_fmaf(base[s * stride + 2 + lane * CPL + c], wgt, accv[c]);
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint16_t* o = a.out + (size_t)bh * D;
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[lane * CPL + c] = (uint16_t)f2h_bits(accv[c] * inv);
}

namespace {

template <int FK, int FV, int D>
hipError_t launch3(const DecodeArgs& a, int nw, hipStream_t st) {
  const int quant_splits = a.num_splits - (FK == F_KIVI ? 1 : 0);
  const dim3 grid((unsigned)quant_splits, (unsigned)((a.H + nw - 1) / nw), (unsigned)a.B);
  hipLaunchKernelGGL((decode_split_kernel<FK, FV, D>), grid, dim3(nw * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (FK == F_KIVI) {
    hipLaunchKernelGGL((kivi_tail_kernel<D>), dim3((unsigned)a.B, (unsigned)a.H), dim3(64), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int FK, int FV>
hipError_t by_dim(int D, const DecodeArgs& a, int nw, hipStream_t s) {
  switch (D) {
    case 64: return launch3<FK, FV, 64>(a, nw, s);
    case 128: return launch3<FK, FV, 128>(a, nw, s);
    case 256: return launch3<FK, FV, 256>(a, nw, s);
  }
  return hipErrorInvalidValue;
}

template <int FK>
hipError_t by_v(int fv, int D, const DecodeArgs& a, int nw, hipStream_t s) {
  switch (fv) {
    case F_INT8: return by_dim<FK, F_INT8>(D, a, nw, s);
    case F_FP8: return by_dim<FK, F_FP8>(D, a, nw, s);
    case F_INT4: return by_dim<FK, F_INT4>(D, a, nw, s);
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
    const int32_t head_groups = (c.n_kv_heads + MAX_WAVES - 1) / MAX_WAVES;
    const int64_t target_wgs = 2048;
    int64_t per_seq = (target_wgs + (int64_t)batch * head_groups - 1) / ((int64_t)batch * head_groups);
    if (per_seq < 1) per_seq = 1;
    pps = (int32_t)((max_blocks + per_seq - 1) / per_seq);
    const int32_t min_pps = (256 + c.block_size - 1) / c.block_size;  // >= 256 tokens per split
    if (pps < min_pps) pps = min_pps;
  }
  pps = ((pps + unit - 1) / unit) * unit;
  if (pps > MAX_PPS) pps = (MAX_PPS / unit) * unit;
  return pps;
}

hipError_t launch_decode(const kvq_cache& c, const DecodeArgs& a, hipStream_t s) {
  int nw = 1;
  while (nw < c.n_kv_heads && nw < MAX_WAVES) nw <<= 1;
  switch (c.k_dtype) {
    case F_INT8: return by_v<F_INT8>(c.v_dtype, c.head_dim, a, nw, s);
    case F_FP8: return by_v<F_FP8>(c.v_dtype, c.head_dim, a, nw, s);
    case F_KIVI: return by_v<F_KIVI>(c.v_dtype, c.head_dim, a, nw, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
