// Quantize-on-write into the paged cache (gfx950).
//
// Symmetric formats ("Use Less Memory: Quantization and Offloading", section
// 2.1; "12 KV Cache Quantization", section 5 "Where the scales live"): every
// (token, head) row is quantized on its own, one fp16 scale per row (INT8,
// FP8 E4M3FN) or per 32 channels (INT4).  One pass streams the fp16 rows:
// each lane owns 16 bytes (8 channels) of a row, a row is D/8 consecutive
// lanes, the group max |x| is a lane-group reduction, and the codes of a row
// leave as one contiguous store per lane.
//
// KIVI-style keys ("12 KV Cache Quantization", section 5 "K is more sensitive
// than V"; "Quantized KV caches in production", Numerical Formats; the
// glossary's asymmetric quantization): the 32 rows of a page are quantized
// together per channel when the page's last row arrives (seal_pages);
// rows of unfinished pages wait in the sequence's fp16 tail, written after
// the seal has read the previous tail: by the value pass that follows the
// seal kernel (calls of up to 2048 tokens), or by kivi_tail_kernel after one
// launch that runs the seal and the value pass side by side (larger calls).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 hv2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ hv2 as_hv2(uint32_t u) { return __builtin_bit_cast(hv2, u); }
__device__ __forceinline__ uint32_t hv2_bits(hv2 v) { return __builtin_bit_cast(uint32_t, v); }
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int FMT>
__device__ __forceinline__ float qmax() {
  return FMT == F_INT8 ? 127.0f : FMT == F_FP8 ? 448.0f : FMT == F_E5M2 ? 57344.0f : 7.0f;
}
// RN(1 / q_max), rounded once at compile time
template <int FMT>
__device__ __forceinline__ float inv_qmax() {
  constexpr float r = FMT == F_INT8   ? 1.0f / 127.0f
                      : FMT == F_FP8  ? 1.0f / 448.0f
                      : FMT == F_E5M2 ? 1.0f / 57344.0f
                                      : 1.0f / 7.0f;
  return r;
}

template <int FMT, int D>
struct WShape {
  static constexpr int LPR = D / 8;                      // lanes per row
  static constexpr int RPP = 256 / LPR;                  // rows per pass of a block
  static constexpr int LPG = FMT == F_INT4 ? 4 : LPR;    // lanes per scale group
  static constexpr int CB = FMT == F_INT4 ? D / 2 : D;   // code bytes per row
  static constexpr int NG = FMT == F_INT4 ? D / 32 : 1;  // scales per row
};

// Codes of 8 channels from their exact quotients y = x / s.
template <int FMT>
__device__ __forceinline__ u32x2 encode8(const float (&y)[8]) {
  u32x2 out;
  if constexpr (FMT == F_FP8) {
    float c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = fminf(fmaxf(y[j], -448.0f), 448.0f);
    out.x = fp8x4(c[0], c[1], c[2], c[3]);
    out.y = fp8x4(c[4], c[5], c[6], c[7]);
  } else if constexpr (FMT == F_E5M2) {
    // saturate before the conversion, which would round past 57344 to the
    // infinity code
    float c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = fminf(fmaxf(y[j], -57344.0f), 57344.0f);
    out.x = bf8x4(c[0], c[1], c[2], c[3]);
    out.y = bf8x4(c[4], c[5], c[6], c[7]);
  } else if constexpr (FMT == F_INT8) {
    // clip, round half to even (rne_low_bits), low bytes gathered by v_perm
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = rne_low_bits(__builtin_amdgcn_fmed3f(y[j], -127.0f, 127.0f));
    out.x = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u),
                                  __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u), 0x05040100u);
    out.y = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0C0C0400u),
                                  __builtin_amdgcn_perm(b[5], b[4], 0x0C0C0400u), 0x05040100u);
  } else {  // INT4: two's-complement nibbles, even channel low
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = rne_low_bits(__builtin_amdgcn_fmed3f(y[2 * j], -7.0f, 7.0f));
      const uint32_t hi = rne_low_bits(__builtin_amdgcn_fmed3f(y[2 * j + 1], -7.0f, 7.0f));
      // byte = low nibble of lo | low nibble of hi << 4: m ? lo : hi << 4 with
      // m = 0x0F (truth table of lo = 0xF0, hi = 0xCC, m = 0xAA)
      p[j] = __builtin_amdgcn_bitop3_b32(lo, hi << 4, 0x0Fu, 0xE4);
    }
    out.x = __builtin_amdgcn_perm(__builtin_amdgcn_perm(p[3], p[2], 0x0C0C0400u),
                                  __builtin_amdgcn_perm(p[1], p[0], 0x0C0C0400u), 0x05040100u);
    out.y = 0;
  }
  return out;
}

// stat: calibrated fp16 scale per KV head (uniform over the launch), or NULL
// for the per-token max|x| / q_max.  ROT: the rows are Walsh-Hadamard rotated
// first (y = H (sigma x), exact, then rounded once to fp32), and y is
// quantized in their place.
template <int FMT, int D, int ITER, bool TAIL, bool ROT>
__device__ __forceinline__ void write_rows(const WriteArgs& a, const uint16_t* __restrict__ src,
                                           uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                           const uint16_t* __restrict__ stat, uint32_t bid) {
  using S = WShape<FMT, D>;
  const int lir = threadIdx.x % S::LPR;
  // the lane's 8 rotation signs (bits 8 lir .. 8 lir + 7 of rot_signs) as
  // masks of the sign bits of its four fp16 pairs: x ^ mask negates them
  uint32_t smask[4] = {0u, 0u, 0u, 0u};
  if constexpr (ROT) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < (S::LPR + 3) / 4; ++i) w = (lir >> 2) == i ? a.rot_signs[i] : w;
    const uint32_t sbits = (w >> (8 * (lir & 3))) & 0xFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) smask[i] = ((sbits >> (2 * i)) & 1u) << 15 | ((sbits >> (2 * i + 1)) & 1u) << 31;
  }
  const uint32_t nrows = (uint32_t)(a.T * a.H);
  const uint32_t row0 = bid * (uint32_t)(S::RPP * ITER) + threadIdx.x / S::LPR;
  u32x4 xin[ITER];
  int64_t slot[ITER];
  uint32_t tok[ITER];
  // Issue every load of the block first so ITER rows per lane are in flight:
  // the slots, then the rows (loads complete in issue order, so the tail
  // lookups below wait for the slots only).
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const uint32_t r = row0 + i * S::RPP;
    slot[i] = -1;
    tok[i] = 0;
    if (r < nrows) {
      tok[i] = fastdiv(r, a.div_h);
      slot[i] = a.slots[tok[i]];
    }
  }
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const uint32_t r = row0 + i * S::RPP;
    if (r < nrows) xin[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)r * D) + lir);
  }
  // calibrated scales: the row's head's scale, loaded beside the rows
  uint32_t sst[ITER];
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const uint32_t r = row0 + i * S::RPP;
    sst[i] = 0;
    if (stat && r < nrows) sst[i] = stat[r - tok[i] * (uint32_t)a.H];
  }
  // KIVI keys: whether the row's page is completed within this call (its
  // last row is at the matching call position).  The lookups are issued
  // while the rows are in flight and compared only when the row is stored.
  // Rows of pages left open go to the sequence's fp16 tail.
  constexpr int NT = TAIL ? ITER : 1;
  int32_t tseq[NT], tseq_e[NT];
  int64_t tslot_e[NT], te_[NT];
  if constexpr (TAIL) {
#pragma unroll
    for (int i = 0; i < ITER; ++i) {
      const int64_t sl = slot[i] >= 0 ? slot[i] : 0;
      const int64_t te = (int64_t)tok[i] + (a.bs - 1 - (int)(sl % a.bs));
      const int64_t tc = te < a.T ? te : a.T - 1;  // in bounds; compared below
      te_[i] = te;
      tseq[i] = a.seq_idx[tok[i]];
      tseq_e[i] = a.seq_idx[tc];
      tslot_e[i] = a.slots[tc];
    }
  }
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const uint32_t r = row0 + i * S::RPP;
    if (r >= nrows) continue;  // uniform over the lanes of a row
    const int64_t s = slot[i];
    const bool valid = s >= 0 && s < a.capacity;
    report_error(a.err, s >= a.capacity, KVQ_DEVERR_SLOT);
    float x[8];
    unpack8(uint4{xin[i].x ^ smask[0], xin[i].y ^ smask[1], xin[i].z ^ smask[2], xin[i].w ^ smask[3]}, x);
    if constexpr (ROT) {
      double y[8];
      fwht_row8<S::LPR>(x, lir, y);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (float)y[j];  // one rounding, to nearest even
    }
    const uint32_t h = r - tok[i] * (uint32_t)a.H;
    uint32_t s16;
    if (stat) {
      s16 = sst[i];  // calibrated: quotients beyond q_max saturate in encode8
    } else {
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
      am = group_max<S::LPG>(am);
      // Scale: fp32 quotient, rounded once more to fp16 for storage; the
      // codes divide by the stored value.
      s16 = f2h_bits_of_f32(exact_div(am, qmax<FMT>(), inv_qmax<FMT>()));
      // beyond fp16 (rotated rows only: their entries reach D x 65504): the
      // largest finite fp16 value, the quotients then saturate
      if constexpr (ROT) s16 = s16 < 0x7BFFu ? s16 : 0x7BFFu;
    }
    const float sc = h2f(s16);
    u32x2 enc = {0u, 0u};
    if (sc != 0.0f) {
      const float rc = recip_fp16(sc);
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = exact_div(x[j], sc, rc);
      enc = encode8<FMT>(y);
    }
    if (valid) {
      const size_t orow = (size_t)s * a.H + h;
      // Codes are streamed out with non-temporal stores (nothing in this
      // call reads them back): measured 9% (FP8) and 4% (INT8/INT4) faster
      // writes than ordinary stores.
      if constexpr (FMT == F_INT4) {
        __builtin_nontemporal_store(enc.x, reinterpret_cast<uint32_t*>(codes + orow * S::CB) + lir);
      } else {
        __builtin_nontemporal_store(enc, reinterpret_cast<u32x2*>(codes + orow * S::CB) + lir);
      }
      if (lir % S::LPG == 0) scales[orow * S::NG + lir / S::LPG] = (uint16_t)s16;
      if constexpr (TAIL) {
        // KIVI keys: a row whose page is not completed within this call is
        // kept in fp16 (key and value) in its sequence's tail.
        const int off = (int)(s % a.bs);
        const int32_t seq = tseq[i];
        const bool sealed = te_[i] < a.T && tseq_e[i] == seq && tslot_e[i] == s + (a.bs - 1 - off);
        const bool seq_ok = seq >= 0 && seq < a.max_seqs;
        report_error(a.err, !seq_ok, KVQ_DEVERR_SEQ);
        if (!sealed && seq_ok) {
          const size_t trow = ((size_t)seq * a.bs + off) * a.H + h;
          reinterpret_cast<u32x4*>(a.v_tail + trow * D)[lir] = xin[i];
          reinterpret_cast<u32x4*>(a.k_tail + trow * D)[lir] =
              reinterpret_cast<const u32x4*>(a.k + (size_t)r * D)[lir];
        }
      }
    }
  }
}

// Workgroups [0, nk) write key rows (IK per lane), the rest value rows (IV
// per lane); nk = 0 for KIVI keys, which the seal writes.
template <int FK, int FV, int D, int IK, int IV, bool ROTK, bool ROTV>
__global__ __launch_bounds__(256) void write_sym_kernel(WriteArgs a, uint32_t nk) {
  const uint32_t b = blockIdx.x;
  if (b < nk) {
    if constexpr (FK != F_KIVI) write_rows<FK, D, IK, false, ROTK>(a, a.k, a.k_codes, a.k_scales, a.k_static, b);
  } else {
    write_rows<FV, D, IV, FK == F_KIVI, ROTV>(a, a.v, a.v_codes, a.v_scales, a.v_static, b - nk);
  }
}

// KIVI key pages.  Wave (chunk of C call tokens, head h); C = 32
// for large calls (a chunk then holds about one page end) and 1 for small
// ones (a decode step may complete a page in every sequence at once, and
// each page gets its own wave).  Every token of the chunk that lands on the
// last row of a page completes that page: its 32 key rows (from this call
// where present at the expected call positions, else from the sequence's
// tail) are quantized per channel:
//   s = fp16(fl32(max - min) / 15), z = min, code = clip(rint((x - z) / s), 0, 15).
// Each lane owns PPL channel pairs of every row (rows are split over RG row
// groups when a row has fewer pairs than the wave has lanes), so one row is
// one coalesced load across the wave and the per-channel min and max stay in
// registers.  The rows are loaded from the call positions while the check
// that they hold the page's tokens is in flight; rows that fail it are
// reloaded from the tail.
//
// Seal workgroup `bid` holds nw waves (waves nw.. of the workgroup idle):
// heads c nw .. c nw + nw - 1 of one chunk, so the waves that read the
// neighbouring head segments of the same token rows (and write neighbouring
// code rows) run on one compute unit.  They never synchronize.
template <int D>
__device__ __forceinline__ void seal_pages(const WriteArgs& a, uint32_t bid, int nw) {
  constexpr int PPL = D >= 256 ? D / 128 : 1;  // channel pairs per lane
  constexpr int LPR = D / 2 / PPL;             // lanes per row
  constexpr int RG = 64 / LPR;                 // row groups
  constexpr int RPL = 32 / RG;                 // rows per lane
  const int wave = (int)(threadIdx.x >> 6);
  if (wave >= nw) return;
  const int wgs_per_chunk = a.H / nw;
  const int h = (int)(bid % (uint32_t)wgs_per_chunk) * nw + wave;
  const int64_t chunk = (int64_t)(bid / (uint32_t)wgs_per_chunk);
  const int C = a.seal_chunk;
  const int64_t t0 = chunk * C;
  const int lane = (int)threadIdx.x & 63;
  // slot and sequence of the chunk's token `lane` (lanes < C)
  int64_t my_slot = -1;
  int32_t my_seq = -1;
  if (lane < C && t0 + lane < a.T) {
    my_slot = a.slots[t0 + lane];
    my_seq = a.seq_idx[t0 + lane];
  }
  uint64_t mask = __ballot(my_slot >= 0 && my_slot < a.capacity && (my_slot & 31) == 31);
  const int pl = lane % LPR, g = lane / LPR;
  while (mask) {
    const int j = __ffsll((unsigned long long)mask) - 1;
    mask &= mask - 1;
    const int64_t te = t0 + j;
    // uniform (lane j's slot): read into scalar registers so the page's
    // addresses stay scalar
    const int64_t se = ((int64_t)__builtin_amdgcn_readfirstlane(__shfl((int)(my_slot >> 32), j)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane(__shfl((int)my_slot, j));
    const int32_t seq = __shfl(my_seq, j);
    if (seq < 0 || seq >= a.max_seqs) continue;
    const int64_t blk = se >> 5;
    // row r of the page is in this call at position te - 31 + r when that
    // token belongs to the same sequence and slot; otherwise it is in the
    // tail.  A page ending on the chunk's last token has its rows in this
    // chunk (already loaded); others look them up.
    bool inc = false;
    if (lane < 32) {
      if (C == 32 && j == 31) {
        inc = my_seq == seq && my_slot == se - 31 + lane;
      } else {
        const int64_t ts = te - 31 + lane;
        if (ts >= 0) inc = a.seq_idx[ts] == seq && a.slots[ts] == se - 31 + lane;
      }
    }
    uint32_t x[RPL][PPL];  // fp16 channel pairs, even channel in the low half
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int row = g + RG * i;
      const int64_t ts = te - 31 + row;  // call position of the row (before the call: a dummy read)
      const uint16_t* src = a.k + ((size_t)(ts >= 0 ? ts : 0) * a.H + h) * D;
#pragma unroll
      for (int q = 0; q < PPL; ++q) x[i][q] = reinterpret_cast<const uint32_t*>(src)[pl * PPL + q];
    }
    const uint64_t incall = __ballot(inc);
    if ((uint32_t)incall != 0xFFFFFFFFu) {
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int row = g + RG * i;
        if (!((incall >> row) & 1)) {
          const uint16_t* src = a.k_tail + (((size_t)seq * 32 + row) * a.H + h) * D;
#pragma unroll
          for (int q = 0; q < PPL; ++q) x[i][q] = reinterpret_cast<const uint32_t*>(src)[pl * PPL + q];
        }
      }
    }
    // per-channel min and max on the packed fp16 pairs (exact)
    float mn[2 * PPL], mx[2 * PPL];
#pragma unroll
    for (int q = 0; q < PPL; ++q) {
      hv2 lo = as_hv2(x[0][q]), hi = lo;
#pragma unroll
      for (int i = 1; i < RPL; ++i) {
        lo = __builtin_elementwise_min(lo, as_hv2(x[i][q]));
        hi = __builtin_elementwise_max(hi, as_hv2(x[i][q]));
      }
#pragma unroll
      for (int m = LPR; m < 64; m <<= 1) {
        lo = __builtin_elementwise_min(lo, as_hv2((uint32_t)__shfl_xor((int)hv2_bits(lo), m)));
        hi = __builtin_elementwise_max(hi, as_hv2((uint32_t)__shfl_xor((int)hv2_bits(hi), m)));
      }
      mn[2 * q] = (float)lo.x;
      mn[2 * q + 1] = (float)lo.y;
      mx[2 * q] = (float)hi.x;
      mx[2 * q + 1] = (float)hi.y;
    }
    uint32_t s16[2 * PPL], z16[2 * PPL];
    float sc[2 * PPL], rc[2 * PPL];
#pragma unroll
    for (int c = 0; c < 2 * PPL; ++c) {
      const float range = mx[c] - mn[c];  // fl32(max - min)
      s16[c] = f2h_bits_of_f32(range / 15.0f);
      z16[c] = f2h_bits(mn[c]);  // exact: mn is an fp16 value
      sc[c] = h2f(s16[c]);
      rc[c] = sc[c] != 0.0f ? recip_fp16(sc[c]) : 0.0f;
    }
    // the page's code rows through a buffer resource: a per-lane offset and a
    // uniform row offset, no 64-bit address arithmetic per store
    const auto rco = __builtin_amdgcn_make_buffer_rsrc(a.k_codes + (size_t)blk * 32 * a.H * (D / 2), (short)0,
                                                       0x7FFFFFFF, 0x00020000);
    const int lane_off = (g * a.H + h) * (D / 2) + pl * PPL;
    // 2 (x - z) and 2 s, r / 2: the quotient is the same (exact scaling), and
    // 2 x - 2 z is one mixed-precision FMA on the fp16 x
    float sc2[2 * PPL], rc2[2 * PPL], mn2[2 * PPL];
#pragma unroll
    for (int c = 0; c < 2 * PPL; ++c) {
      sc2[c] = 2.0f * sc[c];
      rc2[c] = 0.5f * rc[c];
      mn2[c] = 2.0f * mn[c];
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int c = 0; c < 2 * PPL; ++c) {
        // fl32(x - z), then fl32(. / s).  No branch on s = 0: with r = 0 the
        // division of the non-negative difference gives +0, so the code is 0.
        const _Float16 xv = __builtin_bit_cast(hv2, x[i][c >> 1])[c & 1];
        const float d2 = __builtin_fmaf((float)xv, 2.0f, -mn2[c]);
        const float y = exact_div(d2, sc2[c], rc2[c]);
        // clip, round half to even: the integer is in the low byte (bits 4-7
        // are 0), and bits above the stored ones are never read
        const uint32_t code = rne_low_bits(__builtin_amdgcn_fmed3f(y, 0.0f, 15.0f));
        w = c == 0 ? code : (code << (4 * c)) | w;
      }
      const int roff = RG * i * a.H * (D / 2);
      if constexpr (PPL == 1) __builtin_amdgcn_raw_buffer_store_b8((unsigned char)w, rco, lane_off, roff, 0);
      else __builtin_amdgcn_raw_buffer_store_b16((unsigned short)w, rco, lane_off, roff, 0);
    }
    if (g == 0) {
      const size_t m = ((size_t)blk * a.H + h) * D + 2 * PPL * pl;
#pragma unroll
      for (int q = 0; q < PPL; ++q) {
        reinterpret_cast<uint32_t*>(a.k_scales + m)[q] = s16[2 * q] | (s16[2 * q + 1] << 16);
        reinterpret_cast<uint32_t*>(a.k_zeros + m)[q] = z16[2 * q] | (z16[2 * q + 1] << 16);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void kivi_seal_kernel(WriteArgs a) {
  seal_pages<D>(a, blockIdx.x, (int)(blockDim.x >> 6));
}

// A large KIVI call in one launch: the value pass's workgroups, then the
// seal's (key pages).  Neither writes the fp16 tail: kivi_tail_kernel does
// that afterwards, once the seal has read the rows the tail held before the
// call, so the value pass carries no tail lookups.  Measured on the
// 131072-token KIVI layer: 8% faster than the seal kernel followed by a value
// pass that writes the tail; interleaving the two kinds of workgroup in
// block order was 2% slower than this order.  8 waves per SIMD: left to
// itself the compiler gives the combined kernel 119 registers (4 waves),
// which made it slower than the two kernels.
template <int FV, int D, int ITER, bool ROTV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8)))
void kivi_write_kernel(WriteArgs a, uint32_t n_val, int nw) {
  const uint32_t b = blockIdx.x;
  if (b < n_val) write_rows<FV, D, ITER, false, ROTV>(a, a.v, a.v_codes, a.v_scales, a.v_static, b);
  else seal_pages<D>(a, b - n_val, nw);
}

// Rows of the pages a large KIVI call leaves open (the page's last row is not
// at its expected position in the call) go to the sequence's fp16 tail, key
// and value.  A workgroup takes 256 call tokens, a thread each: it decides
// whether its token's page stays open and where the token's tail row is; the
// open tokens are listed in LDS, and then all 256 threads copy their rows (H
// rows of D values, contiguous in the call and in the tail row) in 16-byte
// pieces, the loads of up to 32 tokens in flight per thread.  Most tokens of
// a prefill close their page; a workgroup without an open token stops after
// the check.
template <int D>
__global__ __launch_bounds__(256) void kivi_tail_kernel(WriteArgs a) {
  __shared__ int64_t s_src[256];  // call token of the i-th open token
  __shared__ int64_t s_dst[256];  // its tail row (offset in halves)
  __shared__ int s_cnt[4];
  const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t = (int64_t)blockIdx.x * 256 + tid;
  int64_t dst = -1;
  if (t < a.T) {
    const int64_t s = a.slots[t];
    if (s >= 0 && s < a.capacity) {
      const int32_t seq = a.seq_idx[t];
      const bool seq_ok = seq >= 0 && seq < a.max_seqs;
      report_error(a.err, !seq_ok, KVQ_DEVERR_SEQ);
      const int off = (int)(s % a.bs);
      const int64_t te = t + (a.bs - 1 - off);
      const bool sealed = te < a.T && a.seq_idx[te] == seq && a.slots[te] == s + (a.bs - 1 - off);
      if (seq_ok && !sealed) dst = ((int64_t)seq * a.bs + off) * a.H * D;
    }
  }
  const uint64_t m = __ballot(dst >= 0);
  if (lane == 0) s_cnt[w] = __popcll(m);
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    base += i < w ? s_cnt[i] : 0;
    total += s_cnt[i];
  }
  if (total == 0) return;  // the same for every thread of the workgroup
  if (dst >= 0) {
    const int pos = base + __popcll(m & ((1ull << lane) - 1));
    s_src[pos] = t;
    s_dst[pos] = dst;
  }
  __syncthreads();
  const int nch = a.H * D / 8;  // 16-byte pieces of one token's H rows (keys, then values)
  for (int c = tid; c < 2 * nch; c += 256) {
    const bool isv = c >= nch;
    const size_t cofs = (size_t)(isv ? c - nch : c) * 8;  // in halves
    const uint16_t* src = isv ? a.v : a.k;
    uint16_t* dstb = isv ? a.v_tail : a.k_tail;
    for (int k0 = 0; k0 < total; k0 += 32) {
      u32x4 buf[32];
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (k0 + u < total)
          buf[u] = *reinterpret_cast<const u32x4*>(src + (size_t)s_src[k0 + u] * a.H * D + cofs);
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (k0 + u < total) *reinterpret_cast<u32x4*>(dstb + s_dst[k0 + u] + cofs) = buf[u];
    }
  }
}

namespace {

// Rows per lane of a tensor's rows in write_sym_kernel.  Measured in one
// process (prefill writes of the large workloads): one row per lane, i.e.
// more and shorter workgroups, 5.45 -> 5.88 TB/s for the 8-bit formats
// against 4 rows per lane, and 2-3% faster than 2; INT4 group-32 rows (four
// group maxima and scales per row) 3% faster at 2 than at 1; the KIVI value
// pass is fastest at 2 (with its tail lookups, and in the combined launch of
// large calls without them).  Rotated rows are bound by the issue of the
// transform's vector instructions, and two rows per lane share the lane's
// sign masks and butterfly constants: 7% faster than one (2.76-3.24 GB
// writes; four rows: no further change).
template <int FMT, bool ROT, bool KIVI_V>
constexpr int rows_per_lane() { return FMT == F_INT4 || ROT || KIVI_V ? 2 : 1; }

template <int FK, int FV, int D, bool ROTK, bool ROTV>
hipError_t launch_sym_rot(const WriteArgs& a, hipStream_t s) {
  constexpr int IK = rows_per_lane<FK, ROTK, false>(), IV = rows_per_lane<FV, ROTV, FK == F_KIVI>();
  constexpr int RPP = 256 / (D / 8);
  const int64_t rows = a.T * a.H;
  const int64_t nk = FK == F_KIVI ? 0 : (rows + RPP * IK - 1) / (RPP * IK);
  const int64_t all = nk + (rows + RPP * IV - 1) / (RPP * IV);
  if (all >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((write_sym_kernel<FK, FV, D, IK, IV, ROTK, ROTV>), dim3((unsigned)all), dim3(256), 0, s, a,
                     (uint32_t)nk);
  return hipGetLastError();
}

template <int FK, int FV, int D>
hipError_t launch_sym(const WriteArgs& a, hipStream_t s) {
  constexpr bool RK = FK != F_KIVI;  // KIVI keys are never rotated
  if (a.rot_k && a.rot_v) return launch_sym_rot<FK, FV, D, RK, true>(a, s);
  if (a.rot_k) return launch_sym_rot<FK, FV, D, RK, false>(a, s);
  if (a.rot_v) return launch_sym_rot<FK, FV, D, false, true>(a, s);
  return launch_sym_rot<FK, FV, D, false, false>(a, s);
}

template <int FK, int FV, int D>
hipError_t launch_all(const WriteArgs& a, hipStream_t s) {
  if constexpr (FK == F_KIVI) {
    const int64_t chunks = (a.T + a.seal_chunk - 1) / a.seal_chunk;
    // waves per seal workgroup: the largest divisor of H up to 4 (heads of
    // one chunk; 4 measured 2-3% faster than 8)
    int nw = a.H < 4 ? a.H : 4;
    while (a.H % nw) --nw;
    const int64_t wgs = chunks * (a.H / nw);
    if (a.seal_chunk > 1) {
      // large call: value pass and seal in one launch, then the tail rows
      constexpr int kIter = rows_per_lane<FV, false, true>();
      constexpr int RPP = 256 / (D / 8);
      const int64_t vwgs = (a.T * a.H + RPP * kIter - 1) / (RPP * kIter);
      const int64_t all = wgs + vwgs;
      if (all >= (1ll << 31)) return hipErrorInvalidValue;
      if (a.rot_v)
        hipLaunchKernelGGL((kivi_write_kernel<FV, D, kIter, true>), dim3((unsigned)all), dim3(256), 0, s, a,
                           (uint32_t)vwgs, nw);
      else
        hipLaunchKernelGGL((kivi_write_kernel<FV, D, kIter, false>), dim3((unsigned)all), dim3(256), 0, s, a,
                           (uint32_t)vwgs, nw);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t twgs = (a.T + 255) / 256;
      hipLaunchKernelGGL((kivi_tail_kernel<D>), dim3((unsigned)twgs), dim3(256), 0, s, a);
      return hipGetLastError();
    }
    if (wgs >= (1ll << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((kivi_seal_kernel<D>), dim3((unsigned)wgs), dim3(64 * nw), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_sym<FK, FV, D>(a, s);
}

template <int FK, int FV>
hipError_t by_dim(int D, const WriteArgs& a, hipStream_t s) {
  switch (D) {
    case 64: return launch_all<FK, FV, 64>(a, s);
    case 128: return launch_all<FK, FV, 128>(a, s);
    case 256: return launch_all<FK, FV, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int FK>
hipError_t by_v(int fv, int D, const WriteArgs& a, hipStream_t s) {
  switch (fv) {
    case F_INT8: return by_dim<FK, F_INT8>(D, a, s);
    case F_FP8: return by_dim<FK, F_FP8>(D, a, s);
    case F_INT4: return by_dim<FK, F_INT4>(D, a, s);
    case F_E5M2: return by_dim<FK, F_E5M2>(D, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_write(const kvq_cache& c, const WriteArgs& a, hipStream_t s) {
  switch (c.k_dtype) {
    case F_INT8: return by_v<F_INT8>(c.v_dtype, c.head_dim, a, s);
    case F_FP8: return by_v<F_FP8>(c.v_dtype, c.head_dim, a, s);
    case F_INT4: return by_v<F_INT4>(c.v_dtype, c.head_dim, a, s);
    case F_KIVI: return by_v<F_KIVI>(c.v_dtype, c.head_dim, a, s);
    case F_E5M2: return by_v<F_E5M2>(c.v_dtype, c.head_dim, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
