// Chunked-prefill attention over the quantized pages (gfx950).
//
// What is computed ("Use Less Memory: Quantization and Offloading", What
// Comes Next: a long prompt is processed in scheduled pieces; "12 KV Cache
// Quantization", Interaction with prefix caching: a new piece attends to
// quantized blocks already in the cache): the n queries of sequence b's
// chunk are its last n positions, their keys and values already written;
// query i at position p = L - n + i attends to tokens 0..p,
// o = softmax(q k_hat^T sm_scale) V_hat, query head hq reading KV head hq / G.
//
// How (MI355X design):
//  * A workgroup of 4 waves owns one (sequence, KV head, tile of ROWS query
//    rows).  Query rows are (position, query head) pairs, position-major, so
//    the G heads of a position share every key and value the tile reads.
//    Each wave holds NQB blocks of 16 rows: the 16 columns of its MFMAs.
//  * Keys and values are read once per workgroup in tiles of 32 tokens: the
//    256 threads load tile x + 2 into registers while the waves compute from
//    LDS, and store it at the end of the step (three LDS buffers, one barrier
//    per tile).  In the step of tile x each wave issues the score MFMAs of
//    tile x + 1 before the softmax and P V of tile x, so matrix and vector
//    work of one wave overlap.  Key codes are converted to fp16 once, when
//    stored.  Block ids are fetched two tiles ahead of their loads.
//  * Workgroup order: the grid is dealt to the 8 XCDs round robin; the
//    workgroups an XCD receives are consecutive (sequence, KV head, tile)
//    triples, so the ~64 workgroups resident on one XCD read the same
//    sequence's pages at about the same time through that XCD's L2.  Within
//    a (sequence, KV head) the last (longest) query tile starts first.
//  * Scores S^T = K Q^T (tokens x query rows) and O^T = V^T P^T (channels x
//    query rows) run on the matrix cores.  A lane holds the same query
//    column in both products, so the online softmax state (max, sum) of a
//    column lives in the lanes that hold it and rescaling needs no lane
//    exchange; the probability operand of P V is the lane's own scores.
//  * Operands are those of the decode kernels: exact fp16 key codes against
//    the fp16 query (rotated keys: the rotated query as fp16 hi + lo, two
//    MFMAs), exact bf16 value codes (INT8/INT4 biased to unsigned) against
//    probability x value scale as bf16 hi + lo (two MFMAs).  KIVI keys are
//    dequantized once per tile into LDS as fp16 hi + lo, k_hat = c s + z
//    (two MFMAs against the exact query); the fp16 tail of a KIVI sequence
//    is one more tile at the end, its fp16 values split exactly into bf16
//    hi + lo (four MFMAs).
//  * fp32 softmax in the log2 domain; the result is rounded to fp16 once.
#pragma once

#include "kvq_decode.h"

namespace kvq {

template <int FK, int FV, int D>
struct PLayout {
  static constexpr bool KIVI = FK == F_KIVI;
  // 4-bit keys (KIVI, INT4 group-32) are dequantized when stored: k_hat as
  // fp16 hi and lo planes
  static constexpr bool PLANES = KIVI || FK == F_INT4;
  using VS = VShape<FV, D>;
  static constexpr int NQB = D <= 128 ? 2 : 1;  // 16-column blocks per wave
  static constexpr int NWAVE = 4;
  static constexpr int THREADS = 64 * NWAVE;
  static constexpr int ROWS = NWAVE * 16 * NQB;  // query rows per workgroup
  // LDS: three buffers of [keys fp16 | value codes | key scales fp32 | value
  // scales fp32] (4-bit keys: fp16 hi plane then lo plane), then (KIVI) the
  // tail's values transposed, fp16 [D][32].  Value scales of INT4 groups are
  // stored group-major, [group][token].
  static constexpr int KRB = 2 * D;             // key row bytes in LDS: fp16 (4-bit keys: per plane)
  static constexpr int KCH = KRB / 16;          // 16-byte chunks per key row
  static constexpr int KPLANE = TILE * KRB;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = (PLANES ? 2 : 1) * KPLANE;
  // 8-bit values at head dims up to 128 are staged as their exact bf16
  // operands (converted once per workgroup when stored, read with the 16-bit
  // transpose read), 2 D bytes per token row; otherwise the codes themselves
  static constexpr bool V16 = FV != F_INT4 && D <= 128;
  static constexpr int VRB = V16 ? 2 * D : VS::RB;  // value row bytes in LDS
  static constexpr int OFF_FK = OFF_V + TILE * VRB;
  static constexpr int OFF_FV = OFF_FK + 4 * TILE;
  static constexpr int BUF = (OFF_FV + 4 * TILE * VS::NG + 15) / 16 * 16;
  static constexpr int NBUF = 3;  // tiles x (softmax, P V), x + 1 (scores), x + 2 (being stored)
  static constexpr int OFF_VT = NBUF * BUF;
  static constexpr int LDS = NBUF * BUF + (KIVI ? D * TILE * 2 : 0);
  // a tile's 16-byte chunks of key codes (8-bit formats) and value codes
  static constexpr int NK = TILE * (D / 16);
  static constexpr int NLK = (NK + THREADS - 1) / THREADS;
  static constexpr int NV = TILE * VS::CH;
  static constexpr int NLV = (NV + THREADS - 1) / THREADS;
  // 4-bit keys: thread (t, cg) = (tid / 8, tid % 8) handles channels cg KE
  // .. cg KE + KE - 1 of token t: KE / 2 code bytes; KIVI: KM 16-byte chunks
  // of fp16 scales, zeros (or of the tail's key and value rows); INT4
  // group-32: the channels' one group scale (KE <= 32 and KE divides 32)
  static constexpr int KE = D / 8;
  static constexpr int KM = KE / 8;
};

// N (4, 8 or 16) bytes at p into the low bytes of a u4
template <int N>
__device__ __forceinline__ u4 load_n(const void* p) {
  if constexpr (N == 16) return *reinterpret_cast<const u4*>(p);
  else if constexpr (N == 8) {
    const u2 v = *reinterpret_cast<const u2*>(p);
    return u4{v.x, v.y, 0u, 0u};
  } else if constexpr (N == 4) {
    return u4{*reinterpret_cast<const uint32_t*>(p), 0u, 0u, 0u};
  } else {
    return u4{(uint32_t)*reinterpret_cast<const uint16_t*>(p), 0u, 0u, 0u};
  }
}

__device__ __forceinline__ uint32_t u4_word(const u4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int FK, int FV, int D>
struct PRegs {
  using PL = PLayout<FK, FV, D>;
  u4 k[PL::PLANES ? 1 : PL::NLK];  // key code chunks (8-bit keys); 4-bit keys: the thread's code bytes in k[0]
  u4 ks[PL::KIVI ? PL::KM : 1];  // KIVI: scales of the thread's channels (tail tile: the key row)
  u4 kz[PL::KIVI ? PL::KM : 1];  // KIVI: zero points (tail tile: the value row)
  u4 v[PL::NLV];
  uint16_t fk;                   // wave 0, lanes < 32: fp16 key scale of token lane
  uint16_t kg;                   // INT4 group-32 keys: the scale of the thread's channels' group
  u4 fv;                         // wave 0, lanes >= 32: fp16 value scales of token lane - 32
};

// Value operand of 8-bit codes (as value_operand_8bit) whose INT8 codes were
// stored already biased to c + 128: the bf16 bit patterns u (u 2^-133) are
// placed by two byte permutes per dword pair, no xor.
template <int FV>
__device__ __forceinline__ b8 value_operand_biased(i2 t) {
  if constexpr (FV != F_INT8) {
    return value_operand_8bit<FV>(t);
  } else {
    const uint32_t d0 = (uint32_t)t.x, d1 = (uint32_t)t.y;
    const u4 r = {__builtin_amdgcn_perm(0u, d0, 0x0C010C00u), __builtin_amdgcn_perm(0u, d0, 0x0C030C02u),
                  __builtin_amdgcn_perm(0u, d1, 0x0C010C00u), __builtin_amdgcn_perm(0u, d1, 0x0C030C02u)};
    return __builtin_bit_cast(b8, r);
  }
}

// bf16-staged value rows: 32-byte block m of token row t is stored at block
// m ^ (t mod NB), NB = min(D / 16, 8), so the 16 token rows one transpose
// read touches spread over the LDS banks.
template <int D>
__device__ __forceinline__ int v16swz(int row) {
  constexpr int NB = D / 16 < 8 ? D / 16 : 8;
  return row & (NB - 1);
}
typedef short s4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4v lds_s4v;

// fp16 pair -> bf16 hi (truncated) and lo = x - hi; both exact (an fp16
// value has 11 significant bits, hi keeps 8)
__device__ __forceinline__ void split_f16x2_bf16(uint32_t h2v, uint32_t& hi, uint32_t& lo) {
  const float f0 = h2f(h2v & 0xFFFFu), f1 = h2f(h2v >> 16);
  const uint32_t b0 = __builtin_bit_cast(uint32_t, f0) & 0xFFFF0000u;
  const uint32_t b1 = __builtin_bit_cast(uint32_t, f1) & 0xFFFF0000u;
  hi = (b0 >> 16) | b1;
  const f2 rem = {f0 - __builtin_bit_cast(float, b0), f1 - __builtin_bit_cast(float, b1)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(rem, bf2));
}

// Waves per SIMD: two (each within 256 registers) where the kernel fits
// them without spilling; one for INT4 values with rotated keys (the extra
// query operand) and for KIVI keys at head_dim 256.
template <int FK, int FV, int D, bool ROTQ>
constexpr int prefill_wpe() {
  return (FV == F_INT4 && ROTQ) || ((FK == F_KIVI || FK == F_INT4) && D == 256) ? 1 : 2;
}

template <int FK, int FV, int D, bool ROTQ>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(prefill_wpe<FK, FV, D, ROTQ>(), prefill_wpe<FK, FV, D, ROTQ>())))
void prefill_kernel(PrefillArgs a) {
  using PL = PLayout<FK, FV, D>;
  using VS = VShape<FV, D>;
  constexpr int NQB = PL::NQB, KB = D / 32;
  constexpr bool KIVI = FK == F_KIVI;
  constexpr bool VFP8 = FV == F_FP8 || FV == F_E5M2;
  constexpr float VSC = VFP8 ? 1.f : 0x1p60f;  // value scales carry 2^60 for the u 2^-133 operands
  constexpr int NCS = FV == F_INT4 ? VS::NG : 1;
  constexpr int CHK = D / 16;  // key chunks per row (8-bit keys)
  extern __shared__ __attribute__((aligned(16))) uint8_t s_lds[];

  // ---- workgroup -> (sequence b, KV head h, query tile qt) ------------------
  const int per = (a.n_wg + 7) >> 3;
  const int logical = (int)(blockIdx.x & 7u) * per + (int)(blockIdx.x >> 3);
  if (logical >= a.n_wg) return;
  const int bh = logical / a.n_qtiles;
  const int qt = a.n_qtiles - 1 - (logical - bh * a.n_qtiles);
  const int b = bh / a.H, h = bh - b * a.H;
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave of the workgroup (uniform)
  const int j = lane >> 4, n = lane & 15;
  const int r0q = __builtin_amdgcn_readfirstlane(a.q_start[b]);
  const int r1q = __builtin_amdgcn_readfirstlane(a.q_start[b + 1]);
  const int nq = r1q - r0q;
  if (r0q < 0 || (int64_t)r1q > a.Tq || nq < 0 || nq > a.max_q_len) {
    // a malformed chunk: the sequence is skipped
    if (qt == 0 && h == 0 && wv == 0) report_error(a.err, lane == 0, KVQ_DEVERR_QLEN);
    return;
  }
  const int rows = nq * a.G;  // query rows of the sequence
  const int R0 = qt * PL::ROWS;
  if (R0 >= rows) return;
  const int cap = a.max_blocks << a.log2_bs;
  const int rawL = __builtin_amdgcn_readfirstlane(a.ctx_lens[b]);
  const int L = min(max(rawL, 0), cap);
  if (qt == 0 && h == 0 && wv == 0) report_error(a.err, lane == 0 && (rawL < 0 || rawL > cap), KVQ_DEVERR_CTX);
  const int pos0 = L - nq;  // position of the chunk's first query

  // ---- query columns of this wave -----------------------------------------
  const int Rw = R0 + wv * 16 * NQB;  // first row of the wave
  int pos_c[NQB];                     // position of column n of block cb (-1: no query)
  size_t qrow[NQB];                   // its row in q / out: (query, head) index
  h8 qop[NQB][KB];
  h8 qlo[ROTQ ? NQB : 1][ROTQ ? KB : 1];
#pragma unroll
  for (int cb = 0; cb < NQB; ++cb) {
    const int R = Rw + 16 * cb + n;
    const bool live = R < rows;
    const int i = live ? R / a.G : 0;
    const int g = R - i * a.G;
    pos_c[cb] = live ? pos0 + i : -1;
    qrow[cb] = live ? (size_t)(r0q + i) * a.Hq + (size_t)h * a.G + g : 0;
    const uint16_t* src = (ROTQ ? a.qrot : a.q) + qrow[cb] * D + j * (D / 4);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const h8 v = *reinterpret_cast<const h8*>(src + 8 * kb);
      qop[cb][kb] = live ? v : h8{};
    }
    if constexpr (ROTQ) {
      const uint16_t* lo = src + (size_t)a.Tq * a.Hq * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const h8 v = *reinterpret_cast<const h8*>(lo + 8 * kb);
        qlo[cb][kb] = live ? v : h8{};
      }
    }
  }
  // positions of the wave's first and last live rows (uniform)
  const int pos_lo = __builtin_amdgcn_readfirstlane(Rw < rows ? pos0 + Rw / a.G : INT_MAX);
  const int pos_hi = __builtin_amdgcn_readfirstlane(Rw < rows ? pos0 + (min(Rw + 16 * NQB, rows) - 1) / a.G : -1);

  // ---- tiles ---------------------------------------------------------------
  const int pos_max = pos0 + (min(R0 + PL::ROWS, rows) - 1) / a.G;  // last position of the workgroup
  const int Lq = KIVI ? (L & ~31) : L;                               // tokens in quantized pages
  const int nt = pos_max >= 0 ? pos_max / TILE + 1 : 0;              // tiles with visible tokens
  const int ntm = __builtin_amdgcn_readfirstlane(min(nt, (Lq + TILE - 1) / TILE));  // of those, read from pages
  const bool tail = KIVI && nt > ntm;                                // KIVI: the fp16 tail is visible

  f4 acc[NQB][VS::NPV];
  // l_run + l_err: the column's probability sum (this lane's tokens), kept
  // with its rounding error (two_sum_acc), one add per tile
  float m_run[NQB], l_run[NQB], l_err[NQB], cs_run[NQB][NCS];
#pragma unroll
  for (int cb = 0; cb < NQB; ++cb) {
#pragma unroll
    for (int m = 0; m < VS::NPV; ++m) acc[cb][m] = f4{0.f, 0.f, 0.f, 0.f};
    m_run[cb] = -INFINITY;
    l_run[cb] = 0.f;
    l_err[cb] = 0.f;
#pragma unroll
    for (int g = 0; g < NCS; ++g) cs_run[cb][g] = 0.f;
  }

  // Block-table entry of the page of token 32 x + lane % 32, clamped to the
  // sequence's last quantized page (tokens past Lq are masked where the id
  // is used).  Always issued and never copied before its use a tile later,
  // so the wait for it never covers the tile loads issued after it.
  const int last_page = Lq > 0 ? (Lq - 1) >> a.log2_bs : 0;
  const int* bt_row = a.block_table + (size_t)b * a.max_blocks;
  auto load_id = [&](int x) __attribute__((always_inline)) {
    const int tok = TILE * x + (lane & 31);
    return bt_row[min(tok >> a.log2_bs, last_page)];
  };

  // Issue the loads of page tile x (block id `id` of token lane % 32);
  // returns the live mask (bit t: token 32 x + t is in the context on a
  // valid page).  Dead rows read flat row 0 and are zeroed when stored.
  auto load_tile = [&](int x, int id, PRegs<FK, FV, D>& r) __attribute__((always_inline)) {
    const int tok = TILE * x + (lane & 31);
    const bool in_ctx = tok < Lq;
    const bool ok = in_ctx && id >= 0 && id < a.nb;
    if (wv == 0) report_error(a.err, lane < 32 && in_ctx && !ok, KVQ_DEVERR_BLOCK);
    const uint32_t flat =
        ok ? (((uint32_t)id << a.log2_bs) + (uint32_t)(tok & (a.bs - 1))) * (uint32_t)a.H + (uint32_t)h : 0u;
    const uint32_t live = (uint32_t)__ballot(ok);
    if constexpr (!PL::PLANES) {
#pragma unroll
      for (int i = 0; i < PL::NLK; ++i) {
        const int p = tid + PL::THREADS * i;
        if (PL::NK % PL::THREADS == 0 || p < PL::NK) {
          const int row = p / CHK, col = p % CHK;
          const uint32_t fr = (uint32_t)__shfl((int)flat, row);
          r.k[i] = *reinterpret_cast<const u4*>(a.k_codes + (size_t)fr * D + col * 16);
        }
      }
    } else {
      const int t = tid >> 3, cg = tid & 7;
      const uint32_t fr = (uint32_t)__shfl((int)flat, t);
      r.k[0] = load_n<D / 16>(a.k_codes + (size_t)fr * (D / 2) + cg * (D / 16));
      if constexpr (FK == F_INT4) {
        r.kg = a.k_scales[(size_t)fr * (D / 32) + (cg * PL::KE) / 32];
      } else {
      // the tile is one page (block_size 32): its scales and zeros for head h
      const int id0 = __builtin_amdgcn_readfirstlane(id);
      const bool ok0 = (live & 1u) != 0u;
      const size_t mrow = ((size_t)(ok0 ? id0 : 0) * a.H + h) * D + cg * PL::KE;
#pragma unroll
      for (int k = 0; k < PL::KM; ++k) {
        r.ks[k] = *reinterpret_cast<const u4*>(a.k_scales + mrow + 8 * k);
        r.kz[k] = *reinterpret_cast<const u4*>(a.k_zeros + mrow + 8 * k);
      }
      }
    }
#pragma unroll
    for (int i = 0; i < PL::NLV; ++i) {
      const int p = tid + PL::THREADS * i;
      if (PL::NV % PL::THREADS == 0 || p < PL::NV) {
        const int row = p / VS::CH;
        const int col = PL::V16 ? p % VS::CH : (p % VS::CH) ^ vswz<VS::CH>(row);
        const uint32_t fr = (uint32_t)__shfl((int)flat, row);
        r.v[i] = *reinterpret_cast<const u4*>(a.v_codes + (size_t)fr * VS::RB + col * 16);
      }
    }
    if (wv == 0) {
      // every lane loads both (lanes < 32 keep the key scale, the others
      // the value scales), so no branch waits on a load
      if constexpr (!PL::PLANES) r.fk = a.k_scales[flat];
      r.fv = load_n<2 * VS::NG>(a.v_scales + (size_t)flat * VS::NG);
    }
    return live;
  };

  // Store a loaded page tile into LDS buffer `buf` (layout PLayout).
  auto store_tile = [&](const PRegs<FK, FV, D>& r, uint32_t live, uint8_t* buf) __attribute__((always_inline)) {
    if constexpr (!PL::PLANES) {
#pragma unroll
      for (int i = 0; i < PL::NLK; ++i) {
        const int p = tid + PL::THREADS * i;
        if (PL::NK % PL::THREADS == 0 || p < PL::NK) {
          // 16 codes of row p / CHK, channels 16 (p % CHK) ..: exact fp16
          // values, 16-byte chunks 2 (p % CHK) and 2 (p % CHK) + 1 of the row
          const int row = p / CHK, col = p % CHK;
          const bool lv = (live >> row) & 1u;
          const u4 c = lv ? r.k[i] : u4{0u, 0u, 0u, 0u};
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
          uint32_t hw[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (FK == F_FP8) fp8_to_h4(cw[w], hw[2 * w], hw[2 * w + 1]);
            else if constexpr (FK == F_E5M2) e5m2_to_h4(cw[w], hw[2 * w], hw[2 * w + 1]);
            else int8_to_h4(cw[w], hw[2 * w], hw[2 * w + 1]);
          }
          u4* kr = reinterpret_cast<u4*>(buf + PL::OFF_K);
          kr[row * PL::KCH + ((2 * col) ^ kswz<PL::KCH>(row))] = u4{hw[0], hw[1], hw[2], hw[3]};
          kr[row * PL::KCH + ((2 * col + 1) ^ kswz<PL::KCH>(row))] = u4{hw[4], hw[5], hw[6], hw[7]};
        }
      }
    } else {
      // KIVI: k_hat = c s + z in fp32 (one rounding); INT4 group-32: k_hat =
      // c s, exact (at most 3 + 11 significant bits).  Stored as fp16 hi + lo
      // with hi = RN(min(|k_hat|, 65504)), lo = RN(k_hat - hi)
      const int t = tid >> 3, cg = tid & 7;
      const bool lv = (live >> t) & 1u;
      uint32_t hw[PL::KE / 2], lw[PL::KE / 2];
#pragma unroll
      for (int e2 = 0; e2 < PL::KE / 2; ++e2) {
        const uint32_t codes = u4_word(r.k[0], e2 / 4) >> (8 * (e2 % 4));  // byte e2: channels 2 e2, 2 e2 + 1
        uint32_t hh[2], ll[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float x;
          if constexpr (FK == F_INT4) {
            // two's-complement nibble
            const float c = (float)((int)(((codes >> (4 * q)) & 0xFu) ^ 8u) - 8);
            x = lv ? c * h2f(r.kg) : 0.f;
          } else {
            const uint32_t sw = u4_word(r.ks[e2 / 4], e2 % 4), zw = u4_word(r.kz[e2 / 4], e2 % 4);
            const float c = (float)((codes >> (4 * q)) & 0xFu);
            x = lv ? __builtin_fmaf(c, h2f(sw >> (16 * q)), h2f((zw >> (16 * q)) & 0xFFFFu)) : 0.f;
          }
          const float xs = fminf(fmaxf(x, -65504.f), 65504.f);
          hh[q] = f2h_bits_of_f32(xs);
          ll[q] = f2h_bits(x - h2f(hh[q]));
        }
        hw[e2] = hh[0] | (hh[1] << 16);
        lw[e2] = ll[0] | (ll[1] << 16);
      }
#pragma unroll
      for (int k = 0; k < PL::KM; ++k) {
        const int c = cg * PL::KM + k;  // logical 16-byte chunk of row t
        const int slot = t * PL::KCH + (c ^ kswz<PL::KCH>(t));
        reinterpret_cast<u4*>(buf + PL::OFF_K)[slot] = u4{hw[4 * k], hw[4 * k + 1], hw[4 * k + 2], hw[4 * k + 3]};
        reinterpret_cast<u4*>(buf + PL::OFF_K + PL::KPLANE)[slot] =
            u4{lw[4 * k], lw[4 * k + 1], lw[4 * k + 2], lw[4 * k + 3]};
      }
    }
#pragma unroll
    for (int i = 0; i < PL::NLV; ++i) {
      const int p = tid + PL::THREADS * i;
      if (PL::NV % PL::THREADS == 0 || p < PL::NV) {
        const bool lv = (live >> (p / VS::CH)) & 1u;
        u4 v = lv ? r.v[i] : u4{0u, 0u, 0u, 0u};
        if constexpr (FV == F_INT8) v ^= 0x80808080u;  // codes c + 128 (unsigned), see value_operand_biased
        if constexpr (PL::V16) {
          // 16 codes of token row p / CH, channels 16 (p % CH) ..: their bf16
          // operands (value_operand_8bit's values, in channel order) into
          // the row's 32-byte block (p % CH) ^ v16swz<D>(row)
          const int row = p / VS::CH, col = p % VS::CH;
          const uint32_t cw[4] = {v.x, v.y, v.z, v.w};
          uint32_t bw[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (FV == F_INT8) {
              bw[2 * w] = __builtin_amdgcn_perm(0u, cw[w], 0x0C010C00u);
              bw[2 * w + 1] = __builtin_amdgcn_perm(0u, cw[w], 0x0C030C02u);
            } else if constexpr (FV == F_FP8) {
              bw[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[w], 1.0f, false));
              bw[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[w], 1.0f, true));
            } else {
              bw[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(cw[w], 1.0f, false));
              bw[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(cw[w], 1.0f, true));
            }
          }
          u4* dst = reinterpret_cast<u4*>(buf + PL::OFF_V + row * PL::VRB + ((col ^ v16swz<D>(row)) << 5));
          dst[0] = u4{bw[0], bw[1], bw[2], bw[3]};
          dst[1] = u4{bw[4], bw[5], bw[6], bw[7]};
        } else {
          reinterpret_cast<u4*>(buf + PL::OFF_V)[p] = v;
        }
      }
    }
    if (wv == 0) {
      float* fk = reinterpret_cast<float*>(buf + PL::OFF_FK);
      float* fv = reinterpret_cast<float*>(buf + PL::OFF_FV);
      const int t = lane & 31;
      const bool lv = (live >> t) & 1u;
      if (lane < 32) {
        // A zero key scale comes with zero codes (the writer stores all-zero
        // codes when the scale is 0), so such a row scores 0 with any factor;
        // dead rows and zero scales store factor 1, so that a masked (-inf)
        // raw score stays -inf when scaled.
        if constexpr (!PL::PLANES) fk[t] = (lv && (r.fk & 0x7FFFu) != 0u) ? h2f(r.fk) * a.qscale : 1.f;
      } else {
#pragma unroll
        for (int g = 0; g < VS::NG; ++g)
          fv[g * TILE + t] = lv ? h2f(u4_word(r.fv, g / 2) >> (16 * (g & 1))) * VSC : 0.f;
      }
    }
  };

  // Value transpose reads (as in decode): lane (j, i) points at row T_j[i / 2]
  // of the value tile, byte 8 (i % 2) of the chunk.  bf16-staged values
  // (V16): lane (j, n) of the 16-bit transpose read points at token row
  // 4 j + n / 4 (tokens 16 + 4 j + n / 4 for the second read), channels
  // 16 m + 4 (n % 4) ..: the read hands lane n of each 16-lane group element
  // n % 4 of the rows of lanes n / 4, n / 4 + 4, + 8, + 12, i.e. channel
  // 16 m + n of tokens T_j[0..3] (then T_j[4..7]).
  const int trow = 16 * ((n >> 1) >> 2) + 4 * j + ((n >> 1) & 3);
  const int tbase = PL::OFF_V + trow * VS::RB + 8 * (n & 1);
  const int tswz = vswz<VS::CH>(trow);

  // Raw scores S^T = K Q^T of tile x (held in LDS buffer `buf`) on the matrix
  // cores.  TAILT: the KIVI tail tile (fp16 keys in the hi plane only).
  auto scores = [&](const uint8_t* buf, int x, f4 (&sc)[NQB][2], auto tailc) __attribute__((always_inline)) {
    constexpr bool TAILT = decltype(tailc)::value;
    if (pos_hi < TILE * x) return;  // every query of the wave precedes the tile
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 16 * u + n;
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb) sc[cb][u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int c = j * (D / 32) + kb;
        const int off = PL::OFF_K + (row * PL::KCH + (c ^ kswz<PL::KCH>(row))) * 16;
        const h8 kh = *reinterpret_cast<const h8*>(buf + off);
#pragma unroll
        for (int cb = 0; cb < NQB; ++cb) {
          sc[cb][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, qop[cb][kb], sc[cb][u], 0, 0, 0);
          if constexpr (ROTQ) sc[cb][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, qlo[cb][kb], sc[cb][u], 0, 0, 0);
        }
        if constexpr (PL::PLANES && !TAILT) {
          const h8 kl = *reinterpret_cast<const h8*>(buf + off + PL::KPLANE);
#pragma unroll
          for (int cb = 0; cb < NQB; ++cb)
            sc[cb][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl, qop[cb][kb], sc[cb][u], 0, 0, 0);
        }
      }
    }
  };

  // Online softmax and P V of tile x (held in LDS buffer `buf`) from its raw
  // scores.  TAILT: the KIVI tail tile (fp16 values transposed at OFF_VT;
  // valid tokens t < ntail).
  // Masks of a tile that is not fully visible: raw scores of tokens that are
  // dead (or, in the tail tile, at or past ntail) or after the column's
  // position become -inf (key scale factors are never 0, see store_tile, so
  // the scaled score stays -inf).
  auto mask_scores = [&](int x, uint32_t live, f4 (&sc)[NQB][2]) __attribute__((always_inline)) {
    const int t0 = TILE * x;
    // bit 4 u + r: token 16 u + 4 j + r of the lane is live
    const uint32_t lvm = ((live >> (4 * j)) & 0xFu) | (((live >> (16 + 4 * j)) & 0xFu) << 4);
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
      // visible: live and 16 u + 4 j + r <= pos - t0 - 4 j =: lim
      const int lim = pos_c[cb] - t0 - 4 * j;
      const int n0 = min(max(lim + 1, 0), 4), n1 = min(max(lim - 15, 0), 4);
      const uint32_t vm = lvm & (((1u << n0) - 1u) | (((1u << n1) - 1u) << 4));
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[cb][u][r] = ((vm >> (4 * u + r)) & 1u) ? sc[cb][u][r] : -INFINITY;
    }
  };

  // Online softmax and P V of tile x (held in LDS buffer `buf`) from its
  // masked raw scores.  TAILT: the KIVI tail tile (fp16 values transposed at
  // OFF_VT).
  auto softmax_pv = [&](const uint8_t* buf, const f4 (&sc)[NQB][2], auto tailc) __attribute__((always_inline)) {
    constexpr bool TAILT = decltype(tailc)::value;
    const float* fk = reinterpret_cast<const float*>(buf + PL::OFF_FK);
    const float* fv = reinterpret_cast<const float*>(buf + PL::OFF_FV);
    // key scales of the lane's 8 tokens 16 u + 4 j + r (fp32, x sm_scale log2 e)
    f4 fk4[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (PL::PLANES) fk4[u] = f4{a.qscale, a.qscale, a.qscale, a.qscale};
      else fk4[u] = *reinterpret_cast<const f4*>(fk + 16 * u + 4 * j);
    }
    float p[NQB][2][4];
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
      float s[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[u][r] = sc[cb][u][r] * fk4[u][r];
          tmax = fmaxf(tmax, s[u][r]);
        }
      }
      tmax = max_j(tmax);
      const float m_new = fmaxf(m_run[cb], tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      if (__ballot(m_new != m_run[cb])) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[cb] - m_use);  // 0 on the first visible tile
        l_run[cb] *= alpha;
        l_err[cb] *= alpha;
#pragma unroll
        for (int g = 0; g < NCS; ++g) cs_run[cb][g] *= alpha;
#pragma unroll
        for (int m = 0; m < VS::NPV; ++m) acc[cb][m] *= alpha;
        m_run[cb] = m_new;
      }
      float lt = 0.f;  // this tile's sum
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[cb][u][r] = __builtin_amdgcn_exp2f(s[u][r] - m_use);  // exp2(-inf) = 0 for masked tokens
          lt += p[cb][u][r];
        }
      }
      two_sum_acc(l_run[cb], l_err[cb], lt);
    }
    // ---- P V on the matrix cores ----
    if constexpr (TAILT) {
      // fp16 values (unscaled): probability operand p as bf16 hi + lo in the
      // 8-bit slot order (dword q: rows 2 (q & 1), 2 (q & 1) + 1 of u = q >> 1)
      b8 ph[NQB], pl[NQB];
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb) {
        uint32_t ah[4], al[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = q >> 1, r0 = 2 * (q & 1);
          split_bf16x2(f2{p[cb][u][r0], p[cb][u][r0 + 1]}, ah[q], al[q]);
        }
        ph[cb] = __builtin_bit_cast(b8, u4{ah[0], ah[1], ah[2], ah[3]});
        pl[cb] = __builtin_bit_cast(b8, u4{al[0], al[1], al[2], al[3]});
      }
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m) {
        // channel of row n of block m (the layout of the page tiles' acc)
        const int ch = FV == F_INT4 ? 32 * (m >> 1) + 2 * n + (m & 1) : 16 * m + n;
        const uint8_t* vt = s_lds + PL::OFF_VT + ch * (TILE * 2);
        const u2 w0 = *reinterpret_cast<const u2*>(vt + 8 * j);       // tokens 4 j .. 4 j + 3
        const u2 w1 = *reinterpret_cast<const u2*>(vt + 32 + 8 * j);  // tokens 16 + 4 j ..
        uint32_t vh[4], vl[4];
        split_f16x2_bf16(w0.x, vh[0], vl[0]);
        split_f16x2_bf16(w0.y, vh[1], vl[1]);
        split_f16x2_bf16(w1.x, vh[2], vl[2]);
        split_f16x2_bf16(w1.y, vh[3], vl[3]);
        const b8 vhb = __builtin_bit_cast(b8, u4{vh[0], vh[1], vh[2], vh[3]});
        const b8 vlb = __builtin_bit_cast(b8, u4{vl[0], vl[1], vl[2], vl[3]});
#pragma unroll
        for (int cb = 0; cb < NQB; ++cb) {
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vhb, ph[cb], acc[cb][m], 0, 0, 0);
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vhb, pl[cb], acc[cb][m], 0, 0, 0);
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vlb, ph[cb], acc[cb][m], 0, 0, 0);
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vlb, pl[cb], acc[cb][m], 0, 0, 0);
        }
      }
    } else if constexpr (FV == F_INT4) {
      // dword q holds slots (q >> 1) 4 + (q & 1) and that + 2 (the INT4
      // value operand's token order [0, 2, 1, 3, 4, 6, 5, 7])
#pragma unroll
      for (int grp = 0; grp < VS::NG; ++grp) {
        b8 ph[NQB], pl[NQB];
#pragma unroll
        for (int cb = 0; cb < NQB; ++cb) {
          uint32_t ah[4], al[4];
          float cst = 0.f;  // this tile's operand sum (a short chain, see add_split)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int u = q >> 1, r0 = q & 1;
            const int ta = 16 * u + 4 * j + r0;
            split_bf16x2(f2{p[cb][u][r0] * fv[grp * TILE + ta], p[cb][u][r0 + 2] * fv[grp * TILE + ta + 2]},
                         ah[q], al[q]);
            cst = add_split(cst, ah[q], al[q]);
          }
          cs_run[cb][grp] += cst;
          ph[cb] = __builtin_bit_cast(b8, u4{ah[0], ah[1], ah[2], ah[3]});
          pl[cb] = __builtin_bit_cast(b8, u4{al[0], al[1], al[2], al[3]});
        }
        const i2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(buf + tbase + ((grp ^ tswz) << 4)));
        b8 ve, vo;
        value_operand_int4(raw, ve, vo);
#pragma unroll
        for (int cb = 0; cb < NQB; ++cb) {
          acc[cb][2 * grp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ve, ph[cb], acc[cb][2 * grp], 0, 0, 0);
          acc[cb][2 * grp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ve, pl[cb], acc[cb][2 * grp], 0, 0, 0);
          acc[cb][2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo, ph[cb], acc[cb][2 * grp + 1], 0, 0, 0);
          acc[cb][2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo, pl[cb], acc[cb][2 * grp + 1], 0, 0, 0);
        }
      }
    } else {
      // dword q holds slots 2 q, 2 q + 1: rows 2 (q & 1), 2 (q & 1) + 1 of u = q >> 1
      b8 ph[NQB], pl[NQB];
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb) {
        uint32_t ah[4], al[4];
        float cst = 0.f;  // this tile's operand sum (a short chain, see add_split)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = q >> 1, r0 = 2 * (q & 1);
          const int ta = 16 * u + 4 * j + r0;
          split_bf16x2(f2{p[cb][u][r0] * fv[ta], p[cb][u][r0 + 1] * fv[ta + 1]}, ah[q], al[q]);
          if constexpr (FV == F_INT8) cst = add_split(cst, ah[q], al[q]);
        }
        if constexpr (FV == F_INT8) cs_run[cb][0] += cst;
        ph[cb] = __builtin_bit_cast(b8, u4{ah[0], ah[1], ah[2], ah[3]});
        pl[cb] = __builtin_bit_cast(b8, u4{al[0], al[1], al[2], al[3]});
      }
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m) {
        b8 vop;
        if constexpr (PL::V16) {
          const int ta = 4 * j + (n >> 2);  // token row of the first read; the second reads ta + 16
          const int off = PL::OFF_V + ta * PL::VRB + ((m ^ v16swz<D>(ta)) << 5) + 8 * (n & 3);
          const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(buf + off));
          const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(buf + off + 16 * PL::VRB));
          const u2 w0 = __builtin_bit_cast(u2, lo), w1 = __builtin_bit_cast(u2, hi);
          vop = __builtin_bit_cast(b8, u4{w0.x, w0.y, w1.x, w1.y});
        } else {
          const i2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(buf + tbase + ((m ^ tswz) << 4)));
          vop = value_operand_biased<FV>(raw);
        }
#pragma unroll
        for (int cb = 0; cb < NQB; ++cb) {
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, ph[cb], acc[cb][m], 0, 0, 0);
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pl[cb], acc[cb][m], 0, 0, 0);
        }
      }
    }
  };

  // Remove the value-operand offset from acc now and restart the operand
  // sums (INT8 / INT4 values): acc holds 2^-133 sum P u with u = c + 128
  // (INT8) or c + 8 (INT4; odd channels 16 u), so the offset part is
  // 2^-126 cs (2^-130 cs for even INT4 channels), cs = the column's operand
  // sum since the last call.  Done every 16 tiles, it keeps acc near the size
  // of the signal: a long chain of MFMA accumulations into a large offset
  // drifts (the accumulation does not round like IEEE adds), and the offset
  // would multiply that drift.
  auto remove_offset = [&]() __attribute__((always_inline)) {
    if constexpr (!VFP8) {
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb) {
#pragma unroll
        for (int g = 0; g < NCS; ++g) {
          const float cs = sum_j(cs_run[cb][g]);
          cs_run[cb][g] = 0.f;
          if constexpr (FV == F_INT8) {
#pragma unroll
            for (int m = 0; m < VS::NPV; ++m)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[cb][m][r] = __builtin_fmaf(cs, -0x1p-126f, acc[cb][m][r]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              acc[cb][2 * g][r] = __builtin_fmaf(cs, -0x1p-130f, acc[cb][2 * g][r]);
              acc[cb][2 * g + 1][r] = __builtin_fmaf(cs, -0x1p-126f, acc[cb][2 * g + 1][r]);
            }
          }
        }
      }
    }
  };

  // ---- page tiles, software-pipelined over three LDS buffers: in the step
  //      of tile x the waves issue the scores of tile x + 1, then run the
  //      softmax and P V of tile x (so the matrix cores work on x + 1 while
  //      the vector units work on x), while the loads of tile x + 2 are in
  //      flight; tile x + 2 is stored at the end of the step. -------------------
  auto lbuf = [&](int i) __attribute__((always_inline)) { return s_lds + i * PL::BUF; };
  if (ntm > 0) {
    PRegs<FK, FV, D> regs;
    const int id0 = load_id(0), id1 = load_id(min(1, ntm - 1));
    int id2 = load_id(min(2, ntm - 1)), id3 = load_id(min(3, ntm - 1));
    const uint32_t live0 = load_tile(0, id0, regs);
    store_tile(regs, live0, lbuf(0));
    const uint32_t live1 = load_tile(min(1, ntm - 1), id1, regs);
    store_tile(regs, live1, lbuf(1));
    __syncthreads();
    f4 sc_next[NQB][2];
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) sc_next[cb][0] = sc_next[cb][1] = f4{0.f, 0.f, 0.f, 0.f};
    scores(lbuf(0), 0, sc_next, std::false_type{});
    uint32_t live_cur = live0, live_nx = live1;
    int bx = 0;  // buffer of tile x (x mod 3)
    for (int x = 0; x < ntm; ++x) {
      const int b1 = bx == 2 ? 0 : bx + 1, b2 = b1 == 2 ? 0 : b1 + 1;
      // tile x + 2 (the last tile again past the end: loaded and stored into
      // the free buffer, never read), then the ids of tile x + 4
      const int x2 = min(x + 2, ntm - 1);
      const uint32_t live_n2 = load_tile(x2, id2, regs);
      id2 = id3;
      id3 = load_id(min(x + 4, ntm - 1));
      f4 sc_cur[NQB][2];
#pragma unroll
      for (int cb = 0; cb < NQB; ++cb) {
        sc_cur[cb][0] = sc_next[cb][0];
        sc_cur[cb][1] = sc_next[cb][1];
      }
      if (x + 1 < ntm) scores(lbuf(b1), x + 1, sc_next, std::false_type{});
      if (pos_hi >= TILE * x) {  // some query of the wave sees the tile
        if (live_cur != 0xFFFFFFFFu || TILE * x + TILE - 1 > pos_lo) mask_scores(x, live_cur, sc_cur);
        softmax_pv(lbuf(bx), sc_cur, std::false_type{});
      }
      if ((x & 15) == 15) remove_offset();
      store_tile(regs, live_n2, lbuf(b2));
      __syncthreads();
      live_cur = live_nx;
      live_nx = live_n2;
      bx = b1;
    }
  }

  // ---- back to true units: remove the value-operand offset and factors ----
  // (P = 2^60 p s and value operands u 2^-133 with u = c + 128 (INT8): the
  // sum is 2^73 acc - 2^-53 cs; INT4 (u = c + 8): even channels 2^73 acc -
  // 2^-57 cs, odd channels (16 u 2^-133) 2^69 acc - 2^-57 cs; cs = the sum of
  // the probability operands of the column, per value group)
  if constexpr (!VFP8) {
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
#pragma unroll
      for (int g = 0; g < NCS; ++g) {
        const float cs = sum_j(cs_run[cb][g]);
        if constexpr (FV == F_INT8) {
          const float corr = cs * 0x1p-53f;
#pragma unroll
          for (int m = 0; m < VS::NPV; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[cb][m][r] = __builtin_fmaf(acc[cb][m][r], 0x1p73f, -corr);
        } else {
          const float corr = cs * 0x1p-57f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[cb][2 * g][r] = __builtin_fmaf(acc[cb][2 * g][r], 0x1p73f, -corr);
            acc[cb][2 * g + 1][r] = __builtin_fmaf(acc[cb][2 * g + 1][r], 0x1p69f, -corr);
          }
        }
      }
    }
  }

  // channel of acc[cb][m][r] in lane group j
  auto channel = [&](int m, int r) __attribute__((always_inline)) {
    return FV == F_INT4 ? 32 * (m >> 1) + 8 * j + 2 * r + (m & 1) : 16 * m + 4 * j + r;
  };

  // ---- rotated values: the weighted sum of stored rows y = H (sigma x) is
  //      rotated back, x = sigma (H y) / D.  Per column, the channel bits are
  //      split between the lane's registers (m, r) and the lane group j
  //      (lanes ^ 16, ^ 32); a Hadamard transform is a butterfly over each
  //      bit, in any order.
  if (a.rot_v) {
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) {
      float y[VS::NPV * 4];
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[4 * m + r] = acc[cb][m][r];
#pragma unroll
      for (int s = 1; s < VS::NPV * 4; s <<= 1) {
#pragma unroll
        for (int i = 0; i < VS::NPV * 4; ++i) {
          if (i & s) continue;
          const float u0 = y[i], u1 = y[i + s];
          y[i] = u0 + u1;
          y[i + s] = u0 - u1;
        }
      }
#pragma unroll
      for (int mk = 16; mk <= 32; mk <<= 1) {
#pragma unroll
        for (int i = 0; i < VS::NPV * 4; ++i) {
          const float pv = __shfl_xor(y[i], mk);
          y[i] = (lane & mk) ? pv - y[i] : y[i] + pv;
        }
      }
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = channel(m, r);
          uint32_t wd = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) wd = (c >> 5) == k ? a.rot_signs[k] : wd;
          acc[cb][m][r] = (((wd >> (c & 31)) & 1) ? -y[4 * m + r] : y[4 * m + r]) * (1.0f / D);
        }
      }
    }
  }

  // ---- KIVI: the fp16 tail (last L mod 32 tokens, tail row b) ---------------
  if (tail) {
    const int ntail = L - Lq;
    const int t = tid >> 3, cg = tid & 7;
    const bool lt = t < ntail;
    const size_t trow_off = lt ? (((size_t)b * TILE + t) * a.H + h) * D + cg * PL::KE : 0;
    uint8_t* buf = s_lds;  // every wave has passed the last page tile's barrier
    u4 kr[PL::KM], vr[PL::KM];
#pragma unroll
    for (int k = 0; k < PL::KM; ++k) {
      const u4 kk = *reinterpret_cast<const u4*>(a.k_tail + trow_off + 8 * k);
      const u4 vv = *reinterpret_cast<const u4*>(a.v_tail + trow_off + 8 * k);
      kr[k] = lt ? kk : u4{0u, 0u, 0u, 0u};
      vr[k] = lt ? vv : u4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < PL::KM; ++k) {
      const int c = cg * PL::KM + k;
      reinterpret_cast<u4*>(buf + PL::OFF_K)[t * PL::KCH + (c ^ kswz<PL::KCH>(t))] = kr[k];
    }
    uint16_t* vt = reinterpret_cast<uint16_t*>(s_lds + PL::OFF_VT);
#pragma unroll
    for (int e = 0; e < PL::KE; ++e) {
      const uint32_t w = u4_word(vr[e / 8], (e % 8) / 2);
      vt[(cg * PL::KE + e) * TILE + t] = (uint16_t)(w >> (16 * (e & 1)));
    }
    __syncthreads();
    f4 sc[NQB][2];
#pragma unroll
    for (int cb = 0; cb < NQB; ++cb) sc[cb][0] = sc[cb][1] = f4{0.f, 0.f, 0.f, 0.f};
    scores(buf, Lq / TILE, sc, std::true_type{});
    if (pos_hi >= Lq) {
      mask_scores(Lq / TILE, ntail >= 32 ? 0xFFFFFFFFu : (1u << ntail) - 1u, sc);
      softmax_pv(buf, sc, std::true_type{});
    }
  }

  // ---- out = acc / l, fp16 -------------------------------------------------
#pragma unroll
  for (int cb = 0; cb < NQB; ++cb) {
    const float l = sum_j(l_run[cb]) + sum_j(l_err[cb]);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    if (Rw + 16 * cb + n >= rows) continue;
    uint16_t* o = a.out + qrow[cb] * D;
    if constexpr (FV == F_INT4) {
#pragma unroll
      for (int grp = 0; grp < VS::NG; ++grp) {
        u4 w;
        uint32_t ww[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ww[r] = f2h_bits(acc[cb][2 * grp][r] * inv) | (f2h_bits(acc[cb][2 * grp + 1][r] * inv) << 16);
        w = u4{ww[0], ww[1], ww[2], ww[3]};
        *reinterpret_cast<u4*>(o + 32 * grp + 8 * j) = w;
      }
    } else {
#pragma unroll
      for (int m = 0; m < VS::NPV; ++m) {
        const u2 w = {f2h_bits(acc[cb][m][0] * inv) | (f2h_bits(acc[cb][m][1] * inv) << 16),
                      f2h_bits(acc[cb][m][2] * inv) | (f2h_bits(acc[cb][m][3] * inv) << 16)};
        *reinterpret_cast<u2*>(o + 16 * m + 4 * j) = w;
      }
    }
  }
}

namespace {

template <int FK, int FV, int D, bool ROTQ>
hipError_t prefill_launch(const PrefillArgs& a, hipStream_t s) {
  using PL = PLayout<FK, FV, D>;
  static_assert(PL::LDS <= 160 * 1024, "LDS");
  if constexpr (PL::LDS > 64 * 1024) {
    static bool set = false;
    if (!set) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<FK, FV, D, ROTQ>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, PL::LDS);
      if (e != hipSuccess) return e;
      set = true;
    }
  }
  const unsigned wgs = (unsigned)(((int64_t)a.n_wg + 7) / 8 * 8);
  hipLaunchKernelGGL((prefill_kernel<FK, FV, D, ROTQ>), dim3(wgs), dim3(PL::THREADS), PL::LDS, s, a);
  return hipGetLastError();
}

template <int FK, int FV, bool ROTQ>
hipError_t prefill_by_dim(int D, const PrefillArgs& a, hipStream_t s) {
  switch (D) {
    case 64: return prefill_launch<FK, FV, 64, ROTQ>(a, s);
    case 128: return prefill_launch<FK, FV, 128, ROTQ>(a, s);
    case 256: return prefill_launch<FK, FV, 256, ROTQ>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int FK, bool ROTQ>
hipError_t prefill_for_keys_rot(int fv, int D, const PrefillArgs& a, hipStream_t s) {
  switch (fv) {
    case F_INT8: return prefill_by_dim<FK, F_INT8, ROTQ>(D, a, s);
    case F_FP8: return prefill_by_dim<FK, F_FP8, ROTQ>(D, a, s);
    case F_INT4: return prefill_by_dim<FK, F_INT4, ROTQ>(D, a, s);
    case F_E5M2: return prefill_by_dim<FK, F_E5M2, ROTQ>(D, a, s);
  }
  return hipErrorInvalidValue;
}

// Prefill launch for key format FK, any value format, rotated keys or not
// (one instantiation per translation unit kvq_prefill_k*.hip).
template <int FK>
hipError_t prefill_for_keys(int fv, int D, bool rot, const PrefillArgs& a, hipStream_t s) {
  if constexpr (FK == F_KIVI) {
    if (rot) return hipErrorInvalidValue;
    return prefill_for_keys_rot<FK, false>(fv, D, a, s);
  } else {
    return rot ? prefill_for_keys_rot<FK, true>(fv, D, a, s) : prefill_for_keys_rot<FK, false>(fv, D, a, s);
  }
}

}  // namespace

}  // namespace kvq
