// Device helpers for gfx950: fp16/fp8 conversions, exact quotients, lane
// reductions.  Everything here is plain HIP for CDNA4 (wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/kvq.h"

namespace kvq {

enum Fmt : int {
  F_INT8 = KVQ_INT8,
  F_FP8 = KVQ_FP8_E4M3FN,
  F_INT4 = KVQ_INT4_G32,
  F_KIVI = KVQ_INT4_KIVI,
  F_E5M2 = KVQ_FP8_E5M2
};

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((unsigned short)bits16));
}
// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint32_t f2h_bits(float x) {
  return (uint32_t)__half_as_ushort(__float2half_rn(x));
}

// fp16 bits of an fp32 value computed just before, rounded twice as the
// format requires: first to fp32 (the computation's own rounding), then to
// fp16.  The empty asm pins the fp32 result in a register; without it the
// compiler fuses a final FMA and the conversion into one mixed-precision FMA
// with an fp16 result (v_fma_mixlo_f16), which rounds the exact value once,
// straight to fp16 -- a different result whenever the fp32 value is an exact
// fp16 tie (it happens for quotients of fp32 numerators, such as the rows of
// a rotated cache).
__device__ __forceinline__ uint32_t f2h_bits_of_f32(float x) {
  asm volatile("" : "+v"(x));
  return f2h_bits(x);
}

// Eight fp16 values packed in a uint4 -> fp32.
__device__ __forceinline__ void unpack8(const uint4& u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = h2f(w[i] & 0xFFFFu);
    x[2 * i + 1] = h2f(w[i] >> 16);
  }
}

// IEEE binary32 quotient x / s (round to nearest even) from r = RN(1/s):
// y0 = RN(x r) is within one ulp of x/s, the residual y0 s - x is exact under
// FMA, and RN(y0 - r * residual) is the correctly rounded quotient
// (Markstein's theorem; "Handbook of Floating-Point Arithmetic", division by
// FMA).  Written with the residual's sign flipped so that x = -0 gives -0.
// Checked bit-exact (signed zeros included) against IEEE division on gfx950
// for every fp16 x and every positive finite fp16 s with r from recip_fp16.
__device__ __forceinline__ float exact_div(float x, float s, float r) {
  const float y0 = x * r;
  const float e = __builtin_fmaf(y0, s, -x);
  return __builtin_fmaf(e, -r, y0);
}

// RN(1/s) for a positive finite fp16 value s: the hardware reciprocal and
// one Newton step, e = 1 - s r0 (exact under FMA), r0 + r0 e.  Equal to IEEE
// 1/s for every positive finite fp16 s (checked exhaustively on gfx950).
__device__ __forceinline__ float recip_fp16(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r0, 1.0f);
  return __builtin_fmaf(r0, e, r0);
}

// Round-to-nearest-even integer of |y| < 2^22 in the low bits of the result:
// y + 1.5 2^23 is rounded by the add (ulp 1), and its low 8 bits are the
// integer's two's-complement low byte.
__device__ __forceinline__ uint32_t rne_low_bits(float y) {
  return __builtin_bit_cast(uint32_t, y + 12582912.0f);
}

// Four fp32 values -> four OCP E4M3FN bytes, nearest-even (gfx950 hardware
// conversion).  Callers clamp to [-448, 448] first, which makes the result
// the saturating conversion.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// Four values (within +-57344) to OCP E5M2 bytes, nearest-even (v_cvt_pk_bf8_f32).
__device__ __forceinline__ uint32_t bf8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Lane exchange within rows of 16 lanes (DPP): quad_perm [1,0,3,2] (xor 1),
// [2,3,0,1] (xor 2), row_half_mirror (lane i of 8 reads 7 - i), row_mirror
// (lane i of 16 reads 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Max over aligned groups of N consecutive lanes (N a power of two <= 64).
// Up to 16 lanes: butterflies on the DPP exchanges (after the two quad
// steps a lane holds its quad's max, the half-row mirror pairs the two
// quads of 8 lanes, the row mirror the two halves of 16); beyond, shuffles.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<0x140>(v));
#pragma unroll
  for (int m = 16; m < N; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Exchange of a double with lane ^ M (M < 32) through ds_swizzle (bitmask
// mode: and_mask 0x1F, xor_mask M).
template <int M>
__device__ __forceinline__ double swz_xor(double v) {
  constexpr int pat = (M << 10) | 0x1F;
  const int lo = __builtin_amdgcn_ds_swizzle(__double2loint(v), pat);
  const int hi = __builtin_amdgcn_ds_swizzle(__double2hiint(v), pat);
  return __hiloint2double(hi, lo);
}

// Walsh-Hadamard transform y = H x of one row spread over LPR consecutive
// lanes (aligned, LPR <= 32), 8 channels per lane: lane l of the row holds
// channels 8 l .. 8 l + 7 (fp16 values, the caller has applied the random
// signs).  H is the Sylvester matrix: for each index bit, the pair
// (i, i + 2^k) with bit k of i clear becomes (x_i + x_j, x_i - x_j).  Bits
// 0-2 of the channel are inside the lane, bits 3.. are the lane bits.  Every
// partial sum is a sum of at most 256 fp16 values, exact in float64, so the
// result is the exact transform.
template <int LPR>
__device__ __forceinline__ void fwht_row8(const float (&x)[8], int lir, double (&y)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = (double)x[j];
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & s) continue;
      const double a = y[j], b = y[j + s];
      y[j] = a + b;
      y[j + s] = a - b;
    }
  }
  // lane bits: the lower lane of a pair keeps own + partner, the upper one
  // partner - own
  auto stage = [&](auto mconst) __attribute__((always_inline)) {
    constexpr int M = decltype(mconst)::value;
    const double sg = (lir & M) ? -1.0 : 1.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = __builtin_fma(y[j], sg, swz_xor<M>(y[j]));
  };
  if constexpr (LPR >= 2) stage(std::integral_constant<int, 1>{});
  if constexpr (LPR >= 4) stage(std::integral_constant<int, 2>{});
  if constexpr (LPR >= 8) stage(std::integral_constant<int, 4>{});
  if constexpr (LPR >= 16) stage(std::integral_constant<int, 8>{});
  if constexpr (LPR >= 32) stage(std::integral_constant<int, 16>{});
}

// s + e += x with the rounding error of the add kept in e (TwoSum, six
// IEEE adds): a running sum of probabilities that starts with one large term
// would otherwise drop every later term below half its ulp -- all of them
// positive, so the sum would come out low, not just noisy.
__device__ __forceinline__ void two_sum_acc(float& s, float& e, float x) {
  const float t = s + x;
  const float bx = t - s;
  e += (s - (t - bx)) + (x - bx);
  s = t;
}

// Record a device-side data error: the lowest lane of the wave whose `bad`
// is set ORs `bit` into the error word (one vector atomic per wave at most).
__device__ __forceinline__ void report_error(uint32_t* err, bool bad, uint32_t bit) {
  const uint64_t m = __ballot(bad);
  if (m != 0 && (threadIdx.x & 63u) == (uint32_t)(__ffsll((unsigned long long)m) - 1))
    __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kvq
