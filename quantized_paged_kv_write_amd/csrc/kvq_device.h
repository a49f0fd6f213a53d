// Device helpers for gfx950: fp16/fp8 conversions, exact quotients, lane
// reductions.  Everything here is plain HIP for CDNA4 (wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

enum Fmt : int { F_INT8 = KVQ_INT8, F_FP8 = KVQ_FP8_E4M3FN, F_INT4 = KVQ_INT4_G32, F_KIVI = KVQ_INT4_KIVI };

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((unsigned short)bits16));
}
// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint32_t f2h_bits(float x) {
  return (uint32_t)__half_as_ushort(__float2half_rn(x));
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
// y0 = RN(x r) is within one ulp of x/s, the residual x - y0 s is exact under
// FMA, and RN(y0 + r * residual) is the correctly rounded quotient
// (Markstein's theorem; "Handbook of Floating-Point Arithmetic", division by
// FMA).  Checked bit-exact against IEEE division for every fp16 x and every
// fp16 s, and on 1.4e9 random fp32 differences of fp16 values.
__device__ __forceinline__ float exact_div(float x, float s, float r) {
  const float y0 = x * r;
  const float e = __builtin_fmaf(-y0, s, x);
  return __builtin_fmaf(e, r, y0);
}

// Four fp32 values -> four OCP E4M3FN bytes, nearest-even (gfx950 hardware
// conversion).  Callers clamp to [-448, 448] first, which makes the result
// the saturating conversion.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Max / sum over groups of N consecutive lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
template <int N>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) v = fminf(v, __shfl_xor(v, m));
  return v;
}

}  // namespace kvq
