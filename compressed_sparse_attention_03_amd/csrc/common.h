// Device helpers shared by the libcsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA_WAVE 64

namespace csa {

// Workgroup barrier that orders LDS only: the LDS accesses of every wave before it are complete
// and visible to every wave after it.  Outstanding global loads and stores are not waited for
// (the workgroup-scope fences of __syncthreads wait for them on this target).  Every barrier in
// these kernels orders LDS traffic only: no workgroup reads global memory another of its waves
// wrote in the same launch.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- bf16 storage ---------------------------------------------------------------------------
// Entries visible at position x - 1, i.e. x / m for a token count x >= 0 (C division): 32-bit
// unsigned division whenever x fits, which is every real position (a 64-bit division by a runtime
// value is a long scalar sequence in a kernel prologue).
__device__ __forceinline__ int64_t div_count(int64_t x, int m) {
  if (x >= 0 && x <= int64_t(0xffffffffu)) return int64_t(uint32_t(x) / uint32_t(m));
  return x / m;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// ---- low-precision encoders (the rules stated in csa.h for csa_quantize_keys) ---------------
// e4m3 (bias 7, largest finite 448): round to nearest even, saturate, keep the sign bit.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a < 448.0f)) return sign | 0x7eu;                  // saturate (also catches NaN input)
  if (a < 0.015625f) {                                     // below 2^-6: multiples of 2^-9
    uint32_t k = uint32_t(rintf(a * 512.0f));              // exact scaling, RNE
    return sign | k;                                       // k == 8 is the code of 2^-6
  }
  uint32_t u = __float_as_uint(a);
  uint32_t r = u + 0x7ffffu + ((u >> 20) & 1u);            // RNE to 3 mantissa bits
  uint32_t e = (r >> 23) - 127u + 7u;
  uint32_t code = (e << 3) | ((r >> 20) & 7u);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

// e2m1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}: nearest, ties to the even code, saturate at 6.
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  float a = fabsf(x);
  uint32_t c;
  if (a <= 0.25f) c = 0;            // tie at .25 -> 0 (even)
  else if (a < 0.75f) c = 1;        // (.25,.75) -> .5
  else if (a <= 1.25f) c = 2;       // tie .75 -> 1.0 (even), tie 1.25 -> 1.0
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;        // tie 1.75 -> 2 (even), tie 2.5 -> 2
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;        // tie 3.5 -> 4, tie 5 -> 4
  else c = 7;                       // (5, inf) -> 6 (NaN input is not expected)
  return sign | c;
}

// Smallest e with amax <= 448 * 2^e, clamped to [-126, 127]; 0 for amax == 0.
__device__ __forceinline__ int e4m3_row_exp(float amax) {
  if (amax == 0.0f) return 0;
  int ex = int((__float_as_uint(amax) >> 23) & 0xff);
  if (ex == 0) return -126;                      // every fitting e is <= -126 for amax < 2^-126
  int e = ex - 127 - 8;                          // amax / 2^e lies in [256, 512)
  if (amax > ldexpf(448.0f, e)) ++e;
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// e8m0 byte of the MX scale for a block maximum: clamp(floor(log2 amax) - 2 + 127, 0, 254).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  uint32_t u = __float_as_uint(amax);
  int ex = int((u >> 23) & 0xff);                 // floor(log2) + 127 for normals; 0 for 0/subnormal
  int b = ex - 2;                                 // biased exponent of 2^(floor(log2 amax) - 2)
  if (ex == 0) b = 0;
  return uint32_t(b < 0 ? 0 : (b > 254 ? 254 : b));
}

// ---- order-preserving keys for selection ---------------------------------------------------
// High word: float score mapped to an unsigned order; low word: ~index so equal scores prefer
// the lower index.  Key 0 never occurs for a real entry (marks "no entry").
__device__ __forceinline__ uint32_t score_order(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float s, uint32_t idx) {
  return (uint64_t(score_order(s)) << 32) | uint64_t(~idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~uint32_t(k); }

// ---- wave / block reductions ---------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---- rotary angles ---------------------------------------------------------------------------
// Pair u of an r-dim rotation at position pos turns by pos * base^(-2u/r) radians.  rope_rate
// gives -2 log2(base) / r once per call site; rope_cos_sin forms the angle in double, measured in
// turns, and keeps its fractional part there (so positions near 2^21 keep full fp32 accuracy of
// the reduced angle); the hardware sine and cosine (v_sin_f32 / v_cos_f32, whose argument is in
// turns) take the fp32 fraction.
__device__ __forceinline__ double rope_rate(int r, double log2_base) { return -2.0 * log2_base / double(r); }
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int u, double rate, float *c, float *s) {
  constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
  const double turns = double(pos) * (exp2(double(u) * rate) * kInvTwoPi);
  const float f = float(turns - rint(turns));                   // in [-1/2, 1/2]
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}

}  // namespace csa
