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

// Orders one wave's LDS accesses: its writes before the call are seen by its reads after it (a
// wave's LDS operations complete in order; the fences keep the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// A workgroup barrier after which every wave's LDS writes are visible, without waiting for the
// wave's global loads still in flight (the memory-model fence of lds_barrier makes the compiler
// wait for those as well): each wave's LDS operations have completed (lgkmcnt 0) when it arrives.
__device__ __forceinline__ void lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- hand-over between the workgroups of one launch -------------------------------------------
// Several kernels let the last of a group of workgroups to finish (decided by a device-scope atomic
// counter) combine what the others produced.  The handed-over values are written and read with the
// coherent cache policy (sc1) -- the policy of device-scope atomic stores and loads, which keeps
// them at the device's coherence point rather than in one XCD's L2 -- so no L2 write-back or
// invalidation is needed: a writer waits until its coherent stores have completed and only then
// counts itself in; the last workgroup reads them back coherently after the count.  (A device-scope
// release fence would write back the whole L2 of the XCD, which costs microseconds when every
// workgroup of a launch does it.)  Counters sit on separate 256-byte lines so that arrivals for
// different groups do not queue behind each other.
constexpr int kCoherent = 16;                         // buffer cache-policy operand: sc1
constexpr int kCounterStride = 64;                    // ints between two arrival counters
constexpr int kRawBufferDesc3 = 0x00020000;           // raw-buffer descriptor word 3 (32-bit format)

__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

__device__ __forceinline__ void store_coherent(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_coherent(const int *p) {
  return __hip_atomic_load(const_cast<int *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte coherent accesses through a buffer resource over [base, base + bytes) (base uniform).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_region(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), short(0), int(bytes), kRawBufferDesc3);
}
__device__ __forceinline__ uint4 load_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ void store_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                         off, 0, kCoherent);
}

// Count the calling workgroup in on `counter` after every wave's coherent stores have completed.
// Returns true (in every thread) for the workgroup that arrives last, which also resets the counter
// to zero for the next launch.  `flag` is an LDS int.  No workgroup waits for another.
__device__ __forceinline__ bool arrive_last(int *counter, int group_size, int *flag) {
  wait_stores();
  lds_barrier();
  if (threadIdx.x == 0) {
    const int before = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = before == group_size - 1;
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  lds_barrier();
  return *flag != 0;
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
// The same sum in every lane by DPP inside rows of 16 lanes and the gfx950 half-wave and row swaps
// across them (a fixed order; no LDS round trips).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));  // row half mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));  // row mirror
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Maximum over aligned groups of LANES (1, 2, 4, 8 or 16) consecutive lanes, in every lane of the
// group: quad swaps, then the half-row and row mirrors (DPP, no LDS round trip; a maximum does not
// depend on the order it is taken in).
template <int LANES>
__device__ __forceinline__ float group_max_dpp(float v) {
  static_assert(LANES == 1 || LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16, "a power of two up to 16");
  if constexpr (LANES >= 2) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));
  if constexpr (LANES >= 4) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));
  if constexpr (LANES >= 8) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
  if constexpr (LANES >= 16) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
  return v;
}
// The maximum over the wave, in every lane (rows of 16 by DPP, then the half-wave and row swaps).
__device__ __forceinline__ float wave_max(float v) {
  v = group_max_dpp<16>(v);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---- rotary angles ---------------------------------------------------------------------------
// Pair u of an r-dim rotation at position pos turns by pos * base^(-2u/r) radians.  rope_rate
// gives -2 log2(base) / r once per call site; rope_cos_sin forms the angle in double, measured in
// turns, and keeps its fractional part there (so positions near 2^21 keep full fp32 accuracy of
// the reduced angle); the hardware sine and cosine (v_sin_f32 / v_cos_f32, whose argument is in
// turns) take the fp32 fraction.
__device__ __forceinline__ double rope_rate(int r, double log2_base) { return -2.0 * log2_base / double(r); }
// pair u's turns per position, base^(-2u/r) / (2 pi): independent of the position, so it can be
// formed before the position is known
__device__ __forceinline__ double rope_turns_per_pos(int u, double rate) {
  constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
  return exp2(double(u) * rate) * kInvTwoPi;
}
__device__ __forceinline__ void rope_cos_sin_f(int64_t pos, double turns_per_pos, float *c, float *s) {
  const double turns = double(pos) * turns_per_pos;
  const float f = float(turns - rint(turns));                   // in [-1/2, 1/2]
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int u, double rate, float *c, float *s) {
  rope_cos_sin_f(pos, rope_turns_per_pos(u, rate), c, s);
}

}  // namespace csa
