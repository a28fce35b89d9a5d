// KV compressor: per-channel softmax pooling of each entry's tokens, RMSNorm, partial RoPE.
//
// "DeepSeek-V4: Million-Token Context" (codexsims explainer), CSA walk-through: each group of m
// tokens is pooled into one entry with softmax weights that are learned; HCA walk-through: HCA
// pools disjoint runs of m' = 128 tokens.  "Follow the white rabbit" (sambatista.com), CSA paragraph: an entry's pooling
// reaches back over the preceding group as well; HCA paragraph: the pooling weights vary by channel.
// paperlayer summary, section 2.3 "Other details": RMSNorm on compressed entries.
//
// Layout: one workgroup (4 waves) per entry.  A lane owns CPL = d/64 consecutive channels, so a
// wave reads a 2*d-byte token row with one coalesced vector load per lane.  The waves split the
// entry's tokens; each keeps an online softmax (running max, running sum, weighted sum) per
// channel in registers, and the four states are merged through LDS.  Exponentials are exp2 of
// log2(e)-scaled logits.
#include "common.h"
#include "internal.h"

namespace csa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// A token row's CPL bf16 values as loaded, unpacked at use.
template <int CPL>
struct RawRow {
  uint32_t w[(CPL + 1) / 2];
  __device__ __forceinline__ float at(int j) const {
    if constexpr (CPL == 1) return bf16lo(w[0]);
    return (j & 1) ? bf16hi(w[j >> 1]) : bf16lo(w[j >> 1]);
  }
};
template <int CPL>
__device__ __forceinline__ void load_raw(const uint16_t *p, RawRow<CPL> &r) {
  if constexpr (CPL == 1) {
    r.w[0] = *p;
  } else if constexpr (CPL == 2) {
    r.w[0] = *reinterpret_cast<const uint32_t *>(p);
  } else if constexpr (CPL == 4) {
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    r.w[0] = x.x; r.w[1] = x.y;
  } else {
#pragma unroll
    for (int q = 0; q < CPL / 8; ++q) {
      const uint4 x = reinterpret_cast<const uint4 *>(p)[q];
      r.w[4 * q] = x.x; r.w[4 * q + 1] = x.y; r.w[4 * q + 2] = x.z; r.w[4 * q + 3] = x.w;
    }
  }
}

template <int CPL>
__device__ __forceinline__ void store_raw(uint16_t *p, const RawRow<CPL> &r) {
  if constexpr (CPL == 1) {
    *p = uint16_t(r.w[0]);
  } else if constexpr (CPL == 2) {
    *reinterpret_cast<uint32_t *>(p) = r.w[0];
  } else if constexpr (CPL == 4) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(r.w[0], r.w[1]);
  } else {
#pragma unroll
    for (int q = 0; q < CPL / 8; ++q)
      reinterpret_cast<uint4 *>(p)[q] = make_uint4(r.w[4 * q], r.w[4 * q + 1], r.w[4 * q + 2], r.w[4 * q + 3]);
  }
}

template <int CPL>
__device__ __forceinline__ void store_row(uint16_t *p, const float (&v)[CPL]) {
  if constexpr (CPL == 1) {
    *p = f32_to_bf16(v[0]);
  } else if constexpr (CPL == 2) {
    *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(v[0], v[1]);
  } else if constexpr (CPL == 4) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  } else {
#pragma unroll
    for (int q = 0; q < CPL / 8; ++q)
      reinterpret_cast<uint4 *>(p)[q] =
          make_uint4(pack_bf16x2(v[8 * q + 0], v[8 * q + 1]), pack_bf16x2(v[8 * q + 2], v[8 * q + 3]),
                     pack_bf16x2(v[8 * q + 4], v[8 * q + 5]), pack_bf16x2(v[8 * q + 6], v[8 * q + 7]));
  }
}

// The RMSNorm weights of a lane's channels, loaded once per workgroup with one vector load.
// Without weights (g NULL) the load reads `any` (a valid row of at least d values) and the
// weights are ones.
template <int CPL>
struct NormWeights {
  RawRow<CPL> w;
  bool has;
};
template <int CPL>
__device__ __forceinline__ NormWeights<CPL> load_norm_weights(const uint16_t *g, const uint16_t *any, int lane) {
  NormWeights<CPL> n;
  n.has = g != nullptr;
  load_raw<CPL>((g ? g : any) + lane * CPL, n.w);
  return n;
}

// Quantise-on-write of a key row held as CPL consecutive channels per lane (one wave, d = 64 CPL,
// CPL >= 2), the values already rounded to bf16: fp32 copy (format 0), fp8 e4m3 with a
// power-of-two row scale (1), MXFP4 with 32/CPL lanes per block of 32 (2) -- the encoders and
// rules of csa_quantize_keys.
template <int CPL>
__device__ __forceinline__ void encode_key_lanes(const float (&v)[CPL], int fmt, int d, void *codes, void *scales,
                                                 int64_t row, int lane) {
  static_assert(CPL >= 2 && CPL <= 16, "two to sixteen channels per lane");
  if (fmt == 0) {
    float *dst = static_cast<float *>(codes) + row * d + lane * CPL;
#pragma unroll
    for (int j = 0; j < CPL; j += 2) *reinterpret_cast<float2 *>(dst + j) = make_float2(v[j], v[j + 1]);
  } else if (fmt == 1) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = wave_max(amax);
    const int e = e4m3_row_exp(amax);
    const float inv = ldexpf(1.0f, -e);
    uint8_t *dst = static_cast<uint8_t *>(codes) + row * d + lane * CPL;
#pragma unroll
    for (int j = 0; j < CPL; j += 2)
      *reinterpret_cast<uint16_t *>(dst + j) = uint16_t(f32_to_e4m3(v[j] * inv) | (f32_to_e4m3(v[j + 1] * inv) << 8));
    if (lane == 0) static_cast<float *>(scales)[row] = ldexpf(1.0f, e);
  } else {
    constexpr int LB = 32 / CPL;                    // lanes per block of 32 values
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = group_max_dpp<LB>(amax);
    const uint32_t sb = mx_scale_byte(amax);
    const float inv = ldexpf(1.0f, 127 - int(sb));
    uint8_t *dst = static_cast<uint8_t *>(codes) + row * (d / 2) + lane * (CPL / 2);
#pragma unroll
    for (int j = 0; j < CPL; j += 2) dst[j / 2] = uint8_t(f32_to_e2m1(v[j] * inv) | (f32_to_e2m1(v[j + 1] * inv) << 4));
    if (lane % LB == 0) static_cast<uint8_t *>(scales)[row * (d / 32) + lane / LB] = uint8_t(sb);
  }
}

// RMSNorm (weights gw) then rotation of the channels >= d - r at position pos.
// Every lane of the wave must call this (it reduces across the wave).
template <int CPL>
__device__ __forceinline__ void norm_rope(float (&v)[CPL], const NormWeights<CPL> &gw, int d, int r,
                                          int64_t pos, double log2_base, float eps, int lane) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) ss += v[j] * v[j];
  ss = wave_sum(ss);
  float inv = rsqrtf(ss / float(d) + eps);
  const int c0 = lane * CPL;
#pragma unroll
  for (int j = 0; j < CPL; ++j) v[j] *= inv * (gw.has ? gw.w.at(j) : 1.0f);
  const int rope0 = d - r;
  if constexpr (CPL >= 2) {
    if (c0 + CPL > rope0) {
      const double rate = rope_rate(r, log2_base);
#pragma unroll
      for (int j = 0; j < CPL; j += 2) {
        int ch = c0 + j;
        if (ch >= rope0) {
          float cs, sn;
          rope_cos_sin(pos, (ch - rope0) >> 1, rate, &cs, &sn);
          float a = v[j], b = v[j + 1];
          v[j] = a * cs - b * sn;
          v[j + 1] = a * sn + b * cs;
        }
      }
    }
  } else {
    float partner = __shfl_xor(v[0], 1, 64);
    if (c0 >= rope0) {
      float cs, sn;
      rope_cos_sin(pos, (c0 - rope0) >> 1, rope_rate(r, log2_base), &cs, &sn);
      v[0] = (c0 & 1) ? (partner * sn + v[0] * cs) : (v[0] * cs - partner * sn);
    }
  }
}

// The rotation's per-lane pair frequencies (turns per position), formed before the position is
// known: lane l's pair p is channels l CPL + 2p, 2p + 1 (0 for the channels below d - r).
template <int CPL>
struct RopeFreq {
  double f[(CPL + 1) / 2];
};
template <int CPL>
__device__ __forceinline__ RopeFreq<CPL> rope_freqs(int d, int r, double log2_base, int lane, double *s_f) {
  // each lane forms one pair's frequency (a double-precision exp2: a long chain) into the wave's LDS
  // row s_f[d / 2], then every lane reads its own pairs'
  RopeFreq<CPL> q;
  const int rope0 = d - r, c0 = lane * CPL;
  const double rate = rope_rate(r > 0 ? r : 2, log2_base);
  for (int u = lane; u < r / 2; u += 64) s_f[u] = rope_turns_per_pos(u, rate);
  wave_lds_sync();
#pragma unroll
  for (int p = 0; p < CPL / 2; ++p) {
    const int ch = c0 + 2 * p;
    q.f[p] = ch >= rope0 ? s_f[(ch - rope0) >> 1] : 0.0;
  }
  return q;
}

// norm_rope with the frequencies formed beforehand and the wave's sum of squares by DPP: the
// arithmetic of norm_rope but for the order of that sum.
template <int CPL>
__device__ __forceinline__ void norm_rope_f(float (&v)[CPL], const NormWeights<CPL> &gw, int d, int r, int64_t pos,
                                            const RopeFreq<CPL> &q, float eps, int lane) {
  static_assert(CPL >= 2, "pairs within a lane");
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) ss += v[j] * v[j];
  ss = wave_sum_dpp(ss);
  const float inv = rsqrtf(ss / float(d) + eps);
#pragma unroll
  for (int j = 0; j < CPL; ++j) v[j] *= inv * (gw.has ? gw.w.at(j) : 1.0f);
  const int rope0 = d - r, c0 = lane * CPL;
  if (c0 + CPL > rope0) {
#pragma unroll
    for (int p = 0; p < CPL / 2; ++p) {
      if (c0 + 2 * p >= rope0) {
        float cs, sn;
        rope_cos_sin_f(pos, q.f[p], &cs, &sn);
        const float a = v[2 * p], b = v[2 * p + 1];
        v[2 * p] = a * cs - b * sn;
        v[2 * p + 1] = a * sn + b * cs;
      }
    }
  }
}

template <int CPL, int U, bool WIN, bool KEYS>
__global__ void __launch_bounds__(256) compress_kernel(CompressArgs a) {
  const int d = a.d, m = a.m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = blockIdx.x;                                // local entry index
  const int b = blockIdx.y;
  const int64_t gi = a.pos0 / m + i;                           // global entry index
  const bool has_prev = a.overlap && gi > 0;
  const int nt = has_prev ? 2 * m : m;
  const int64_t row_first = a.halo + (has_prev ? (i - 1) * m : i * m);
  const int slot_first = has_prev ? 0 : (a.overlap ? m : 0);
  const int own_first = has_prev ? m : 0;                      // token index where the own group starts
  const int64_t rows = a.halo + a.n_new;
  const uint16_t *cb = a.c + (int64_t(b) * rows) * d + lane * CPL;
  const uint16_t *zb = a.z + (int64_t(b) * rows) * d + lane * CPL;
  const NormWeights<CPL> gw = load_norm_weights<CPL>(a.norm_w, a.bias, lane);

  float mx[CPL], sm[CPL], acc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) { mx[j] = -INFINITY; sm[j] = 0.f; acc[j] = 0.f; }

  const int per = (nt + 3) >> 2;
  const int k0 = wave * per, k1 = min(nt, k0 + per);
  // Tokens go in groups of U (at most the wave's token count): the group's loads are all in
  // flight together, and the running maximum is updated once per group (one rescale for U
  // tokens).  Past the wave's last token the loads repeat that token (in bounds) and its logit
  // is -inf.
  for (int k = k0; k < k1; k += U) {
    RawRow<CPL> rc[U], rz[U], rb[U];                          // as loaded; unpacked at use
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(k + u, k1 - 1);
      const int64_t row = row_first + kk;
      load_raw<CPL>(cb + row * d, rc[u]);
      load_raw<CPL>(zb + row * d, rz[u]);
      load_raw<CPL>(a.bias + int64_t(slot_first + kk) * d + lane * CPL, rb[u]);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float l[U], gm = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        l[u] = k + u < k1 ? (rz[u].at(j) + rb[u].at(j)) * kLog2e : -INFINITY;
        gm = fmaxf(gm, l[u]);
      }
      const float nm = fmaxf(mx[j], gm);                      // finite: token k is real
      const float sc = exp2f(mx[j] - nm);                     // 0 on the first group
      float es = 0.f, ea = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float e = exp2f(l[u] - nm);
        es += e;
        ea += e * rc[u].at(j);
      }
      sm[j] = sm[j] * sc + es;
      acc[j] = acc[j] * sc + ea;
      mx[j] = nm;
    }
    if constexpr (WIN) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k + u;
        if (kk < k1 && kk >= own_first) {                      // per-token window row
          const int64_t tok = i * m + (kk - own_first);       // index among the new tokens
          float cv[CPL];
#pragma unroll
          for (int j = 0; j < CPL; ++j) cv[j] = rc[u].at(j);
          norm_rope<CPL>(cv, gw, d, a.rope_dim, a.pos0 + tok, a.log2_base, a.eps, lane);
          store_row<CPL>(a.win_rows + (int64_t(b) * a.n_new + tok) * d + lane * CPL, cv);
        }
      }
    }
  }

  __shared__ float s_state[3][4][64 * CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    s_state[0][wave][lane * CPL + j] = mx[j];
    s_state[1][wave][lane * CPL + j] = sm[j];
    s_state[2][wave][lane * CPL + j] = acc[j];
  }
  lds_barrier();
  if (wave != 0) return;
  float p[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int ch = lane * CPL + j;
    float M = fmaxf(fmaxf(s_state[0][0][ch], s_state[0][1][ch]), fmaxf(s_state[0][2][ch], s_state[0][3][ch]));
    float S = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float mw = s_state[0][w][ch];
      float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      S += s_state[1][w][ch] * f;
      A += s_state[2][w][ch] * f;
    }
    p[j] = A / S;
  }
  const int64_t row = int64_t(b) * (a.n_new / m) + i;
  if constexpr (KEYS) {
    // an indexer key: pooled only, rounded to bf16 as a stored key would be, then quantised
#pragma unroll
    for (int j = 0; j < CPL; ++j) p[j] = bf16_to_f32(f32_to_bf16(p[j]));
    if (a.entries) store_row<CPL>(a.entries + row * d + lane * CPL, p);
    encode_key_lanes<CPL>(p, a.key_format, d, a.k_codes, a.k_scales, row, lane);
  } else {
    norm_rope<CPL>(p, gw, d, a.rope_dim, gi * m, a.log2_base, a.eps, lane);
    store_row<CPL>(a.entries + row * d + lane * CPL, p);
  }
}

// ---- decode-time cache maintenance --------------------------------------------------------
// "DeepSeek-V4: Million-Token Context" (codexsims explainer), CSA walk-through: the compressed
// store gains one entry per m tokens; "Follow the white rabbit" (sambatista.com), sliding-window
// paragraph: the newest tokens are kept as separate rows, and a group becomes an entry once it is
// complete; indexer paragraph: the indexer keys are stored in low precision.
//
// One workgroup per sequence (and stream: the fused launch runs the KV stream's and the indexer
// stream's workgroups side by side).  The token's raw c, z rows go into the sequence's ring of the
// last (1+overlap) m tokens (slot = position mod ring size); its window row (RMSNorm, RoPE at its
// own position) into the window ring (slot = position mod W_cap).  When the token closes a group
// the entry is pooled from the ring, with the new token taken from registers -- the same tokens,
// bias rows and softmax as the batch compressor, accumulated in ring-slot order -- normalised,
// rotated at i m and written; the entry's indexer key is quantised into the key cache (the
// encoders of csa_quantize_keys) and n_entries is advanced.  A closing group's tokens fill the
// whole ring, so the waves load their ring slots, and both bias rows a slot can take, before the
// position arrives: the position only decides which rows take part and with which bias row.

// Quantise-on-write of one indexer key row (one wave; D_I % 32 == 0, <= 1024): lane l holds the
// value pairs l, l + 64, ... (all loaded before any store).  fp32 copy, fp8 e4m3 with a
// power-of-two row scale, or MXFP4 (a block of 32 values is the pairs of 16 lanes).
__device__ void store_key_row(const AppendArgs &a, const uint16_t *x, int64_t row, int lane) {
  const int np = a.D_I / 2;
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = lane + 64 * k;
    w[k] = q < np ? reinterpret_cast<const uint32_t *>(x)[q] : 0u;
  }
  if (a.key_format == 0) {
    float2 *dst = reinterpret_cast<float2 *>(static_cast<float *>(a.k_codes) + row * a.D_I);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (lane + 64 * k < np) dst[lane + 64 * k] = make_float2(bf16lo(w[k]), bf16hi(w[k]));
  } else if (a.key_format == 1) {
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(w[k])), fabsf(bf16hi(w[k]))));
    amax = wave_max(amax);
    const int e = e4m3_row_exp(amax);
    const float inv = ldexpf(1.0f, -e);
    uint16_t *dst = reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(a.k_codes) + row * a.D_I);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (lane + 64 * k < np)
        dst[lane + 64 * k] = uint16_t(f32_to_e4m3(bf16lo(w[k]) * inv) | (f32_to_e4m3(bf16hi(w[k]) * inv) << 8));
    if (lane == 0) static_cast<float *>(a.k_scales)[row] = ldexpf(1.0f, e);
  } else {
    uint8_t *dst = static_cast<uint8_t *>(a.k_codes) + row * np;
    uint8_t *sdst = static_cast<uint8_t *>(a.k_scales) + row * (a.D_I / 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (64 * k >= np) break;                                  // uniform
      float amax = fmaxf(fabsf(bf16lo(w[k])), fabsf(bf16hi(w[k])));
      amax = group_max_dpp<16>(amax);                           // the block's 16 lanes
      const uint32_t sb = mx_scale_byte(amax);
      const float inv = ldexpf(1.0f, 127 - int(sb));
      const int q = lane + 64 * k;
      if (q < np) {
        dst[q] = uint8_t(f32_to_e2m1(bf16lo(w[k]) * inv) | (f32_to_e2m1(bf16hi(w[k]) * inv) << 4));
        if ((q & 15) == 0) sdst[q >> 4] = uint8_t(sb);
      }
    }
  }
}

// Rings of at most kSmallRing rows (CSA: 2 m = 8) are pooled by waves 0 and 1 over half the slots
// each while waves 2 and 3 write the token's window row and ring rows; longer rings (HCA:
// m' = 128) by all four waves over their shares of the slots.  The partial softmax states meet in
// LDS and wave 0 merges them in wave order.
constexpr int kSmallRing = 8;

template <int CPL, bool KEYS>
__device__ __forceinline__ void append_sequence(const AppendArgs &a, int b) {
  const int d = a.d, m = a.m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = (1 + a.overlap) * m;                           // ring rows per sequence
  const int64_t ring0 = int64_t(b) * R;
  const int npw = R <= kSmallRing ? 2 : 4;                     // pooling waves
  const bool pools = wave < npw;
  // everything that does not need the position first: the token's rows, the norm weights, the
  // rotation's frequencies, and the ring slots with both of their candidate bias rows
  RawRow<CPL> rc, rz;
  load_raw<CPL>(a.c_new + int64_t(b) * d + lane * CPL, rc);
  load_raw<CPL>(a.z_new + int64_t(b) * d + lane * CPL, rz);
  const NormWeights<CPL> gw = load_norm_weights<CPL>(a.norm_w, a.bias, lane);
  constexpr int U = 4;                                         // slots held in registers at once
  const int per = (R + npw - 1) / npw;                         // ring slots per pooling wave
  const int s0 = pools ? wave * per : 0, s1 = pools ? min(R, s0 + per) : 0;
  // (xb, the other bias row, is read only with overlap: without it the zeros stay unused -- a copy
  // of xa here would make the loads wait for one another)
  RawRow<CPL> xc[U], xz[U], xa[U], xb[U] = {};
  auto load_slots = [&](int k) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sl = min(k + u, max(s1 - 1, 0));              // past the wave's slots: repeat (in bounds)
      load_raw<CPL>(a.tok_c + (ring0 + sl) * d + lane * CPL, xc[u]);
      load_raw<CPL>(a.tok_z + (ring0 + sl) * d + lane * CPL, xz[u]);
      load_raw<CPL>(a.bias + int64_t(sl) * d + lane * CPL, xa[u]);
      if (a.overlap) load_raw<CPL>(a.bias + int64_t((sl + m) % R) * d + lane * CPL, xb[u]);
    }
  };
  if (s0 < s1) load_slots(s0);
  __shared__ float s_state[3][4][64 * CPL];
  __shared__ double s_freq[2][32 * CPL];                       // waves 0 and 2: d / 2 pair frequencies
  RopeFreq<CPL> rq;                                            // (one channel per lane: formed at use)
  if constexpr (!KEYS && CPL >= 2) {
    if (wave == 0 || wave == 2) rq = rope_freqs<CPL>(d, a.rope_dim, a.log2_base, lane, s_freq[wave >> 1]);
  }
  const int64_t t = a.pos[b];
  if (t < 0) return;
  const int64_t i = (t + 1) / m - 1;                           // the entry this token closes, if any
  const bool closes = (t + 1) % m == 0 && i < a.N_cap;         // uniform over the workgroup

  // the token's own rows: the window row (RMSNorm, RoPE at t) and the raw rows into the ring
  auto token_jobs = [&]() __attribute__((always_inline)) {
    if (wave == 2) {
      if constexpr (!KEYS) {
        float v[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) v[j] = rc.at(j);
        if constexpr (CPL >= 2) norm_rope_f<CPL>(v, gw, d, a.rope_dim, t, rq, a.eps, lane);
        else norm_rope<CPL>(v, gw, d, a.rope_dim, t, a.log2_base, a.eps, lane);
        store_row<CPL>(a.win_ring + (int64_t(b) * a.W_cap + t % a.W_cap) * d + lane * CPL, v);
      }
    } else if (wave == 3) {
      store_raw<CPL>(a.tok_c + (ring0 + t % R) * d + lane * CPL, rc);
      store_raw<CPL>(a.tok_z + (ring0 + t % R) * d + lane * CPL, rz);
    }
  };
  if (!closes) {
    token_jobs();
    return;
  }

  // the entry's tokens: positions p_first .. p_first + nt - 1, token kk in ring slot
  // (p_first + kk) mod R with bias row slot_first + kk; a slot's token is (slot - ring_first) mod R
  const bool has_prev = a.overlap && i > 0;
  const int nt = has_prev ? 2 * m : m;
  const int64_t p_first = has_prev ? (i - 1) * m : i * m;
  const int slot_first = has_prev ? 0 : (a.overlap ? m : 0);
  const int ring_first = int(p_first % R);
  const int slot_t = int(t % R);                               // the new token: from registers
  float mx[CPL], sm[CPL], acc[CPL];                            // this wave's online softmax
#pragma unroll
  for (int j = 0; j < CPL; ++j) { mx[j] = -INFINITY; sm[j] = 0.f; acc[j] = 0.f; }
  if (pools) {
    for (int k = s0; k < s1; k += U) {
      if (k != s0) load_slots(k);
      bool use_b[U], valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sl = k + u;
        const int kk = (sl - ring_first + R) % R;
        valid[u] = sl < s1 && kk < nt;
        use_b[u] = a.overlap && valid[u] && slot_first + kk != sl;   // then it is (sl + m) mod R
        if (sl == slot_t) { xc[u] = rc; xz[u] = rz; }
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float l[U], gm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float bj = use_b[u] ? xb[u].at(j) : xa[u].at(j);
          l[u] = valid[u] ? (xz[u].at(j) + bj) * kLog2e : -INFINITY;
          gm = fmaxf(gm, l[u]);
        }
        const float nm = fmaxf(mx[j], gm);
        const float sc = nm == -INFINITY ? 0.f : exp2f(mx[j] - nm);
        float es = 0.f, ea = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float e = nm == -INFINITY ? 0.f : exp2f(l[u] - nm);
          es += e;
          ea += e * xc[u].at(j);
        }
        sm[j] = sm[j] * sc + es;
        acc[j] = acc[j] * sc + ea;
        mx[j] = nm;
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        s_state[0][wave][lane * CPL + j] = mx[j];
        s_state[1][wave][lane * CPL + j] = sm[j];
        s_state[2][wave][lane * CPL + j] = acc[j];
      }
    }
  } else {
    token_jobs();                                              // meanwhile
  }
  lds_barrier();
  if (wave == 0) {
    // merge the pooling waves' states in wave order (wave 0's own from registers)
    float pv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int ch = lane * CPL + j;
      float M = mx[j];
      for (int w = 1; w < npw; ++w) M = fmaxf(M, s_state[0][w][ch]);
      float S = 0.f, A = 0.f;
      for (int w = 0; w < npw; ++w) {
        const float mw = w == 0 ? mx[j] : s_state[0][w][ch];
        const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        S += (w == 0 ? sm[j] : s_state[1][w][ch]) * f;
        A += (w == 0 ? acc[j] : s_state[2][w][ch]) * f;
      }
      pv[j] = A / S;
    }
    const int64_t row = int64_t(b) * a.N_cap + i;
    if constexpr (KEYS) {
      // the indexer stream: the pooled key, rounded to bf16 and quantised into the key cache
#pragma unroll
      for (int j = 0; j < CPL; ++j) pv[j] = bf16_to_f32(f32_to_bf16(pv[j]));
      if (a.entries) store_row<CPL>(a.entries + row * d + lane * CPL, pv);
      encode_key_lanes<CPL>(pv, a.key_format, d, a.k_codes, a.k_scales, row, lane);
    } else {
      if constexpr (CPL >= 2) norm_rope_f<CPL>(pv, gw, d, a.rope_dim, i * m, rq, a.eps, lane);
      else norm_rope<CPL>(pv, gw, d, a.rope_dim, i * m, a.log2_base, a.eps, lane);
      store_row<CPL>(a.entries + row * d + lane * CPL, pv);
      if (lane == 0) a.n_entries[b] = i + 1;
    }
  } else if (wave == 1) {
    if (!KEYS && a.k_new) store_key_row(a, a.k_new + int64_t(b) * a.D_I, int64_t(b) * a.N_cap + i, lane);
  } else if (pools) {
    token_jobs();                                              // long rings: after the pooling
  }
}

template <int CPL, bool KEYS>
__global__ void __launch_bounds__(256) decode_append_kernel(AppendArgs a) {
  append_sequence<CPL, KEYS>(a, blockIdx.x);
}

// Both streams of one decode step in one launch: workgroups (b, 0) maintain the KV stream, (b, 1)
// the indexer stream.
template <int CPL, int CPLI>
__global__ void __launch_bounds__(256) decode_append_step_kernel(AppendArgs a, AppendArgs ai) {
  if (blockIdx.y == 0) append_sequence<CPL, false>(a, blockIdx.x);
  else append_sequence<CPLI, true>(ai, blockIdx.x);
}

template <int CPL, bool WIN>
hipError_t launch_compress_win(const CompressArgs &a, dim3 grid, hipStream_t stream) {
  // Tokens per wave: 2m with the previous group (every entry but the sequence's first), else m.
  const int per = ((a.overlap ? 2 * a.m : a.m) + 3) / 4;
  const dim3 block(256);
  if (per >= 8) return launch("compress", compress_kernel<CPL, 8, WIN, false>, grid, block, stream, a);
  if (per >= 4) return launch("compress", compress_kernel<CPL, 4, WIN, false>, grid, block, stream, a);
  if (per >= 2) return launch("compress", compress_kernel<CPL, 2, WIN, false>, grid, block, stream, a);
  return launch("compress", compress_kernel<CPL, 1, WIN, false>, grid, block, stream, a);
}

template <int CPL>
hipError_t launch_compress_keys_cpl(const CompressArgs &a, dim3 grid, hipStream_t stream) {
  const int per = ((a.overlap ? 2 * a.m : a.m) + 3) / 4;
  const dim3 block(256);
  if (per >= 8) return launch("compress_keys", compress_kernel<CPL, 8, false, true>, grid, block, stream, a);
  if (per >= 4) return launch("compress_keys", compress_kernel<CPL, 4, false, true>, grid, block, stream, a);
  if (per >= 2) return launch("compress_keys", compress_kernel<CPL, 2, false, true>, grid, block, stream, a);
  return launch("compress_keys", compress_kernel<CPL, 1, false, true>, grid, block, stream, a);
}

// The per-token window rows (normalised and rotated token rows) are a separate instantiation:
// their code holds many registers even when not taken, which would cost the pooling occupancy.
template <int CPL>
hipError_t launch_compress_cpl(const CompressArgs &a, dim3 grid, hipStream_t stream) {
  return a.win_rows ? launch_compress_win<CPL, true>(a, grid, stream)
                    : launch_compress_win<CPL, false>(a, grid, stream);
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t stream) {
  const dim3 grid(unsigned(a.B)), block(256);
  switch (a.d / 64) {
    case 1: return launch("decode_append", decode_append_kernel<1, false>, grid, block, stream, a);
    case 2: return launch("decode_append", decode_append_kernel<2, false>, grid, block, stream, a);
    case 4: return launch("decode_append", decode_append_kernel<4, false>, grid, block, stream, a);
    case 8: return launch("decode_append", decode_append_kernel<8, false>, grid, block, stream, a);
    case 16: return launch("decode_append", decode_append_kernel<16, false>, grid, block, stream, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append_keys(const AppendArgs &a, hipStream_t stream) {
  const dim3 grid(unsigned(a.B)), block(256);
  switch (a.d / 64) {
    case 2: return launch("decode_append_keys", decode_append_kernel<2, true>, grid, block, stream, a);
    case 4: return launch("decode_append_keys", decode_append_kernel<4, true>, grid, block, stream, a);
    case 8: return launch("decode_append_keys", decode_append_kernel<8, true>, grid, block, stream, a);
    case 16: return launch("decode_append_keys", decode_append_kernel<16, true>, grid, block, stream, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append_step(const AppendArgs &a, const AppendArgs &ai, hipStream_t stream) {
  const dim3 grid(unsigned(a.B), 2), block(256);
#define CSA_STEP_CASES(C)                                                                                      \
  switch (ai.d / 64) {                                                                                        \
    case 2: return launch("decode_append_step", decode_append_step_kernel<C, 2>, grid, block, stream, a, ai);  \
    case 4: return launch("decode_append_step", decode_append_step_kernel<C, 4>, grid, block, stream, a, ai);  \
    case 8: return launch("decode_append_step", decode_append_step_kernel<C, 8>, grid, block, stream, a, ai);  \
    case 16: return launch("decode_append_step", decode_append_step_kernel<C, 16>, grid, block, stream, a, ai); \
    default: return hipErrorInvalidValue;                                                                     \
  }
  switch (a.d / 64) {
    case 2: CSA_STEP_CASES(2)
    case 4: CSA_STEP_CASES(4)
    case 8: CSA_STEP_CASES(8)
    case 16: CSA_STEP_CASES(16)
    default: return hipErrorInvalidValue;
  }
#undef CSA_STEP_CASES
}

hipError_t launch_compress_keys(const CompressArgs &a, hipStream_t stream) {
  const dim3 grid(unsigned(a.n_new / a.m), unsigned(a.B));
  switch (a.d / 64) {
    case 2: return launch_compress_keys_cpl<2>(a, grid, stream);
    case 4: return launch_compress_keys_cpl<4>(a, grid, stream);
    case 8: return launch_compress_keys_cpl<8>(a, grid, stream);
    case 16: return launch_compress_keys_cpl<16>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_compress(const CompressArgs &a, hipStream_t stream) {
  const dim3 grid(unsigned(a.n_new / a.m), unsigned(a.B));
  switch (a.d / 64) {
    case 1: return launch_compress_cpl<1>(a, grid, stream);
    case 2: return launch_compress_cpl<2>(a, grid, stream);
    case 4: return launch_compress_cpl<4>(a, grid, stream);
    case 8: return launch_compress_cpl<8>(a, grid, stream);
    case 16: return launch_compress_cpl<16>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa
