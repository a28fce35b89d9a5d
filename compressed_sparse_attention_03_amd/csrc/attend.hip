// Core attention of CSA and HCA: shared-KV multi-query attention over a row list
// (selected compressed entries, or every visible entry for HCA) followed by the sliding-window
// rows, in one joint softmax.
//
// "DeepSeek-V4: Million-Token Context" (codexsims explainer), CSA walk-through: each query head
// attends to the picked set plus a sliding window of the most recent tokens; HCA walk-through:
// dense multi-query attention over every compressed entry plus the window.  paperlayer summary,
// section 2.3: shared-KV multi-query attention; RMSNorm on the query heads before core attention.
// dev.to "Two Compression Strategies": partial RoPE.
//
// Work split (split-K decode): workgroup = (query, block of 16 heads, slice of the row list),
// 4 waves.  A wave takes 16 rows at a time:
//   S^T[16 rows x 16 heads] = K[16 x D] * Q^T      v_mfma_f32_16x16x32_bf16, rows as A operand
//                                                   (one 16-byte load per lane per 32 channels)
//   V^T fragments                                  v_mfma_f32_16x16x16_bf16 against an identity
//                                                   fragment (exact: bf16 * 1 in fp32)
//   O[16 heads x D] += P * V                       v_mfma_f32_16x16x16_bf16, P straight from the
//                                                   S^T accumulator layout
// with an online softmax in the exp2 domain (the softmax scale and log2(e) are folded into q).
// The four waves' (max, sum, O) states merge through LDS; the slice writes a normalised fp32
// partial and its log2-sum-exp, and a combine kernel merges the slices in a fixed order.
#include "common.h"
#include "internal.h"

namespace csa {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

union Frag8 {      // 8 bf16 = 16 bytes
  uint4 u;
  v8bf b;
  v4s h[2];
};

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
union Pack4 {
  v4bf b;
  v4s s;
};

// Round four floats to bf16 (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ v4s pack4(float a, float b, float c, float d) {
  Pack4 p;
  p.b[0] = __bf16(a); p.b[1] = __bf16(b); p.b[2] = __bf16(c); p.b[3] = __bf16(d);
  return p.s;
}

constexpr int kMaxRowsPerSplit = 2048;
constexpr float kRescaleSlack = 8.0f;     // log2 units: the running max may lag the true max by 2^8

// Row code of slot `ri` of the query's row list: an entry index (< N_cap), N_cap + window row, or
// -1 when the slot is empty.
__device__ __forceinline__ int row_code(const AttendArgs &a, int64_t qi, int b, int64_t t, int64_t n_vis,
                                        int64_t ri) {
  if (ri < a.n_sel) {
    int64_t e;
    if (a.topk_idx) {
      e = a.topk_idx[qi * a.n_sel + ri];
      if (e < 0 || e >= a.N_cap) return -1;
    } else {
      e = ri;
      if (e >= n_vis) return -1;
    }
    return int(e);
  }
  const int64_t w = ri - a.n_sel;
  if (w >= a.window) return -1;
  const int64_t p = t - a.window + 1 + w;                  // window position
  if (p < 0) return -1;
  const int64_t wr = p - a.win_pos0[b];
  if (wr < 0 || wr >= a.W_cap) return -1;
  return int(a.N_cap + wr);
}

// Workgroup -> (query, split, head block).  Workgroups are dispatched to the 8 XCDs round-robin by
// linear id, so the head blocks of one (query, split) -- which read the same rows -- are given ids
// that are equal modulo 8 and share that XCD's L2.
struct AttendTile {
  int64_t qi;
  int split, hb;
  bool valid;
};
__device__ __forceinline__ AttendTile attend_tile(const AttendArgs &a, int64_t n_queries) {
  const int64_t L = blockIdx.x;
  const int64_t x = L & 7, rest = L >> 3;
  const int hb = int(rest % a.plan.n_hb);
  const int64_t pair = (rest / a.plan.n_hb) * 8 + x;
  AttendTile t;
  t.valid = pair < n_queries * a.plan.n_splits;
  t.qi = pair / a.plan.n_splits;
  t.split = int(pair % a.plan.n_splits);
  t.hb = hb;
  return t;
}

// Sum / maximum over lanes l, l^16, l^32 and l^48 (the four row groups of one head), in every lane,
// with the gfx950 half-wave and row swaps.
__device__ __forceinline__ float group4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr int kWaves = 4;                  // waves per workgroup; each takes whole 16-row chunks
template <int D>
constexpr int ring_of() { return D == 512 ? 2 : 4; }   // chunks in flight per wave (registers)

typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int D>
__global__ void __launch_bounds__(64 * kWaves) attend_split_kernel(AttendArgs a, int64_t n_queries) {
  constexpr int NT = 64 * kWaves;
  constexpr int NS = D / 32;          // 32-channel steps of a row (QK^T)
  constexpr int NB = D / 16;          // 16-channel blocks of O (PV)
  constexpr int QCH = D / 32;         // prologue: threads per head (32 channels each)
  constexpr int RING = ring_of<D>();
  constexpr int RS = 2 * D + 16;      // staging row stride in bytes: 16 B of padding per row, so
                                      // the rows one wide LDS access touches fall in different banks
  constexpr int QS = D + 8;           // q^ row stride (bf16), padded likewise
  constexpr int HD = D / 2;           // the merge runs over two halves of the channels
  constexpr int OS = HD + 4;          // merge row stride (fp32)
  // LDS: per-wave staging of the current chunk (for the transposing V reads), q^, row codes.
  // After the row loop the staging area holds the four waves' scaled O, half the channels at a time.
  __shared__ __align__(16) unsigned char s_stage[kWaves * 16 * RS];
  __shared__ __align__(16) uint16_t s_q[16 * QS];
  __shared__ int s_row[kMaxRowsPerSplit];
  __shared__ float s_cs[256], s_sn[256];
  __shared__ float s_m[kWaves][16], s_l[kWaves][16];
  static_assert(kWaves * 16 * OS * 4 <= kWaves * 16 * RS, "merge buffers must fit in the staging area");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const AttendTile tl = attend_tile(a, n_queries);
  if (!tl.valid) return;
  const int split = tl.split, hb = tl.hb;
  const int64_t qi = tl.qi;
  const int b = int(qi / a.Sq), s_idx = int(qi % a.Sq);
  const int64_t t = a.q_pos0[b] + s_idx;
  const int64_t n_vis = a.topk_idx ? 0 : min(a.n_entries[b], (t + 1) / a.m);
  const int64_t r0 = int64_t(split) * a.plan.rows_per_split;
  const int64_t r1 = min(int64_t(a.plan.n_rows), r0 + a.plan.rows_per_split);
  const int nr = int(r1 - r0);
  const int n_chunks = (nr + 15) >> 4;
  const int my_chunks = n_chunks > wave ? (n_chunks - wave + kWaves - 1) / kWaves : 0;   // chunks wave, wave+4, ...

  // ---- prologue.  The raw q chunk (and norm weights) of this thread are loaded first: loads
  // complete in issue order, so anything issued later (the row prefetch) does not delay them.
  const bool qthread = tid < 16 * QCH;
  const int qh = tid / QCH, qc = tid % QCH;
  const int qhead = hb * 16 + qh;
  uint4 qraw[4], wraw[4];
  {
    const int qt = qthread ? tid : 0;
    const int h0 = hb * 16 + qt / QCH, c0 = qt % QCH;
    const uint4 *src = reinterpret_cast<const uint4 *>(a.q + (qi * a.H + (h0 < a.H ? h0 : 0)) * D + 32 * c0);
    const uint4 *wsrc = reinterpret_cast<const uint4 *>(a.q_norm_w ? a.q_norm_w + 32 * c0 : a.q + 32 * c0);
#pragma unroll
    for (int k = 0; k < 4; ++k) { qraw[k] = src[k]; wraw[k] = wsrc[k]; }
  }
  // row codes and rotary angles; the first chunks' loads go out before q^ is built
  for (int i = tid; i < nr; i += NT) s_row[i] = row_code(a, qi, b, t, n_vis, r0 + i);
  const int npairs = a.rope_dim / 2;
  for (int u = tid; u < npairs; u += NT) rope_cos_sin(t, u, a.rope_dim, a.log2_base, &s_cs[u], &s_sn[u]);
  const uint16_t *ent_b = a.entries + int64_t(b) * a.N_cap * D;
  const uint16_t *win_b = a.win_rows + int64_t(b) * a.W_cap * D;
  __syncthreads();

  // ring of row fragments: lane (r, g) holds row r of the chunk, channels 32s + 8g .. +7 for every s
  Frag8 ring[RING][NS];
  int codes[RING];
  // Loads are unconditional (an empty slot reads entry row 0, which exists and is finite; its
  // softmax weight is exactly 0): branch-free code lets the compiler wait only for the chunk in use
  // instead of every outstanding load.
  auto issue = [&](int j, int slot) {            // this wave's j-th chunk
    const int i = (wave + kWaves * j) * 16 + r;
    const int code = (j < my_chunks && i < nr) ? s_row[i] : -1;
    codes[slot] = code;
    const uint16_t *rp = code < 0 ? ent_b
                                  : (code < a.N_cap ? ent_b + int64_t(code) * D : win_b + (int64_t(code) - a.N_cap) * D);
#pragma unroll
    for (int s = 0; s < NS; ++s) ring[slot][s].u = *reinterpret_cast<const uint4 *>(rp + 32 * s + 8 * g);
  };
#pragma unroll
  for (int j = 0; j < RING; ++j) issue(j, j);

  // q^ = RoPE(RMSNorm(q)) * scale * log2(e) for the 16 heads, into LDS
  if (qthread) {
    const int h = qh, c = qc;
    float v[32];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 w = qraw[k];
      v[8 * k + 0] = bf16lo(w.x); v[8 * k + 1] = bf16hi(w.x); v[8 * k + 2] = bf16lo(w.y);
      v[8 * k + 3] = bf16hi(w.y); v[8 * k + 4] = bf16lo(w.z); v[8 * k + 5] = bf16hi(w.z);
      v[8 * k + 6] = bf16lo(w.w); v[8 * k + 7] = bf16hi(w.w);
    }
    if (qhead >= a.H) {
#pragma unroll
      for (int k = 0; k < 32; ++k) v[k] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) ss += v[k] * v[k];
#pragma unroll
    for (int o = 1; o < QCH; o <<= 1) ss += __shfl_xor(ss, o, 64);   // the head's QCH threads
    const float inv = rsqrtf(ss / float(D) + a.eps) * a.scale_log2;
    float gw[32];
    const bool has_w = a.q_norm_w != nullptr;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 w = wraw[k];
      gw[8 * k + 0] = bf16lo(w.x); gw[8 * k + 1] = bf16hi(w.x); gw[8 * k + 2] = bf16lo(w.y);
      gw[8 * k + 3] = bf16hi(w.y); gw[8 * k + 4] = bf16lo(w.z); gw[8 * k + 5] = bf16hi(w.z);
      gw[8 * k + 6] = bf16lo(w.w); gw[8 * k + 7] = bf16hi(w.w);
    }
    if (!has_w) {
#pragma unroll
      for (int k = 0; k < 32; ++k) gw[k] = 1.0f;
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) v[k] *= inv * gw[k];
    const int rope0 = D - a.rope_dim;
    if (32 * c + 32 > rope0) {
#pragma unroll
      for (int k = 0; k < 32; k += 2) {
        const int ch = 32 * c + k;
        if (ch >= rope0) {
          const int u = (ch - rope0) >> 1;
          const float cs = s_cs[u], sn = s_sn[u], x0 = v[k], x1 = v[k + 1];
          v[k] = x0 * cs - x1 * sn;
          v[k + 1] = x0 * sn + x1 * cs;
        }
      }
    }
    uint4 *dst = reinterpret_cast<uint4 *>(s_q + h * QS + 32 * c);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      Pack4 lo, hi;
      lo.s = pack4(v[8 * k], v[8 * k + 1], v[8 * k + 2], v[8 * k + 3]);
      hi.s = pack4(v[8 * k + 4], v[8 * k + 5], v[8 * k + 6], v[8 * k + 7]);
      dst[k] = make_uint4(uint32_t(uint16_t(lo.s[0])) | (uint32_t(uint16_t(lo.s[1])) << 16),
                          uint32_t(uint16_t(lo.s[2])) | (uint32_t(uint16_t(lo.s[3])) << 16),
                          uint32_t(uint16_t(hi.s[0])) | (uint32_t(uint16_t(hi.s[1])) << 16),
                          uint32_t(uint16_t(hi.s[2])) | (uint32_t(uint16_t(hi.s[3])) << 16));
    }
  }
  __syncthreads();

  // O^T block nb (O^T = V^T P^T): lane (r, g) element v = head r, channel 16 nb + 4g + v, so a
  // lane owns one head: the rescale is lane-local and the merge writes 16 B per block
  v4f o[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) o[k] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;           // of head r (same in the four lanes of head r)
  unsigned char *stage = s_stage + wave * 16 * RS;

  // One chunk of 16 rows: S^T = K q^T over all D channels (K from registers, q^ from LDS), online
  // softmax, then the rows go to the wave's staging area once and O += P V takes V^T fragments
  // from it with the transposing LDS read.  `slot` is a compile-time ring position.
  auto chunk = [&](int slot) {
    const uint64_t vmask = __ballot(codes[slot] >= 0);
    // four independent accumulation chains over the channel steps, summed at the end
    constexpr int NCH = NS < 4 ? NS : 4;
    v4f sp[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) sp[c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      Frag8 qf;
      qf.u = *reinterpret_cast<const uint4 *>(s_q + r * QS + 32 * s + 8 * g);
      sp[s % NCH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[slot][s].b, qf.b, sp[s % NCH], 0, 0, 0);
    }
    v4f st = sp[0];
#pragma unroll
    for (int c = 1; c < NCH; ++c) { st[0] += sp[c][0]; st[1] += sp[c][1]; st[2] += sp[c][2]; st[3] += sp[c][3]; }
#pragma unroll
    for (int s = 0; s < NS; ++s)
      *reinterpret_cast<uint4 *>(stage + r * RS + (32 * s + 8 * g) * 2) = ring[slot][s].u;
    // st[v] = logit of row 4g+v for head r
    float sv[4], cmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = ((vmask >> (4 * g + v)) & 1) ? st[v] : -INFINITY;
      cmax = fmaxf(cmax, sv[v]);
    }
    cmax = group4_max(cmax);
    // lazy running max: rescale only when some head's max grew past the slack
    const bool grow = cmax > m_run + kRescaleSlack || (m_run == -INFINITY && cmax != -INFINITY);
    if (__any(grow)) {
      const bool empty = __all(m_run == -INFINITY);        // nothing accumulated yet: O is zero
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      if (!empty) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
#pragma unroll
          for (int v = 0; v < 4; ++v) o[k][v] *= alpha;
        }
      }
    }
    float p[4], psum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = (sv[v] == -INFINITY) ? 0.f : exp2f(sv[v] - m_run);
      psum += p[v];
    }
    l_run += group4_sum(psum);
    const v4s pf = pack4(p[0], p[1], p[2], p[3]);
    // V^T fragment of block nb: lane (n, g) reads row 4g + n/4, channels 16 nb + 4(n%4) .. +3;
    // the transposing read hands lane (n, g) rows 4g .. 4g+3 of channel 16 nb + n -- the A
    // operand (channel n, rows 4g..) of O^T += V^T P^T, with P^T as B (lane (r, g): head r, rows 4g..)
    const unsigned char *vbase = stage + (4 * g + (r >> 2)) * RS + 8 * (r & 3);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const v4s vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vbase + 32 * nb));
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pf, o[nb], 0, 0, 0);
    }
  };
  for (int j0 = 0; j0 < my_chunks; j0 += RING) {
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      if (j0 + k < my_chunks) {
        chunk(k);
        issue(j0 + k + RING, k);     // refill the slot
      }
    }
  }

  // ---- merge the four waves' (m, l, O) states, half of the channels at a time -----------------
  if (g == 0) { s_m[wave][r] = m_run; s_l[wave][r] = l_run; }
  __syncthreads();                                   // every wave is done with its staging area
  // head r's merged maximum, sum and this wave's share (every lane of head r computes the same)
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][r]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) L += s_m[w][r] == -INFINITY ? 0.f : s_l[w][r] * exp2f(s_m[w][r] - M);
  const float share = (s_m[wave][r] == -INFINITY || !(L > 0.f)) ? 0.f : exp2f(s_m[wave][r] - M) / L;
  const bool direct = a.plan.n_splits == 1;
  float *po = static_cast<float *>(a.workspace);
  float *plse = po + n_queries * a.H * a.plan.n_splits * D;
  float *mb = reinterpret_cast<float *>(s_stage);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // each wave writes its O^T blocks of this half, scaled by its share, as [head][channel]
    float *mine = mb + wave * 16 * OS;
#pragma unroll
    for (int k = 0; k < NB / 2; ++k) {
      const v4f x = o[half * (NB / 2) + k];
      *reinterpret_cast<float4 *>(mine + r * OS + 16 * k + 4 * g) =
          make_float4(x[0] * share, x[1] * share, x[2] * share, x[3] * share);
    }
    __syncthreads();
    // every thread sums four consecutive channels of one head over the waves and writes them
    constexpr int Q4 = HD / 4;
    for (int e = tid; e < 16 * Q4; e += NT) {
      const int h = e / Q4, c4 = (e - h * Q4) * 4;
      const int gh = hb * 16 + h;
      if (gh >= a.H) continue;
      float4 acc = *reinterpret_cast<const float4 *>(mb + h * OS + c4);
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const float4 x = *reinterpret_cast<const float4 *>(mb + (w * 16 + h) * OS + c4);
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
      }
      const int ch = half * HD + c4;
      if (direct)
        *reinterpret_cast<v4s *>(a.out + (qi * a.H + gh) * D + ch) = pack4(acc.x, acc.y, acc.z, acc.w);
      else
        *reinterpret_cast<float4 *>(po + ((qi * a.H + gh) * a.plan.n_splits + split) * int64_t(D) + ch) = acc;
    }
    if (half == 0) __syncthreads();
  }
  if (wave == 0 && g == 0) {
    const int gh = hb * 16 + r;
    if (gh < a.H) {
      const float lse2 = L > 0.f ? M + log2f(L) : -INFINITY;
      if (direct) {
        if (a.lse) a.lse[qi * a.H + gh] = lse2 * 0.6931471805599453f;
      } else {
        plse[(qi * a.H + gh) * a.plan.n_splits + split] = lse2;
      }
    }
  }
}

// One workgroup per (query, head): merge the slices in order.
template <int D>
__global__ void __launch_bounds__(D / 4) attend_combine_kernel(AttendArgs a, int64_t n_queries) {
  constexpr int kBatch = 8;                       // slices whose loads are in flight together
  const int64_t qh = blockIdx.x;                  // query * H + head
  const int ns = a.plan.n_splits;
  const float *po = static_cast<const float *>(a.workspace) + qh * ns * int64_t(D);
  const float *plse = static_cast<const float *>(a.workspace) + n_queries * a.H * ns * int64_t(D) + qh * ns;
  const int ch = threadIdx.x * 4;
  // every slice's log2-sum-exp and partial are loaded before any is used (one round trip per
  // batch of slices), then merged in slice order with a running maximum
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < ns; s0 += kBatch) {
    float ls[kBatch];
    float4 x[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = s0 + j < ns ? s0 + j : ns - 1;
      ls[j] = plse[s];
      x[j] = *reinterpret_cast<const float4 *>(po + s * int64_t(D) + ch);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j >= ns || ls[j] == -INFINITY) continue;
      const float Mn = fmaxf(M, ls[j]);
      const float c = M == -INFINITY ? 0.f : exp2f(M - Mn), w = exp2f(ls[j] - Mn);
      L = L * c + w;
      acc.x = acc.x * c + w * x[j].x; acc.y = acc.y * c + w * x[j].y;
      acc.z = acc.z * c + w * x[j].z; acc.w = acc.w * c + w * x[j].w;
      M = Mn;
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  uint16_t *dst = a.out + qh * D + ch;
  *reinterpret_cast<v4s *>(dst) = pack4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse && threadIdx.x == 0) a.lse[qh] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

}  // namespace

AttendPlan plan_attend(int64_t n_queries, int H, int64_t n_sel, int window, int D) {
  AttendPlan p;
  p.n_hb = (H + 15) / 16;
  p.n_rows = int(n_sel + window);
  // A split is a multiple of 64 rows (four waves x 16-row chunks).  Aim at two chunks per wave,
  // but no more splits than keep the grid within one round of resident workgroups (one per CU at
  // D = 512, two below); every split costs a partial [16 x D] fp32 write and read.
  const int64_t units = n_queries * p.n_hb;
  const int64_t resident = D == 512 ? 256 : 512;
  int64_t splits = (p.n_rows + 127) / 128;
  const int64_t by_grid = resident / units;
  if (splits > by_grid) splits = by_grid;
  if (splits < 1) splits = 1;
  int64_t rps = (p.n_rows + splits - 1) / splits;
  rps = (rps + 63) / 64 * 64;
  if (rps > kMaxRowsPerSplit) rps = kMaxRowsPerSplit;
  p.rows_per_split = int(rps);
  p.n_splits = int((p.n_rows + rps - 1) / rps);
  return p;
}

size_t attend_workspace_bytes(int64_t n_queries, int H, int D, int64_t n_sel, int window) {
  AttendPlan p = plan_attend(n_queries, H, n_sel, window, D);
  if (p.n_splits == 1) return 256;
  return size_t(n_queries * H * p.n_splits * (int64_t(D) + 1) * 4 + 256);
}

hipError_t launch_attend(const AttendArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  const int64_t nq = int64_t(a.B) * a.Sq;
  const int64_t pairs = nq * a.plan.n_splits;
  dim3 grid(unsigned(((pairs + 7) / 8) * 8 * a.plan.n_hb));
  switch (a.D) {
    case 64: e = launch("attend_split", attend_split_kernel<64>, grid, dim3(64 * kWaves), stream, a, nq); break;
    case 128: e = launch("attend_split", attend_split_kernel<128>, grid, dim3(64 * kWaves), stream, a, nq); break;
    case 256: e = launch("attend_split", attend_split_kernel<256>, grid, dim3(64 * kWaves), stream, a, nq); break;
    case 512: e = launch("attend_split", attend_split_kernel<512>, grid, dim3(64 * kWaves), stream, a, nq); break;
    default: return hipErrorInvalidValue;
  }
  return e;
}

hipError_t launch_combine(const AttendArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.plan.n_splits == 1) return hipSuccess;
  const int64_t nq = int64_t(a.B) * a.Sq;
  dim3 grid(unsigned(nq * a.H));
  switch (a.D) {
    case 64: e = launch("attend_combine", attend_combine_kernel<64>, grid, dim3(16), stream, a, nq); break;
    case 128: e = launch("attend_combine", attend_combine_kernel<128>, grid, dim3(32), stream, a, nq); break;
    case 256: e = launch("attend_combine", attend_combine_kernel<256>, grid, dim3(64), stream, a, nq); break;
    case 512: e = launch("attend_combine", attend_combine_kernel<512>, grid, dim3(128), stream, a, nq); break;
    default: return hipErrorInvalidValue;
  }
  return e;
}

}  // namespace csa
