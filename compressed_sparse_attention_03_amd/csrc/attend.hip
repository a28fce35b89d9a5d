// Core attention of CSA and HCA: shared-KV multi-query attention over a row list
// (selected compressed entries, or every visible entry for HCA) followed by the sliding-window
// rows, in one joint softmax.
//
// "DeepSeek-V4: Million-Token Context" (codexsims explainer), CSA walk-through: every query head's
// attention covers the selected entries together with a window of the newest tokens; HCA walk-through:
// dense multi-query attention over every compressed entry plus the window.  paperlayer summary,
// section 2.3: shared-KV multi-query attention; RMSNorm on the query heads before core attention.
// dev.to "Two Compression Strategies": partial RoPE.
//
// Work split (split-K decode): workgroup = (query, block of 16 heads, slice of the row list).  Its
// NW = D / 128 waves split the channels (wave w owns 128 of them in q, in every row and in O) and
// take the slice's 16-row chunks together:
//   S^T partial [16 rows x 16 heads] = K_w Q_w^T    v_mfma_f32_16x16x32_bf16, the rows' channel
//                                                   slice as A operand (16-byte loads per lane)
//   S^T = sum over the waves                        through LDS, one barrier per pair of chunks
//   online softmax in the exp2 domain               every wave alike (the softmax scale and
//                                                   log2(e) are folded into q)
//   O_w^T [128 ch x 16 heads] += V_w^T P^T          v_mfma_f32_16x16x16_bf16, V^T fragments from a
//                                                   transposing LDS read of the staged rows
// Each wave writes its channels of the slice's normalised partial (O / l rounded to bf16); wave 0
// writes the slice's log2-sum-exp, and a combine kernel merges the slices in a fixed order.
#include <mutex>

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

// Element e (0..7) of eight packed bf16.
__device__ __forceinline__ float elem8(const uint4 &w, int e) {
  const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
  return (e & 1) ? bf16hi(x) : bf16lo(x);
}

constexpr int kMaxRowsPerSplit = 2048;

// Row code of slot `ri` of the query's row list: an entry index (< N_cap), N_cap + window row, or
// -1 when the slot is empty.  Slots below n_sel: selected entry e (SEL; e read from topk_idx) or
// entry ri (HCA, visible when below n_vis); then the window.
__device__ __forceinline__ int selected_code(const AttendArgs &a, int e) { return (e < 0 || e >= a.N_cap) ? -1 : e; }
// wp0: win_pos0[b] when the window rows are stored from a position on (read once, with the query's
// position), unused for a ring.
__device__ __forceinline__ int window_code(const AttendArgs &a, int64_t wp0, int64_t t, int64_t ri) {
  const int64_t w = ri - a.n_sel;
  if (w >= a.window) return -1;
  const int64_t p = t - a.window + 1 + w;                  // window position
  if (p < 0) return -1;
  if (a.win_pos0 == nullptr) return int(a.N_cap + p % a.W_cap);   // ring: row of p at p mod W_cap
  const int64_t wr = p - wp0;
  if (wr < 0 || wr >= a.W_cap) return -1;
  return int(a.N_cap + wr);
}
template <bool SEL>
__device__ __forceinline__ int row_code(const AttendArgs &a, int64_t qi, int64_t wp0, int64_t t, int64_t n_vis,
                                        int64_t ri) {
  if (ri >= a.n_sel) return window_code(a, wp0, t, ri);
  if constexpr (SEL) return selected_code(a, a.topk_idx[qi * a.n_sel + ri]);
  return ri < n_vis ? int(ri) : -1;
}

// Workgroup -> (query, split, head block).  Workgroups are dispatched to the 8 XCDs round-robin by
// linear id, so the head blocks of one (query, split) -- which read the same rows -- are given ids
// that are equal modulo 8 and share that XCD's L2.
struct AttendTile {
  int64_t qi;
  int split, hb;
  bool valid;
};
__device__ __forceinline__ AttendTile attend_tile(const AttendArgs &a, int64_t n_queries, int grid_splits) {
  // 32-bit unsigned arithmetic: the grid holds fewer than 2^31 workgroups
  const uint32_t L = blockIdx.x;
  const uint32_t x = L & 7u, rest = L >> 3;
  const uint32_t n_hb = uint32_t(a.plan.n_hb), gs = uint32_t(grid_splits);
  const uint32_t hb = rest % n_hb;
  const uint32_t pair = (rest / n_hb) * 8u + x;
  AttendTile t;
  t.valid = int64_t(pair) < n_queries * grid_splits;
  t.qi = int64_t(pair / gs);
  t.split = int(pair % gs);
  t.hb = hb;
  return t;
}

// The merge of slice partials, shared by the combine kernel and the fused path so that both give
// the same bits: a slice's partial is x = O / l, rounded to bf16 (the split-K path stores it so:
// half the bytes of fp32 through HBM and back, and a rounding like the output's own), with
// log2-sum-exp m + log2 l in fp32; slices are merged in order with a running maximum M and sum L
// (explicit roundings: no contraction choices).
__device__ __forceinline__ float slice_scale(float l) { return l > 0.f ? 1.0f / l : 0.f; }
__device__ __forceinline__ float slice_value(float o, float inv) {
  return float(__bf16(__fmul_rn(o, inv)));                    // v_cvt_pk_bf16_f32: round to nearest even
}
__device__ __forceinline__ float slice_lse2(float m, float l) { return l > 0.f ? m + log2f(l) : -INFINITY; }
struct MergeWeights {
  float c, w;   // factor of the running sums, weight of the slice
};
__device__ __forceinline__ MergeWeights merge_slice(float &M, float &L, float ls) {
  const float Mn = fmaxf(M, ls);
  MergeWeights k;
  k.c = M == -INFINITY ? 0.f : exp2f(M - Mn);
  k.w = exp2f(ls - Mn);
  L = __fmaf_rn(L, k.c, k.w);
  M = Mn;
  return k;
}
__device__ __forceinline__ float merge_value(float acc, const MergeWeights &k, float x) {
  return __fmaf_rn(k.w, x, __fmul_rn(acc, k.c));
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

// Channel split: a workgroup has NW = D / C waves and wave w owns the channels [C w, C w + C) of
// q, of every row and of O.  All waves take every chunk of the workgroup's slice together.
template <int D>
constexpr int slice_of() { return D >= 128 ? 128 : D; }
template <int D>
constexpr int waves_of() { return D / slice_of<D>(); }
// The launch bound asks for two workgroups per CU (at D = 512: 178 VGPRs, no spills); the split
// planner counts on that.
constexpr int kRing = 4;                   // chunks in flight per wave; chunks go in pairs

typedef __attribute__((address_space(3))) v4s lds_v4s;

// FUSED: one workgroup per (query, head block) takes every slice in order and merges them in
// registers exactly as the combine kernel does (for calls with many queries: no workspace, same
// bits as the split-K path).
template <int D, bool FUSED, bool SEL>
__global__ void __launch_bounds__(64 * waves_of<D>(), 2) attend_split_kernel(AttendArgs a, int64_t n_queries) {
  constexpr int C = slice_of<D>(), NW = waves_of<D>(), NT = 64 * NW;
  constexpr int NS = C / 32;          // 32-channel steps of the wave's slice (QK^T)
  constexpr int NB = C / 16;          // 16-channel blocks of the wave's O^T (PV)
  constexpr int QCH = D / 32;         // prologue: threads per head (32 channels each)
  constexpr int RING = kRing;
  constexpr int RS = 2 * C + 16;      // staging row stride in bytes: 16 B of padding per row, so
                                      // the rows one wide LDS access touches fall in different banks
  constexpr int QS = D + 8;           // q^ row stride (bf16), padded likewise
  constexpr int BUF = (16 * QS * 2 > NW * 32 * RS) ? 16 * QS * 2 : NW * 32 * RS;
  static_assert(QCH * 16 <= NT, "the q prologue needs one thread per 32 channels of a head");
  static_assert(QCH >= 2 && QCH <= 16, "a head's prologue threads share one row of 16 lanes");
  static_assert(D / 2 <= NT, "one rotary pair per thread");
  // LDS: q^ during the prologue, then (same bytes) every wave's staging of its current pair of
  // chunks (their row slices) for the transposing V reads; the waves' S partials (two pairs of chunks, double-buffered); row
  // codes; rotary angles.
  __shared__ __align__(16) unsigned char s_buf[BUF];
  __shared__ __align__(16) float4 s_part[3][2][NW][64];
  __shared__ int s_row[kMaxRowsPerSplit];
  __shared__ float s_cs[256], s_sn[256];
  uint16_t *s_q = reinterpret_cast<uint16_t *>(s_buf);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const AttendTile tl = attend_tile(a, n_queries, FUSED ? 1 : a.plan.n_splits);
  if (!tl.valid) return;
  const int hb = tl.hb;
  const int64_t qi = tl.qi;
  const int b = int(uint32_t(qi) / uint32_t(a.Sq)), s_idx = int(qi) - b * a.Sq;   // B * Sq < 2^16
  const int split_first = FUSED ? 0 : tl.split;
  const int split_end = FUSED ? a.plan.n_splits : tl.split + 1;

  // A segment of the row list -- one slice, or in the fused path every slice when the whole list
  // fits the row-code buffer (one continuous stream of chunks, no restart between slices) --
  // begins with its row codes in LDS and its first chunks' loads in flight.
  const bool stream = FUSED && a.plan.n_rows <= kMaxRowsPerSplit;
  const int n_seg = stream ? 1 : split_end - split_first;
  // ---- prologue.  The selection behind the first segment's row-code table (thread tid: rows
  // tid + k NT) is read first of all: it needs no position, so its round trip runs beside the
  // position's instead of after it.  Reads are clamped to the query's selection; a clamped value
  // is not used.  Then the raw q chunk (and norm weights) of this thread -- loads complete in
  // issue order, so anything issued later (the row prefetch) does not delay them.
  const int64_t r0_first = stream ? 0 : int64_t(split_first) * a.plan.rows_per_split;
  const int nr_first = int((stream ? int64_t(a.plan.n_rows)
                                   : min(int64_t(a.plan.n_rows), r0_first + a.plan.rows_per_split)) - r0_first);
  constexpr int KP = 4;
  int pre_e[KP];
  if constexpr (SEL) {
    const int32_t *sel = a.topk_idx + qi * a.n_sel;
    const int64_t last = a.n_sel - 1;
#pragma unroll
    for (int k = 0; k < KP; ++k) pre_e[k] = sel[min(r0_first + min(tid + k * NT, nr_first - 1), last)];
  }
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
  __builtin_amdgcn_sched_barrier(0);             // keep the q loads ahead of the position wait
  // the rotary frequencies do not need the position: thread u forms pair u's (rope_dim / 2 <= D / 2
  // <= NT pairs) while the position is on its way
  const int npairs = a.rope_dim / 2;
  const double rf = tid < npairs ? rope_turns_per_pos(tid, rope_rate(a.rope_dim, a.log2_base)) : 0.0;
  const int64_t t = a.q_pos0[b] + s_idx;
  const int64_t wp0 = a.win_pos0 ? a.win_pos0[b] : 0;
  const int64_t n_vis = SEL ? 0 : min(a.n_entries[b], div_count(t + 1, a.m));
  if (tid < npairs) rope_cos_sin_f(t, rf, &s_cs[tid], &s_sn[tid]);
  const uint16_t *ent_b = a.entries + int64_t(b) * a.N_cap * D + C * wave;
  const uint16_t *win_b = a.win_rows + int64_t(b) * a.W_cap * D + C * wave;
  // the fused path's running merge of the slices (per head r; lane's channels as in O^T below)
  float fM = -INFINITY, fL = 0.f;
  v4f facc[FUSED ? NB : 1];
#pragma unroll
  for (int k = 0; k < (FUSED ? NB : 1); ++k) facc[k] = v4f{0.f, 0.f, 0.f, 0.f};
  Frag8 qf[NS];

  // slice state: its row count and chunks, the ring of row-slice fragments (lane (r, g) holds row
  // r of the chunk, channels C w + 32 s + 8 g .. +7) and the row codes in the ring
  int nr = 0, n_chunks = 0;
  Frag8 ring[RING][NS];
  int codes[RING];
  // Loads are unconditional (an empty slot reads entry row 0, which exists and is finite; its
  // softmax weight is exactly 0): every path through the loop issues the same loads in the same
  // order, so the wait before a chunk covers that chunk's slot only.
  auto issue = [&](int j, int slot) {            // the slice's j-th chunk
    const int i = j * 16 + r;
    const int code = (j < n_chunks && i < nr) ? s_row[i] : -1;
    codes[slot] = code;
    const uint16_t *rp = code < 0 ? ent_b
                                  : (code < a.N_cap ? ent_b + int64_t(code) * D : win_b + (int64_t(code) - a.N_cap) * D);
#pragma unroll
    for (int s = 0; s < NS; ++s) ring[slot][s].u = *reinterpret_cast<const uint4 *>(rp + 32 * s + 8 * g);
  };
  // (the first segment's table takes the selection read at the start)
  auto begin_segment = [&](int seg) __attribute__((always_inline)) {
    const int64_t r0 = stream ? 0 : int64_t(split_first + seg) * a.plan.rows_per_split;
    const int64_t r1 = stream ? a.plan.n_rows : min(int64_t(a.plan.n_rows), r0 + a.plan.rows_per_split);
    nr = int(r1 - r0);
    n_chunks = (nr + 15) >> 4;
    int i0 = tid;
    if (seg == 0) {
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int i = tid + k * NT;
        if (i < nr) {
          const int64_t ri = r0 + i;
          s_row[i] = (SEL && ri < a.n_sel) ? selected_code(a, pre_e[k]) : row_code<SEL>(a, qi, wp0, t, n_vis, ri);
        }
      }
      i0 = tid + KP * NT;
    }
    for (int i = i0; i < nr; i += NT) s_row[i] = row_code<SEL>(a, qi, wp0, t, n_vis, r0 + i);
    lds_barrier();
#pragma unroll
    for (int j = 0; j < RING; ++j) issue(j, j);
  };
  begin_segment(0);                              // its loads go out before q^ is built

  // q^ = RoPE(RMSNorm(q)) * scale * log2(e) for the 16 heads, into LDS, 8 channels at a time
  // (few registers: the row loads above are in flight meanwhile)
  if (qthread) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = elem8(qraw[k], e);
        ss += x * x;
      }
    }
    // over the head's QCH (2 to 16) consecutive threads, inside one row of 16 lanes: DPP
    ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0xb1, 0xf, 0xf, false));
    if constexpr (QCH >= 4) ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x4e, 0xf, 0xf, false));
    if constexpr (QCH >= 8) ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x141, 0xf, 0xf, false));
    if constexpr (QCH >= 16) ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x140, 0xf, 0xf, false));
    const float inv = qhead < a.H ? rsqrtf(ss / float(D) + a.eps) * a.scale_log2 : 0.f;
    const bool has_w = a.q_norm_w != nullptr;
    const int rope0 = D - a.rope_dim;
    // the rotary pairs of this thread's 32 channels (pair u = (ch - rope0) / 2 = u0 + p), read from
    // LDS together so that one wait covers them all; reads below the rotated part are clamped
    // to pair 0 and not used
    float rcs[16], rsn[16];
    {
      const int u0 = (32 * qc - rope0) >> 1;       // rope0 is even: exact
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int u = max(u0 + p, 0);
        rcs[p] = s_cs[u];
        rsn[p] = s_sn[u];
      }
    }
    uint4 *dst = reinterpret_cast<uint4 *>(s_q + qh * QS + 32 * qc);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = elem8(qraw[k], e) * inv * (has_w ? elem8(wraw[k], e) : 1.0f);
      const int ch0 = 32 * qc + 8 * k;
      if (ch0 + 8 > rope0) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int ch = ch0 + e;
          if (ch >= rope0) {
            const float cs = rcs[(8 * k + e) >> 1], sn = rsn[(8 * k + e) >> 1], x0 = v[e], x1 = v[e + 1];
            v[e] = x0 * cs - x1 * sn;
            v[e + 1] = x0 * sn + x1 * cs;
          }
        }
      }
      Pack4 lo, hi;
      lo.s = pack4(v[0], v[1], v[2], v[3]);
      hi.s = pack4(v[4], v[5], v[6], v[7]);
      dst[k] = make_uint4(uint32_t(uint16_t(lo.s[0])) | (uint32_t(uint16_t(lo.s[1])) << 16),
                          uint32_t(uint16_t(lo.s[2])) | (uint32_t(uint16_t(lo.s[3])) << 16),
                          uint32_t(uint16_t(hi.s[0])) | (uint32_t(uint16_t(hi.s[1])) << 16),
                          uint32_t(uint16_t(hi.s[2])) | (uint32_t(uint16_t(hi.s[3])) << 16));
    }
  }
  lds_barrier();
  // this wave's q^ slice as B operands (lane (r, g): head r, channels C w + 32 s + 8 g .. +7).  The
  // staging area reuses these bytes: every wave's reads complete before any wave stages rows.
#pragma unroll
  for (int s = 0; s < NS; ++s) qf[s].u = *reinterpret_cast<const uint4 *>(s_q + r * QS + C * wave + 32 * s + 8 * g);
  lds_barrier();

  // O^T block nb (O^T = V^T P^T): lane (r, g) element v = head r, channel C w + 16 nb + 4 g + v
  v4f o[NB];
  float m_run, l_run;                             // of head r; the same in every wave
  auto reset_slice = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NB; ++k) o[k] = v4f{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  };
  reset_slice();
  unsigned char *stage = s_buf + wave * 32 * RS;
  int split = split_first;                        // the slice being accumulated

  // Two chunks (32 rows) per step, straight-line code.  Row order within the step: k = 8g + v is
  // row 4g + v of the first chunk for v < 4 and row 4g + v - 4 of the second for v >= 4, so the
  // S^T accumulator layout (lane (r, g): rows 4g..4g+3 of head r) gives the P^T operand directly.
  //   S^T partial = K_slice q^_slice^T over the wave's channels (rows as A operand, q^ as B),
  //   summed over the waves through LDS in wave order; then one running-max update and rescale
  //   for the 32 rows (every wave runs the same arithmetic on the same logits, so m and l agree
  //   across the waves); the rows go to the wave's staging area and two transposing LDS reads give
  //   the A operand V^T[16 channels x 32 rows] of O^T += V^T P^T.
  // A pair is taken in two halves, software-pipelined one pair apart: half A stages the pair's
  // rows, reads its V^T fragments back and forms this wave's S^T partial (MFMAs), which it leaves
  // in LDS; half B sums the waves' partials (the exchange, one barrier) and runs the softmax and
  // O^T += V^T P^T.  After pair p's exchange, half A of pair p + 1 is issued before the rest of
  // pair p's half B, so the next pair's LDS traffic and products run through this pair's softmax
  // chain.  The arithmetic of each pair is unchanged (the same bits as taking the halves back to
  // back).  Partial buffers rotate (pair p uses p mod 3): pair p + 1's are written after the
  // barrier of pair p, which no wave passes before every wave has read pair p - 1's.
  Frag8 vtp[2][NB];                               // V^T fragments of the pairs in flight (by parity)
  v4f spp[2][2];                                  // their S^T (this wave's partial, then the sum)
  uint64_t vmp[2][2];                             // their rows' validity masks
  auto pair_a = [&](int slot0, int par, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
        *reinterpret_cast<uint4 *>(stage + (16 * c + r) * RS + (32 * s + 8 * g) * 2) = ring[slot0 + c][s].u;
    }
    // V^T fragment of block nb: lane (n, g) reads row 4g + n/4, channels 16 nb + 4(n%4) .. +3;
    // the transposing read hands lane (n, g) rows 4g .. 4g+3 of channel 16 nb + n
    const unsigned char *vbase = stage + (4 * g + (r >> 2)) * RS + 8 * (r & 3);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      vtp[par][nb].h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vbase + 32 * nb));
      vtp[par][nb].h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vbase + 16 * RS + 32 * nb));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      spp[par][c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        spp[par][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[slot0 + c][s].b, qf[s].b, spp[par][c], 0, 0, 0);
    }
    if constexpr (NW > 1) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
        s_part[buf][c][wave][lane] = make_float4(spp[par][c][0], spp[par][c][1], spp[par][c][2], spp[par][c][3]);
    }
    vmp[par][0] = __ballot(codes[slot0] >= 0);
    vmp[par][1] = __ballot(codes[slot0 + 1] >= 0);
  };
  // half B, first the exchange: the waves' partials of the pair summed in wave order
  auto pair_x = [&](int par, int buf) __attribute__((always_inline)) {
    if constexpr (NW > 1) {
      lds_barrier();
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float4 x = s_part[buf][c][0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
          const float4 y = s_part[buf][c][w][lane];
          x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
        }
        spp[par][c] = v4f{x.x, x.y, x.z, x.w};
      }
    }
  };
  // then the softmax and O^T += V^T P^T
  auto pair_b = [&](int par) __attribute__((always_inline)) {
    const v4f sp[2] = {spp[par][0], spp[par][1]};
    const uint64_t vm0 = vmp[par][0], vm1 = vmp[par][1];
    float sv[8], cmax = -INFINITY;
    if ((vm0 & vm1) == ~uint64_t(0)) {            // every row of the pair present (wave-uniform)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[v] = sp[0][v];
        sv[4 + v] = sp[1][v];
      }
    } else {                                      // rows 4g .. 4g+3 of each chunk: this lane's bits
      const uint32_t bits = (uint32_t(vm0 >> (4 * g)) & 0xfu) | ((uint32_t(vm1 >> (4 * g)) & 0xfu) << 4);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[v] = (bits & (1u << v)) ? sp[0][v] : -INFINITY;
        sv[4 + v] = (bits & (16u << v)) ? sp[1][v] : -INFINITY;
      }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) cmax = fmaxf(cmax, sv[v]);
    cmax = group4_max(cmax);
    // v_exp_f32 directly: every argument is <= 0, tiny results may flush to zero (they are below
    // 2^-126 of the head's largest weight), and exp2(-inf) = 0 masks the empty rows
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;      // no valid row yet: every sv is -inf
    float p[8], psum = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      p[v] = __builtin_amdgcn_exp2f(sv[v] - m_use);
      psum += p[v];
    }
    l_run = l_run * alpha + group4_sum(psum);
    m_run = m_new;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
#pragma unroll
      for (int v = 0; v < 4; ++v) o[k][v] *= alpha;
    }
    Frag8 pf;
    pf.h[0] = pack4(p[0], p[1], p[2], p[3]);
    pf.h[1] = pack4(p[4], p[5], p[6], p[7]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vtp[par][nb].b, pf.b, o[nb], 0, 0, 0);
  };
  // ---- end of a slice: this wave's channels of O / l and the slice's log2-sum-exp ------------
  auto end_slice = [&]() __attribute__((always_inline)) {
  const int gh = hb * 16 + r;
  const float inv = slice_scale(l_run);
  const float ls = slice_lse2(m_run, l_run);
  const int c0 = C * wave + 4 * g;
  if constexpr (FUSED) {
    if (ls != -INFINITY) {                        // as the combine kernel: empty slices are skipped
      const MergeWeights k = merge_slice(fM, fL, ls);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) facc[nb][v] = merge_value(facc[nb][v], k, slice_value(o[nb][v], inv));
    }
  } else if (gh < a.H) {
    if (a.plan.n_splits == 1) {
      uint16_t *dst = a.out + (qi * a.H + gh) * D + c0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<v4s *>(dst + 16 * nb) = pack4(slice_value(o[nb][0], inv), slice_value(o[nb][1], inv),
                                                       slice_value(o[nb][2], inv), slice_value(o[nb][3], inv));
      if (a.lse && wave == 0 && g == 0) a.lse[qi * a.H + gh] = ls * 0.6931471805599453f;
    } else {
      // workspace: bf16 partials [query, head, slice, D], then fp32 log2-sum-exps [query, head, slice]
      uint16_t *po = static_cast<uint16_t *>(a.workspace);
      float *plse = reinterpret_cast<float *>(po + n_queries * a.H * a.plan.n_splits * D);
      uint16_t *dst = po + ((qi * a.H + gh) * a.plan.n_splits + split) * int64_t(D) + c0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<v4s *>(dst + 16 * nb) = pack4(slice_value(o[nb][0], inv), slice_value(o[nb][1], inv),
                                                       slice_value(o[nb][2], inv), slice_value(o[nb][3], inv));
      if (wave == 0 && g == 0) plse[(qi * a.H + gh) * a.plan.n_splits + split] = ls;
    }
  }
  };

  // The barrier inside a pair is reached by every wave (n_chunks is the same for all of them); the
  // S partial buffers alternate between consecutive pairs, so one barrier per pair suffices.  An
  // empty second chunk (odd chunk count) reads the dummy row and is masked out.  Slices are whole
  // pairs (rows_per_split is a multiple of 32), so in a stream a slice ends between two pairs and
  // its pairs are exactly the ones the split-K path takes for it.
  const int cps = a.plan.rows_per_split >> 4;     // chunks per slice (even)
  for (int seg = 0; seg < n_seg; ++seg) {
    if (seg != 0) {
      lds_barrier();                              // the previous segment's readers of the row codes are done
      begin_segment(seg);
    }
    // pair q uses ring slots 2 (q mod 2) and +1 and partial buffer q mod 3; its slots are refilled
    // (with pair q + 2's chunks) once its half A has read them
    // (the fused kernel, short of registers for two pairs in flight, takes the halves back to back)
    const int np = (n_chunks + 1) >> 1;
    if constexpr (!FUSED) pair_a(0, 0, 0);
    for (int q0 = 0; q0 < np; q0 += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = q0 + h;
        if (q < np) {
          const int j = 2 * q;
          if constexpr (FUSED) {
            pair_a(2 * h, 0, q % 3);
            issue(j + RING, 2 * h);               // pair q's slots: pair q + 2
            issue(j + 1 + RING, 2 * h + 1);
            pair_x(0, q % 3);
            pair_b(0);
            if ((j + 2) % cps == 0 && j + 2 < n_chunks) {   // a slice ends inside the stream
              end_slice();
              ++split;
              reset_slice();
            }
          } else {
            // pair q's exchange first (its partials were written an iteration ago), then pair
            // q + 1's half A, whose LDS traffic and products overlap pair q's softmax
            pair_x(h, q % 3);
            issue(j + RING, 2 * h);               // pair q's slots: pair q + 2
            issue(j + 1 + RING, 2 * h + 1);
            if (q + 1 < np) pair_a(2 * (h ^ 1), h ^ 1, (q + 1) % 3);
            pair_b(h);
          }
        }
      }
    }
    end_slice();
    ++split;
    reset_slice();
  }

  if constexpr (FUSED) {
    const int gh = hb * 16 + r;
    if (gh < a.H) {
      const float finv = fL > 0.f ? 1.0f / fL : 0.f;
      uint16_t *dst = a.out + (qi * a.H + gh) * D + C * wave + 4 * g;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<v4s *>(dst + 16 * nb) = pack4(__fmul_rn(facc[nb][0], finv), __fmul_rn(facc[nb][1], finv),
                                                       __fmul_rn(facc[nb][2], finv), __fmul_rn(facc[nb][3], finv));
      if (a.lse && wave == 0 && g == 0)
        a.lse[qi * a.H + gh] = fL > 0.f ? (fM + log2f(fL)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

// One workgroup per (query, head): merge the slices in order.
template <int D>
__global__ void __launch_bounds__(D / 4) attend_combine_kernel(AttendArgs a, int64_t n_queries) {
  constexpr int kBatch = 8;                       // slices whose loads are in flight together
  const int64_t qh = blockIdx.x;                  // query * H + head
  const int ns = a.plan.n_splits;
  const uint16_t *po = static_cast<const uint16_t *>(a.workspace) + qh * ns * int64_t(D);
  const float *plse = reinterpret_cast<const float *>(static_cast<const uint16_t *>(a.workspace) +
                                                      n_queries * a.H * ns * int64_t(D)) + qh * ns;
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
      const uint2 w = *reinterpret_cast<const uint2 *>(po + s * int64_t(D) + ch);
      x[j] = make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j >= ns || ls[j] == -INFINITY) continue;
      const MergeWeights k = merge_slice(M, L, ls[j]);
      acc.x = merge_value(acc.x, k, x[j].x); acc.y = merge_value(acc.y, k, x[j].y);
      acc.z = merge_value(acc.z, k, x[j].z); acc.w = merge_value(acc.w, k, x[j].w);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  uint16_t *dst = a.out + qh * D + ch;
  *reinterpret_cast<v4s *>(dst) = pack4(__fmul_rn(acc.x, inv), __fmul_rn(acc.y, inv), __fmul_rn(acc.z, inv),
                                        __fmul_rn(acc.w, inv));
  if (a.lse && threadIdx.x == 0) a.lse[qh] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

}  // namespace

AttendPlan plan_attend(int64_t n_queries, int H, int64_t n_sel, int window, int D) {
  AttendPlan p;
  p.n_hb = (H + 15) / 16;
  p.n_rows = int(n_sel + window);
  // The slices depend on the row count alone -- never on how many queries share the call -- so a
  // query's output has the same bits in any batch (batch invariance): up to 16 slices of about 144
  // rows or more, each a multiple of 32 rows (a pair of 16-row chunks).  (k + W = 1,152 rows give 8
  // slices: 512 workgroups, one round, for 16 queries of 64 heads.)
  int64_t splits = (p.n_rows + 143) / 144;
  if (splits > 16) splits = 16;
  if (splits < 1) splits = 1;
  int64_t rps = (p.n_rows + splits - 1) / splits;
  rps = (rps + 31) / 32 * 32;
  if (rps > kMaxRowsPerSplit) rps = kMaxRowsPerSplit;
  p.rows_per_split = int(rps);
  p.n_splits = int((p.n_rows + rps - 1) / rps);
  // Split-K (a workgroup per slice, partials merged by the combine kernel) while the grid stays
  // within a few rounds of resident workgroups (two per CU); beyond that one workgroup per
  // (query, head block) takes the slices in order and merges them itself, with no workspace.
  p.fused = (p.n_splits > 1 && n_queries * p.n_hb * p.n_splits > 4 * 512) ? 1 : 0;
  (void)D;
  return p;
}

size_t attend_workspace_bytes(int64_t n_queries, int H, int D, int64_t n_sel, int window) {
  AttendPlan p = plan_attend(n_queries, H, n_sel, window, D);
  if (p.n_splits == 1 || p.fused) return 256;
  return size_t(n_queries * H * p.n_splits * (int64_t(D) * 2 + 4) + 256);   // bf16 partials, fp32 lse
}

// ---- the library's own scratch for csa_attend_noalloc -------------------------------------------
// One file-scope device array (each GPU the library runs on holds its own copy from module load to
// process exit).  Host code never passes the array's name to a kernel: its device address on the
// current device comes from hipGetSymbolAddress, taken once per device and kept.
namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

size_t attend_scratch_bytes() { return kScratchBytes; }

hipError_t attend_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attend(const AttendArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  const int64_t nq = int64_t(a.B) * a.Sq;
  const int64_t pairs = nq * (a.plan.fused ? 1 : a.plan.n_splits);
  dim3 grid(unsigned(((pairs + 7) / 8) * 8 * a.plan.n_hb));
#define CSA_ATTEND_LAUNCH(DD)                                                                          \
  if (a.topk_idx)                                                                                      \
    e = a.plan.fused ? launch("attend_split", attend_split_kernel<DD, true, true>, grid, dim3(64 * waves_of<DD>()), stream, a, nq) \
                     : launch("attend_split", attend_split_kernel<DD, false, true>, grid, dim3(64 * waves_of<DD>()), stream, a, nq); \
  else                                                                                                 \
    e = a.plan.fused ? launch("attend_split", attend_split_kernel<DD, true, false>, grid, dim3(64 * waves_of<DD>()), stream, a, nq) \
                     : launch("attend_split", attend_split_kernel<DD, false, false>, grid, dim3(64 * waves_of<DD>()), stream, a, nq)
  switch (a.D) {
    case 64: CSA_ATTEND_LAUNCH(64); break;
    case 128: CSA_ATTEND_LAUNCH(128); break;
    case 256: CSA_ATTEND_LAUNCH(256); break;
    case 512: CSA_ATTEND_LAUNCH(512); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA_ATTEND_LAUNCH
  return e;
}

hipError_t launch_combine(const AttendArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.plan.n_splits == 1 || a.plan.fused) return hipSuccess;
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
