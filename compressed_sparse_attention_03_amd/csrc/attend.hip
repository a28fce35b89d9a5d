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
// Long row lists at D = 512 take a head-shared kernel instead (attend_rows_kernel below: one
// workgroup of 64 heads per slice, rows streamed once through LDS), which gives the same bits.
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
constexpr int kLongList = 2048;     // row lists longer than this are sliced finer (see plan_attend)

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

// One pair's online-softmax step for head r, shared by every attention kernel so that all give
// the same bits.  Lane (r, g) holds the pair's logits of rows 4g .. 4g+3 of each chunk (exp2
// domain); vm0 / vm1 are the chunks' row-validity ballots (bit i: row i mod 16 present).  The
// reference maximum of a head moves only when a logit exceeds it by more than 2^kLazy (or on its
// first valid row): weights stay below 2^kLazy (no overflow, and bf16 keeps its relative
// precision), and the running output needs rescaling only on such a move -- rarely after the first
// rows -- so the caller skips the multiply when no lane of the wave moved.  O / l and m + log2 l
// are unchanged by the choice of reference.
constexpr float kLazy = 8.f;
struct PairSoftmax {
  float alpha;      // factor of the running output and sum (1 when the maximum stayed)
  bool rescale;     // some lane of the wave has alpha != 1
};
__device__ __forceinline__ PairSoftmax pair_softmax(const v4f &s0, const v4f &s1, uint64_t vm0, uint64_t vm1, int g,
                                                    float &m_run, float &l_run, Frag8 &pf) {
  float sv[8], cmax = -INFINITY;
  if ((vm0 & vm1) == ~uint64_t(0)) {              // every row of the pair present (wave-uniform)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = s0[v];
      sv[4 + v] = s1[v];
    }
  } else {                                        // rows 4g .. 4g+3 of each chunk: this lane's bits
    const uint32_t bits = (uint32_t(vm0 >> (4 * g)) & 0xfu) | ((uint32_t(vm1 >> (4 * g)) & 0xfu) << 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = (bits & (1u << v)) ? s0[v] : -INFINITY;
      sv[4 + v] = (bits & (16u << v)) ? s1[v] : -INFINITY;
    }
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) cmax = fmaxf(cmax, sv[v]);
  cmax = group4_max(cmax);
  // (m_run = -inf: any valid row moves it; cmax = -inf: no valid row, nothing moves)
  const bool move = cmax > m_run + kLazy;
  const float m_new = move ? cmax : m_run;
  PairSoftmax r;
  r.alpha = !move ? 1.f : (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new));
  r.rescale = __ballot(move) != 0;
  // v_exp_f32 directly: every argument is <= kLazy, tiny results may flush to zero (below 2^-126
  // of the reference), and exp2(-inf) = 0 masks the empty rows
  const float m_use = m_new == -INFINITY ? 0.f : m_new;   // no valid row yet: every sv is -inf
  float p[8], psum = 0.f;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    p[v] = __builtin_amdgcn_exp2f(sv[v] - m_use);
    psum += p[v];
  }
  l_run = __fmaf_rn(l_run, r.alpha, group4_sum(psum));
  m_run = m_new;
  pf.h[0] = pack4(p[0], p[1], p[2], p[3]);
  pf.h[1] = pack4(p[4], p[5], p[6], p[7]);
  return r;
}

// The query operands of S^T = K Q^T: q^ = RoPE(RMSNorm(q)) * softmax scale * log2(e).  Every
// kernel forms them with the same arithmetic, so all give the same bits, whichever lanes hold
// which channels: a head's D channels are 32-channel groups k (k = 0 .. D/32 - 1) of four 8-channel
// runs j (channels 32k + 8j .. +7); the sum of squares is, per run j, a sequential sum over its 8
// channels within each group k, then a butterfly over k (k ^ 1, k ^ 2, the mirror within eight, the
// mirror within sixteen -- the lane-row DPP exchanges, for QCH = D / 32 groups), then over the runs
// as (U0 + U1) + (U2 + U3).  The channel-split kernel's prologue has a thread per (head, group k)
// and does the butterfly across lanes; the head-shared kernel's lane (head, run j) holds run j of
// every group and does it in registers.
__device__ __forceinline__ float run_sumsq(const uint4 &x) {     // sequential over the 8 channels
  float p = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = elem8(x, e);
    p = __fmaf_rn(v, v, p);
  }
  return p;
}
// The butterfly over 16 groups held in one lane (P[k] of run j; every P[k] ends with the same total).
__device__ __forceinline__ float groups16_sum(float (&P)[16]) {
  float t[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) t[k] = P[k] + P[k ^ 1];
#pragma unroll
  for (int k = 0; k < 16; ++k) P[k] = t[k] + t[k ^ 2];
#pragma unroll
  for (int k = 0; k < 16; ++k) t[k] = P[k] + P[(k & 8) | (7 - (k & 7))];
  return t[0] + t[15];
}
// (U0 + U1) + (U2 + U3) over the lanes (head, run j) = l, l ^ 16, l ^ 32, l ^ 48, in every lane.
__device__ __forceinline__ float runs4_sum(float u) {
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(u), false, false);
  const float y = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float q_inv(const AttendArgs &a, float ss, int D, int head) {
  return head < a.H ? rsqrtf(ss / float(D) + a.eps) * a.scale_log2 : 0.f;
}
// Operand of the channels ch0 .. ch0 + 7 (ch0 = 32k + 8g): x = q's channels, w = the norm weight's
// (unused without one); the last rope_dim channels (from rope0) are rotated by pairs with the cos /
// sin table.  rot (wave-uniform): some lane's channels of this k reach rope0.
__device__ __forceinline__ Frag8 q_frag(const uint4 &x, const uint4 &w, bool has_w, int ch0, bool rot, float inv,
                                        int rope0, const float *s_cs, const float *s_sn) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = __fmul_rn(__fmul_rn(elem8(x, e), inv), has_w ? elem8(w, e) : 1.0f);
  if (rot) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int ch = ch0 + e;
      const int u = max(ch - rope0, 0) >> 1;        // rope0 is even: exact; below rope0 unused
      const float cs = s_cs[u], sn = s_sn[u], x0 = v[e], x1 = v[e + 1];
      const float y0 = __fmaf_rn(x0, cs, -__fmul_rn(x1, sn));
      const float y1 = __fmaf_rn(x0, sn, __fmul_rn(x1, cs));
      v[e] = ch >= rope0 ? y0 : x0;
      v[e + 1] = ch >= rope0 ? y1 : x1;
    }
  }
  Frag8 f;
  f.h[0] = pack4(v[0], v[1], v[2], v[3]);
  f.h[1] = pack4(v[4], v[5], v[6], v[7]);
  return f;
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
  // chunks (their row slices) for the transposing V reads; the waves' S partials (three pairs in
  // rotation); row codes; rotary angles.
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
  // prologue thread (head qh, group qc): q's channels 32 qc .. +31 and the norm weight's
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

  // q^ of the 16 heads into LDS (the rotary table is published by the row-code barrier above): run
  // sums, the butterfly over the head's QCH threads (one lane row), then over the runs
  if (qthread) {
    float P[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) P[j] = run_sumsq(qraw[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      P[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(P[j]), 0xb1, 0xf, 0xf, false));
      if constexpr (QCH >= 4) P[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(P[j]), 0x4e, 0xf, 0xf, false));
      if constexpr (QCH >= 8) P[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(P[j]), 0x141, 0xf, 0xf, false));
      if constexpr (QCH >= 16) P[j] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(P[j]), 0x140, 0xf, 0xf, false));
    }
    const float inv = q_inv(a, (P[0] + P[1]) + (P[2] + P[3]), D, qhead);
    const bool has_w = a.q_norm_w != nullptr;
    const int rope0 = D - a.rope_dim;
    uint4 *dst = reinterpret_cast<uint4 *>(s_q + qh * QS + 32 * qc);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ch0 = 32 * qc + 8 * k;
      dst[k] = q_frag(qraw[k], wraw[k], has_w, ch0, ch0 + 8 > rope0, inv, rope0, s_cs, s_sn).u;
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
    Frag8 pf;
    const PairSoftmax sm = pair_softmax(spp[par][0], spp[par][1], vmp[par][0], vmp[par][1], g, m_run, l_run, pf);
    if (sm.rescale) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
#pragma unroll
        for (int v = 0; v < 4; ++v) o[k][v] *= sm.alpha;
      }
    }
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
  } else {
    // through the wave's staging area (only this wave reads it, and its last pair's V^T fragments
    // are in registers): each store writes whole 2C-byte rows of four heads instead of 32-byte
    // pieces of sixteen
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<v4s *>(stage + r * RS + 2 * (16 * nb + 4 * g)) =
          pack4(slice_value(o[nb][0], inv), slice_value(o[nb][1], inv), slice_value(o[nb][2], inv),
                slice_value(o[nb][3], inv));
    wave_lds_sync();
    // workspace: bf16 partials [query, head, slice, D], then fp32 log2-sum-exps [query, head, slice]
    uint16_t *po = static_cast<uint16_t *>(a.workspace);
    const int ns = a.plan.n_splits;
    if (gh < a.H && wave == 0 && g == 0) {
      if (ns == 1) {
        if (a.lse) a.lse[qi * a.H + gh] = ls * 0.6931471805599453f;
      } else {
        reinterpret_cast<float *>(po + n_queries * a.H * ns * D)[(qi * a.H + gh) * ns + split] = ls;
      }
    }
    constexpr int LPH = C / 8;                    // lanes per head row (16 bytes each)
#pragma unroll
    for (int j = 0; j < 16 * LPH / 64; ++j) {
      const int h = j * (64 / LPH) + lane / LPH, part = lane % LPH;
      const int64_t head = qi * a.H + hb * 16 + h;
      if (hb * 16 + h < a.H) {
        const uint4 v = *reinterpret_cast<const uint4 *>(stage + h * RS + 16 * part);
        uint16_t *dst = ns == 1 ? a.out + head * D : po + (head * ns + split) * int64_t(D);
        *reinterpret_cast<uint4 *>(dst + C * wave + 8 * part) = v;
      }
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

// ---- head-shared decode attention (D = 512) ------------------------------------------------------
// One workgroup per (query, slice of the row list, group of 64 heads): wave w owns head block w of
// the group (16 heads) over all 512 channels, so no S partial crosses waves and every row is read
// from memory once for the 64 heads.  A slice's rows stream through a ring of three 32-row LDS
// buffers filled by direct-to-LDS buffer loads (one 1 KiB row per wave instruction); every wave
// reads its MFMA operands from the shared buffers:
//   S^T [16 rows x 16 heads] per 128-channel quarter = K_q Q_q^T   (16-byte LDS reads, A operand)
//   S^T = ((S_0 + S_1) + S_2) + S_3                                  in fp32, in quarter order
//   online softmax in the exp2 domain (pair_softmax), per 32 rows
//   O^T [512 ch x 16 heads] += V^T P^T                               (transposing LDS reads)
// It takes the split-K path of long row lists (HCA's every entry), where one read of each row for
// all 64 heads and a whole CU per workgroup beat four head-block workgroups re-reading it.
// These are the channel-split kernel's operations on the same operands in the same order (its
// waves' S partials summed in wave order are the quarters' sums here), so both kernels -- and the
// fused path, which runs the channel-split kernel -- give the same bits.
//
// Rows sit kRowsStride bytes apart (1 KiB + 32: rows 8 apart fall on the same banks) and a row's
// 16-byte column c is stored at slot c ^ row_swz(row) (row_swz = bit 3 of the row): the 16 rows of
// one operand read (16 lanes x 16 bytes) cover every bank once, and so do the 32 lanes of a
// transposing read (8 rows x 32 bytes).
constexpr int kRowsBytes = 1024;                  // one 512-channel bf16 row
constexpr int kRowsStride = 1056;                 // its LDS footprint
constexpr int kRowsPair = 32 * kRowsStride;       // one ring buffer: 32 rows
constexpr int kRowsRing = 3;

__device__ __forceinline__ int row_swz(int row) { return (row >> 3) & 1; }

__device__ __forceinline__ uint32_t rows_lds_address(const void *p) {      // p points into LDS
  const __attribute__((address_space(3))) void *l = (const __attribute__((address_space(3))) void *)(p);
  return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(l)));
}
// Lane l's 16 bytes at byte offset voff of the buffer go to LDS address m0 + 16 l.  The compiler
// knows of no load in flight; every wait for these is an explicit vmcnt count.
__device__ __forceinline__ void rows_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void rows_wait() {                 // at most N vector loads in flight
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

template <bool SEL>
__global__ void __launch_bounds__(256, 1) attend_rows_kernel(AttendArgs a, int64_t n_queries) {
  constexpr int D = 512, NT = 256;
  __shared__ __align__(16) unsigned char s_rows[kRowsRing][kRowsPair];
  __shared__ int s_row[kMaxRowsPerSplit];
  __shared__ float s_cs[256], s_sn[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int ns = a.plan.n_splits;
  const int n_hg = (a.plan.n_hb + 3) >> 2;
  const uint32_t L = blockIdx.x;
  const int hg = int(L % uint32_t(n_hg));
  const uint32_t rest = L / uint32_t(n_hg);
  const int64_t qi = int64_t(rest / uint32_t(ns));
  const int split = int(rest % uint32_t(ns));
  if (qi >= n_queries) return;
  const int hb = hg * 4 + wave;                   // this wave's head block
  const int b = int(uint32_t(qi) / uint32_t(a.Sq)), s_idx = int(qi) - b * a.Sq;   // B * Sq < 2^16
  const int64_t r0 = int64_t(split) * a.plan.rows_per_split;
  const int nr = int(min(int64_t(a.plan.n_rows), r0 + a.plan.rows_per_split) - r0);
  const int n_chunks = (nr + 15) >> 4;
  const int np = (n_chunks + 1) >> 1;             // 32-row pairs

  // ---- prologue: every global load of the workgroup except the rows, in one round trip --------
  constexpr int KP = 4;
  int pre_e[KP];
  if constexpr (SEL) {
    const int32_t *sel = a.topk_idx + qi * a.n_sel;
    const int64_t last = a.n_sel - 1;
#pragma unroll
    for (int k = 0; k < KP; ++k) pre_e[k] = sel[min(r0 + min(tid + k * NT, nr - 1), last)];
  }
  // head r's channels 32k + 8g .. +7 of q and of the norm weight, k = 0 .. 15
  const int qhead = hb * 16 + r;
  uint4 qraw[16], wraw[16];
  {
    const uint16_t *src = a.q + (qi * a.H + (qhead < a.H ? qhead : 0)) * D + 8 * g;
    const uint16_t *wsrc = (a.q_norm_w ? a.q_norm_w : a.q) + 8 * g;
#pragma unroll
    for (int k = 0; k < 16; ++k) qraw[k] = *reinterpret_cast<const uint4 *>(src + 32 * k);
    if (a.q_norm_w) {
#pragma unroll
      for (int k = 0; k < 16; ++k) wraw[k] = *reinterpret_cast<const uint4 *>(wsrc + 32 * k);
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) wraw[k] = make_uint4(0, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int npairs = a.rope_dim / 2;
  const double rf = tid < npairs ? rope_turns_per_pos(tid, rope_rate(a.rope_dim, a.log2_base)) : 0.0;
  const int64_t t = a.q_pos0[b] + s_idx;
  const int64_t wp0 = a.win_pos0 ? a.win_pos0[b] : 0;
  const int64_t n_vis = SEL ? 0 : min(a.n_entries[b], div_count(t + 1, a.m));
  if (tid < npairs) rope_cos_sin_f(t, rf, &s_cs[tid], &s_sn[tid]);
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int i = tid + k * NT;
    if (i < nr) {
      const int64_t ri = r0 + i;
      s_row[i] = (SEL && ri < a.n_sel) ? selected_code(a, pre_e[k]) : row_code<SEL>(a, qi, wp0, t, n_vis, ri);
    }
  }
  for (int i = tid + KP * NT; i < nr; i += NT) s_row[i] = row_code<SEL>(a, qi, wp0, t, n_vis, r0 + i);
  for (int i = nr + tid; i < 32 * np; i += NT) s_row[i] = -1;     // the last pair's missing rows
  // every load the compiler issued is complete from here on (it counts none of the row loads)
  __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0)
  lds_barrier();

  // rows of pair P (this wave: rows 8w .. 8w+7 of the pair), one wave instruction per row; an
  // empty row reads entry row 0 (finite, weight exactly 0)
  const __amdgpu_buffer_rsrc_t ent_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.entries + int64_t(b) * a.N_cap * D), short(0), int(uint32_t(a.N_cap) * kRowsBytes),
      kRawBufferDesc3);
  const __amdgpu_buffer_rsrc_t win_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.win_rows + int64_t(b) * a.W_cap * D), short(0), int(uint32_t(a.W_cap) * kRowsBytes),
      kRawBufferDesc3);
  const int n_cap = int(a.N_cap);
  auto issue_pair = [&](int P) __attribute__((always_inline)) {
    unsigned char *buf = s_rows[P % kRowsRing];
    const int4 ca = *reinterpret_cast<const int4 *>(s_row + P * 32 + wave * 8);
    const int4 cb = *reinterpret_cast<const int4 *>(s_row + P * 32 + wave * 8 + 4);
    const int cs[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = wave * 8 + j;
      const int code = __builtin_amdgcn_readfirstlane(cs[j]);
      const bool win = code >= n_cap;
      const uint32_t roff = code < 0 ? 0u : uint32_t(win ? code - n_cap : code) * uint32_t(kRowsBytes);
      const uint32_t voff = roff + 16u * uint32_t(lane ^ row_swz(row));
      rows_load16(win ? win_rs : ent_rs, voff, rows_lds_address(buf + row * kRowsStride));
    }
  };
  if (np > 0) issue_pair(0);
  if (np > 1) issue_pair(1);

  // ---- q^ as this wave's B operands (the rotary table is published by the barrier above) ---------
  Frag8 qf[16];                                   // [quarter q * 4 + step s]: head r, channels 128q + 32s + 8g
  {
    float P[16];                                  // run g of every group k
#pragma unroll
    for (int k = 0; k < 16; ++k) P[k] = run_sumsq(qraw[k]);
    const float inv = q_inv(a, runs4_sum(groups16_sum(P)), D, qhead);
    const bool has_w = a.q_norm_w != nullptr;
    const int rope0 = D - a.rope_dim;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      qf[k] = q_frag(qraw[k], wraw[k], has_w, 32 * k + 8 * g, 32 * k + 32 > rope0, inv, rope0, s_cs, s_sn);
  }

  // ---- the slice's pairs ------------------------------------------------------------------------
  v4f o[32];                                      // [q * 8 + nb]: head r, channels 128q + 16nb + 4g + v
#pragma unroll
  for (int k = 0; k < 32; ++k) o[k] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;           // of head r
  const int kx = row_swz(r);                      // operand rows r and 16 + r
  const int vrow = 4 * g + (r >> 2), vx = row_swz(vrow), vcol = (r & 3) >> 1, vhalf = 8 * (r & 1);
  // O^T += V^T P^T over the pair in `buf`, software-pipelined one channel quarter apart: quarter
  // q + 1's transposing reads are issued before quarter q's products (scheduling fences keep them
  // there)
  auto pv = [&](const unsigned char *buf, const Frag8 &pf) __attribute__((always_inline)) {
    const unsigned char *v0 = buf + vrow * kRowsStride + vhalf;
    Frag8 vt[2][8];
    auto read_v = [&](int q, Frag8 (&dst)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int off = 16 * (16 * q + ((2 * nb + vcol) ^ vx));
        dst[nb].h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(v0 + off));
        dst[nb].h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(v0 + 16 * kRowsStride + off));
      }
    };
    read_v(0, vt[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < 3) read_v(q + 1, vt[(q + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        o[8 * q + nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[q & 1][nb].b, pf.b, o[8 * q + nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The pairs.  A pair whose softmax moves some head's reference maximum leaves the inner loop, and
  // the outer one rescales the running output before its products: the running output then stays
  // in the accumulation registers through the inner loop (no copies for the rare multiply).
  int p = 0;
  const unsigned char *buf = s_rows[0];
  Frag8 pf;
  float alpha = 1.f;
  for (;;) {
    bool moved = false;
    for (; p < np; ++p) {
      if (p + 1 < np) rows_wait<8>(); else rows_wait<0>();   // this wave's rows of pair p are in LDS
      lds_sync();                                 // ... every wave's; and pair p - 1's buffer is free
      if (p + 2 < np) issue_pair(p + 2);
      buf = s_rows[p % kRowsRing];
      // validity of rows r and 16 + r (row order as in the channel-split kernel's masks)
      const uint64_t vm0 = __ballot(s_row[32 * p + r] >= 0);
      const uint64_t vm1 = __ballot(s_row[32 * p + 16 + r] >= 0);
      // S^T of both chunks, quarter by quarter, software-pipelined like the products above: quarter
      // q + 1's eight operand reads go out before quarter q's eight products; then the running
      // sum ((S_0 + S_1) + S_2) + S_3
      v4f sp[2];
      {
        Frag8 kf[2][2][4];
        auto read_k = [&](int q, Frag8 (&dst)[2][4]) __attribute__((always_inline)) {
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int s = 0; s < 4; ++s)
              dst[c][s].u = *reinterpret_cast<const uint4 *>(buf + (16 * c + r) * kRowsStride +
                                                             16 * (16 * q + ((4 * s + g) ^ kx)));
        };
        read_k(0, kf[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < 3) read_k(q + 1, kf[(q + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          v4f part[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < 2; ++c)
              part[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[q & 1][c][s].b, qf[4 * q + s].b, part[c], 0, 0, 0);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            if (q == 0) {
              sp[c] = part[c];
            } else {
              sp[c][0] += part[c][0]; sp[c][1] += part[c][1]; sp[c][2] += part[c][2]; sp[c][3] += part[c][3];
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const PairSoftmax sm = pair_softmax(sp[0], sp[1], vm0, vm1, g, m_run, l_run, pf);
      if (sm.rescale) {
        alpha = sm.alpha;
        moved = true;
        break;
      }
      pv(buf, pf);
    }
    if (!moved) break;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
#pragma unroll
      for (int v = 0; v < 4; ++v) o[k][v] *= alpha;
    }
    pv(buf, pf);
    ++p;
  }
  rows_wait<0>();

  // ---- this wave's heads of the slice: O / l (bf16) and the log2-sum-exp -----------------------
  // The values go through LDS (the ring is idle once every wave is past its last pair) so that each
  // store instruction writes one head's whole 1 KiB row: every workgroup stores its 64 KiB at
  // once at the end, and rows written in 32-byte pieces made that burst several times slower.
  const int gh = hb * 16 + r;
  const float inv = slice_scale(l_run);
  const float ls = slice_lse2(m_run, l_run);
  constexpr int kOutStride = kRowsBytes + 16;     // staging row stride: the lanes of a write differ by row
  static_assert(4 * 16 * kOutStride <= kRowsRing * kRowsPair, "the output staging fits the ring");
  unsigned char *stage = &s_rows[0][0] + wave * 16 * kOutStride;
  lds_sync();                                     // every wave is done with the ring
#pragma unroll
  for (int k = 0; k < 32; ++k)
    *reinterpret_cast<v4s *>(stage + r * kOutStride + 2 * (128 * (k >> 3) + 16 * (k & 7) + 4 * g)) =
        pack4(slice_value(o[k][0], inv), slice_value(o[k][1], inv), slice_value(o[k][2], inv),
              slice_value(o[k][3], inv));
  wave_lds_sync();
  uint16_t *po = static_cast<uint16_t *>(a.workspace);
  const int64_t head0 = qi * a.H + hb * 16;       // this wave's first head (query-major)
  if (gh < a.H && g == 0) {
    if (ns == 1) {
      if (a.lse) a.lse[qi * a.H + gh] = ls * 0.6931471805599453f;
    } else {
      reinterpret_cast<float *>(po + n_queries * a.H * ns * D)[(qi * a.H + gh) * ns + split] = ls;
    }
  }
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (hb * 16 + h >= a.H) break;                // (wave-uniform)
    const uint4 v = *reinterpret_cast<const uint4 *>(stage + h * kOutStride + 16 * lane);
    uint16_t *dst = ns == 1 ? a.out + (head0 + h) * D : po + ((head0 + h) * ns + split) * int64_t(D);
    *reinterpret_cast<uint4 *>(dst + 8 * lane) = v;
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
  const int ch = threadIdx.x * 4, lane = threadIdx.x & 63;
  // every slice's log2-sum-exp and partial are loaded before any is used (one round trip per
  // batch of slices), then merged in slice order with a running maximum.  The log2-sum-exps of a
  // window of slices come in one vector load (lane s: slice w0 + s) and are taken by readlane: as
  // uniform scalar loads, which complete out of order, each use waited for all of them and the
  // compiler issued them one round trip apart.
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int WIN = D / 4 < 64 ? D / 4 : 64;   // slices per window: one per active lane
  static_assert(WIN % kBatch == 0, "a batch stays inside one window");
  for (int w0 = 0; w0 < ns; w0 += WIN) {
    const float lsv = plse[min(w0 + lane, ns - 1)];
    const int wend = min(ns, w0 + WIN);
    for (int s0 = w0; s0 < wend; s0 += kBatch) {
      float ls[kBatch];
      float4 x[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int s = s0 + j < ns ? s0 + j : ns - 1;
        ls[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsv), s - w0));
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
  // query's output has the same bits in any batch (batch invariance), each a multiple of 32 rows (a
  // pair of 16-row chunks).  Lists of up to kLongList rows (CSA selections: k + W = 1,152 rows give
  // 8 slices, 512 channel-split workgroups in one round for 16 queries of 64 heads): up to 16 slices
  // of 144 rows or more.  Longer lists (HCA's every entry; at D = 512 taken by the head-shared
  // kernel, one workgroup of 64 heads per CU): up to 32 slices of 96 rows or more (8,320 rows give
  // 29 slices of 288: 232 workgroups for 8 queries).
  const bool long_list = p.n_rows > kLongList;
  int64_t splits = long_list ? (p.n_rows + 95) / 96 : (p.n_rows + 143) / 144;
  if (splits > (long_list ? 32 : 16)) splits = long_list ? 32 : 16;
  if (splits < 1) splits = 1;
  int64_t rps = (p.n_rows + splits - 1) / splits;
  rps = (rps + 31) / 32 * 32;
  if (rps > kMaxRowsPerSplit) rps = kMaxRowsPerSplit;
  p.rows_per_split = int(rps);
  p.n_splits = int((p.n_rows + rps - 1) / rps);
  // Split-K (a workgroup per slice, partials merged by the combine kernel) while the grid stays
  // within a few rounds of resident workgroups (at D = 512 one head-shared workgroup of 64 heads
  // per CU, else two of 16 heads); beyond that one workgroup per (query, head block) takes the
  // slices in order and merges them itself, with no workspace.
  const bool rows = D == 512 && long_list;
  const int64_t wgs = rows ? n_queries * ((p.n_hb + 3) / 4) * p.n_splits : n_queries * p.n_hb * p.n_splits;
  p.fused = (p.n_splits > 1 && wgs > (rows ? 4 * 256 : 4 * 512)) ? 1 : 0;
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
  // split-K over a long row list at D = 512 (row offsets within 32 bits): the head-shared kernel,
  // which gives the same bits as the channel-split one
  if (a.D == 512 && !a.plan.fused && a.plan.n_rows > kLongList && a.N_cap <= (int64_t(1) << 22) - 1 &&
      a.W_cap <= (int64_t(1) << 22) - 1) {
    dim3 rgrid(unsigned(nq * a.plan.n_splits * ((a.plan.n_hb + 3) / 4)));
    return a.topk_idx ? launch("attend_split", attend_rows_kernel<true>, rgrid, dim3(256), stream, a, nq)
                      : launch("attend_split", attend_rows_kernel<false>, rgrid, dim3(256), stream, a, nq);
  }
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
