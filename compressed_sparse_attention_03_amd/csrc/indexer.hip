// Lightning indexer and top-k selector.
//
// "DeepSeek-V4: Million-Token Context" (codexsims explainer), CSA walk-through: a lightweight
// scoring head rates each compressed block for the present query and only the k highest-rated
// blocks are kept.  "Follow the white rabbit" (sambatista.com), indexer paragraph: at the longest
// context some 262,000 entries are rated and 1,024 survive; compact, low-precision operands keep
// the rating cheap, though its cost still rises with the context length.
//
// score[i] = sum_h w[h] * max(0, <q~_h, k~_i>)  (the form stated in csa.h).
//
// Kernel 1 (index_score): grid (tiles, queries).  The query's [H_I x 128] head matrix is quantised
// once per workgroup into LDS and held as MFMA A-operands; key tiles stream from HBM in groups of
// 16 entries, each group costing one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 heads (fp8 e4m3,
// or MXFP4 with its e8m0 block scales applied by the instruction).  The tile's scores stay in LDS;
// a block radix select keeps the tile's `cand` best (score, index) keys, written in ascending
// index order together with the smallest kept key.
// Kernel 1b (index_score_multi_kernel, calls with eight or more queries per sequence): a tile of
// 512 keys is loaded into LDS once and scored against eight queries, one per wave, each wave
// keeping its own candidates (same scores, same candidate layout).
// Kernel 2 (index_merge): one workgroup per query selects the k best keys among all candidates.
// A tile whose smallest kept key beats the k-th best may hide further winners; such tiles are
// re-scored in the merge workgroup (exact, slow, rare).
#include "common.h"
#include "internal.h"

namespace csa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxCand = 8192;        // candidates per query seen by the merge kernel
constexpr int kMergeThreads = 512;
constexpr int kMaxTile = 2048;
constexpr int kMaxK = 2048;
// groups of 16 entries per wave per load batch: 4 KB of keys in flight per wave and batch
template <int FMT>
constexpr int batch_of() { return FMT == 1 ? 2 : 4; }

// Cross-lane moves use DPP (a VALU operand modifier: no LDS round trip) inside rows of 16 lanes and
// v_readlane for the four row results, so a scan or reduction is a short VALU chain.
constexpr int kDppRowShr = 0x110;            // row_shr:n = kDppRowShr + n
constexpr int kDppQuadXor1 = 0xb1;           // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;           // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {   // lanes without a source read 0
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = uint32_t(dpp<CTRL>(int(uint32_t(v)))), hi = uint32_t(dpp<CTRL>(int(uint32_t(v >> 32))));
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), l));
  return (uint64_t(hi) << 32) | lo;
}

// Sum over lanes l, l^16, l^32 and l^48, in every lane (gfx950 half-wave and row swaps).
__device__ __forceinline__ float lane_group_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

struct alignas(16) QueryLds {         // quantised query of one indexer query token
  uint8_t codes[64 * 128];            // fp8: [head][128]; MXFP4: [head][64] packed
  uint8_t sbytes[64 * 4];             // MXFP4 block scales [head][4]
  float f[64];                        // per-head factor: w_h * fp8 scale (w_h for MXFP4); 0 if absent
};

// Raw bf16 values of one indexer query for thread t: head t/4 (clamped to the last head), values
// 32*(t%4) .. +31, and that head's weight.  Every thread loads (threads >= 256 repeat threads
// t - 256), so the number of loads in flight is the same in every wave.
struct QueryRaw {
  uint32_t wv[16];
  float w;
};
__device__ __forceinline__ void load_query_raw(const uint16_t *q, const float *w, int H_I, QueryRaw &raw,
                                               int t = int(threadIdx.x & 255)) {
  const int h = min(t >> 2, H_I - 1), c = t & 3;
  const uint4 *src = reinterpret_cast<const uint4 *>(q + h * 128 + c * 32);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint4 v = src[k];
    raw.wv[4 * k] = v.x; raw.wv[4 * k + 1] = v.y; raw.wv[4 * k + 2] = v.z; raw.wv[4 * k + 3] = v.w;
  }
  raw.w = w[h];
}

// Quantise one query's [H_I x 128] bf16 heads into LDS.  Thread t < 256 owns head t/4, values
// 32*(t%4) .. +31; heads >= H_I are written as zeros (factor 0) so 4 head blocks are always valid.
// Slot t (< 256) of the quantised query: head t/4, values 32*(t%4) .. +31; the 4 slots of a head
// are 4 consecutive lanes (the head's maximum is reduced over them).
template <int FMT>
__device__ __forceinline__ void prep_query_slot(const QueryRaw &raw, int t, int H_I, QueryLds &ql) {
  {
    const bool act = t < 4 * H_I;
    const int h = t >> 2, c = t & 3;
    uint32_t wv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) wv[k] = act ? raw.wv[k] : 0u;
    const float wh = raw.w;
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(wv[k])), fabsf(bf16hi(wv[k]))));
    if (FMT == 1) {
      amax = fmaxf(amax, __int_as_float(dpp<kDppQuadXor1>(__float_as_int(amax))));
      amax = fmaxf(amax, __int_as_float(dpp<kDppQuadXor2>(__float_as_int(amax))));
      const int e = e4m3_row_exp(amax);
      const float inv = ldexpf(1.0f, -e);
      uint32_t outw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t b0 = f32_to_e4m3(bf16lo(wv[2 * k]) * inv), b1 = f32_to_e4m3(bf16hi(wv[2 * k]) * inv);
        uint32_t b2 = f32_to_e4m3(bf16lo(wv[2 * k + 1]) * inv), b3 = f32_to_e4m3(bf16hi(wv[2 * k + 1]) * inv);
        outw[k] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
      }
      uint4 *dst = reinterpret_cast<uint4 *>(ql.codes + h * 128 + c * 32);
      dst[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
      dst[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
      if (c == 0) ql.f[h] = act ? wh * ldexpf(1.0f, e) : 0.f;
    } else {
      const uint32_t sb = mx_scale_byte(amax);
      const float inv = ldexpf(1.0f, 127 - int(sb));
      uint32_t outw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t p = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t lo = f32_to_e2m1(bf16lo(wv[4 * k + j]) * inv), hi = f32_to_e2m1(bf16hi(wv[4 * k + j]) * inv);
          p |= (lo | (hi << 4)) << (8 * j);
        }
        outw[k] = p;
      }
      *reinterpret_cast<uint4 *>(ql.codes + h * 64 + c * 16) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
      ql.sbytes[h * 4 + c] = uint8_t(sb);
      if (c == 0) ql.f[h] = act ? wh : 0.f;
    }
  }
}

template <int FMT>
__device__ void prep_query_lds(const QueryRaw &raw, int H_I, QueryLds &ql) {
  if (threadIdx.x < 256) prep_query_slot<FMT>(raw, int(threadIdx.x), H_I, ql);
}

// Per-lane MFMA operands of the quantised query (NHB head blocks of 16).
template <int NHB>
struct QueryFrag {
  v8i a[NHB];
  int sa[NHB];
  float f[NHB][4];
};

template <int FMT, int NHB>
__device__ __forceinline__ void load_query_frag(const QueryLds &ql, int lane, QueryFrag<NHB> &qf) {
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int head = hb * 16 + r;
    if (FMT == 1) {
      const uint4 *p = reinterpret_cast<const uint4 *>(ql.codes + head * 128 + g * 32);
      uint4 x0 = p[0], x1 = p[1];
      qf.a[hb] = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      qf.sa[hb] = 127;
    } else {
      uint4 x0 = *reinterpret_cast<const uint4 *>(ql.codes + head * 64 + g * 16);
      qf.a[hb] = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), 0, 0, 0, 0};
      qf.sa[hb] = ql.sbytes[head * 4 + g];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) qf.f[hb][v] = ql.f[hb * 16 + g * 4 + v];
  }
}

// Key operand of one lane for a group of 16 entries: entry (lane & 15), K-chunk (lane >> 4).
// Held exactly as loaded (no arithmetic on the loaded values until they are used, so issuing a
// batch never waits for it).
template <int FMT>
struct KeyFrag {
  uint4 c0, c1;     // codes (c1 unused for MXFP4)
  uint32_t s;       // fp8: the row scale's bits; MXFP4: the row's four e8m0 scale bytes
};

// The key rows of one tile, read through buffer resources.  The whole byte offset goes in the
// per-lane offset operand, which the hardware range check always covers: rows past the tile's last
// valid row, and whole groups past the tile, read as zeros without touching memory (their scores are
// discarded), so loads are issued unconditionally and nothing is clamped.
constexpr int kRawBufferWord3 = 0x00020000;   // gfx9 raw-buffer descriptor word 3 (32-bit data format)

template <int FMT>
struct TileKeys {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t code_off, scale_off;   // this lane's byte offsets inside a group
};

template <int FMT>
__device__ __forceinline__ TileKeys<FMT> make_tile_keys(const void *codes, const void *scales, int64_t row0,
                                                        int rows, int lane) {
  constexpr int RB = FMT == 1 ? 128 : 64;     // code bytes per row
  TileKeys<FMT> tk;
  tk.codes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(static_cast<const uint8_t *>(codes) + row0 * RB), short(0), rows * RB, kRawBufferWord3);
  tk.scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(static_cast<const uint8_t *>(scales) + row0 * 4), short(0), rows * 4, kRawBufferWord3);
  tk.code_off = uint32_t((lane & 15) * RB + (lane >> 4) * (FMT == 1 ? 32 : 16));
  tk.scale_off = uint32_t((lane & 15) * 4);
  return tk;
}

template <int FMT>
__device__ __forceinline__ void load_key_frag(const TileKeys<FMT> &tk, int grp, int lane, KeyFrag<FMT> &kf) {
  constexpr int RB = FMT == 1 ? 128 : 64;
  const uint32_t goff = uint32_t(grp) * (16 * RB);
  kf.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(tk.codes, tk.code_off + goff, 0, 0));
  if (FMT == 1)
    kf.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(tk.codes, tk.code_off + goff + 16, 0, 0));
  kf.s = __builtin_amdgcn_raw_buffer_load_b32(tk.scales, tk.scale_off + uint32_t(grp) * 64, 0, 0);
}

template <int FMT>
__device__ __forceinline__ void load_batch(const TileKeys<FMT> &tk, int g0, int lane, KeyFrag<FMT> (&kf)[batch_of<FMT>()]) {
#pragma unroll
  for (int u = 0; u < batch_of<FMT>(); ++u) load_key_frag<FMT>(tk, g0 + u, lane, kf[u]);
}

// max(x, 0) for a float: non-negative floats order like their bit patterns as signed integers, and
// every negative float (and -0) is a negative integer.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Scores of one group of 16 entries: the NHB MFMAs of the group (query head blocks x the group's
// keys), then the per-head ReLU/weight epilogue.  Each entry's score is reduced across its 4 lanes
// and written to s_scores by lanes 0..15; entries at tile-local index >= vis get -inf.
template <int FMT, int NHB>
__device__ __forceinline__ void group_mfma(const QueryFrag<NHB> &qf, const KeyFrag<FMT> &kf, int lane, v4f (&c)[NHB]) {
  constexpr int fmt = FMT == 1 ? 0 : 4;   // instruction format code: 0 = fp8 e4m3, 4 = fp4 e2m1
  const uint4 x0 = kf.c0, x1 = FMT == 1 ? kf.c1 : make_uint4(0, 0, 0, 0);
  const v8i bop = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
  const int sb = FMT == 1 ? 127 : int((kf.s >> (8 * (lane >> 4))) & 0xff);
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
    c[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf.a[hb], bop, v4f{0.f, 0.f, 0.f, 0.f}, fmt, fmt, 0,
                                                             qf.sa[hb], 0, sb);
}

template <int FMT, int NHB>
__device__ __forceinline__ void group_epilogue(const QueryFrag<NHB> &qf, const v4f (&c)[NHB], uint32_t s, int grp,
                                               int ngroups, int vis, int lane, float *s_scores) {
  float acc = 0.f;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc = fmaf(qf.f[hb][v], relu(c[hb][v]), acc);
  acc = lane_group_sum(acc);
  const int el = grp * 16 + (lane & 15);
  const float ks = FMT == 1 ? __uint_as_float(s) : 1.0f;
  if (lane < 16 && grp < ngroups) s_scores[el] = el < vis ? acc * ks : -INFINITY;
}

// Scores of one batch of groups, software-pipelined by one group: the MFMAs of group u + 1 are
// issued before the epilogue of group u, so an epilogue does not wait on MFMA latency and only two
// groups' results are live at a time.
template <int FMT, int NHB>
__device__ __forceinline__ void score_batch(const QueryFrag<NHB> &qf, const KeyFrag<FMT> (&kf)[batch_of<FMT>()], int g0,
                                            int ngroups, int vis, int lane, float *s_scores) {
  v4f c[2][NHB];
  group_mfma<FMT, NHB>(qf, kf[0], lane, c[0]);
#pragma unroll
  for (int u = 0; u < batch_of<FMT>(); ++u) {
    if (u + 1 < batch_of<FMT>()) group_mfma<FMT, NHB>(qf, kf[u + 1], lane, c[(u + 1) & 1]);
    group_epilogue<FMT, NHB>(qf, c[u & 1], kf[u].s, g0 + u, ngroups, vis, lane, s_scores);
  }
}

// Score the `tile` entries of a tile into s_scores (LDS); entries at tile-local index >= vis are
// written as -inf.  The block's waves split the groups; each wave alternates two load batches so the
// next batch is in flight while the current one is scored.  `ka` holds the wave's first batch,
// issued by the caller.
template <int FMT, int NHB>
__device__ void score_tile_mfma(const QueryFrag<NHB> &qf, KeyFrag<FMT> (&ka)[batch_of<FMT>()],
                                KeyFrag<FMT> (&kb)[batch_of<FMT>()], const TileKeys<FMT> &tk, int tile, int vis,
                                float *s_scores) {
  // the wave index is uniform: say so, so group offsets stay scalar (no per-lane loop over them)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int ngroups = tile >> 4;
  const int stride = nwaves * batch_of<FMT>();
  // On entry ka holds groups from wave * batch and kb the batch one stride later (both in flight).
  // Each batch is scored while the other one's loads are in flight; loads are unconditional, so
  // the count of loads in flight is the same on every path and each wait covers only the batch
  // about to be scored.
  for (int g0 = wave * batch_of<FMT>(); g0 < ngroups; g0 += 2 * stride) {
    score_batch<FMT, NHB>(qf, ka, g0, ngroups, vis, lane, s_scores);
    load_batch<FMT>(tk, g0 + 2 * stride, lane, ka);
    if (g0 + stride < ngroups) score_batch<FMT, NHB>(qf, kb, g0 + stride, ngroups, vis, lane, s_scores);
    load_batch<FMT>(tk, g0 + 3 * stride, lane, kb);
  }
}

// fp32 keys: one thread per entry, query heads from LDS.
__device__ void score_tile_f32(const float *q_lds, const float *w, int H_I, int D_I, const float *keys,
                               int64_t row0, int tile, int vis, float *s_scores) {
  for (int i = threadIdx.x; i < tile; i += blockDim.x) {
    float s = -INFINITY;
    if (i < vis) {
      const float4 *kr = reinterpret_cast<const float4 *>(keys + (row0 + i) * D_I);
      s = 0.f;
      for (int h = 0; h < H_I; ++h) {
        const float4 *qh = reinterpret_cast<const float4 *>(q_lds + h * D_I);
        float dot = 0.f;
        for (int k = 0; k < D_I / 4; ++k) {
          float4 a = qh[k], b = kr[k];
          dot += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
        }
        s += w[h] * fmaxf(dot, 0.f);
      }
    }
    s_scores[i] = s;
  }
}

// ---- wave and block helpers ------------------------------------------------------------------
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Inclusive prefix sum over the wave's 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += dpp<kDppRowShr + 1>(v);
  v += dpp<kDppRowShr + 2>(v);
  v += dpp<kDppRowShr + 4>(v);
  v += dpp<kDppRowShr + 8>(v);
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2);
}

// Wave-uniform minimum / maximum of a u64 over the 64 lanes.
template <bool MIN>
__device__ __forceinline__ uint64_t wave_minmax_u64(uint64_t v) {
  auto pick = [](uint64_t a, uint64_t b) { return MIN ? umin64(a, b) : umax64(a, b); };
  v = pick(v, dpp64<kDppQuadXor1>(v));
  v = pick(v, dpp64<kDppQuadXor2>(v));
  v = pick(v, dpp64<kDppRowHalfMirror>(v));
  v = pick(v, dpp64<kDppRowMirror>(v));
  return pick(pick(readlane64(v, 0), readlane64(v, 16)), pick(readlane64(v, 32), readlane64(v, 48)));
}

// Exclusive prefix over the block of one int per thread; returns (prefix, total).
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *s_tmp, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = NT / 64;
  int incl = wave_incl_scan(v, lane);
  if (lane == 63) s_tmp[wave] = incl;
  lds_barrier();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int x = s_tmp[w];
    base += (w < wave) ? x : 0;
    tot += x;
  }
  lds_barrier();
  total = tot;
  return base + incl - v;
}

struct alignas(16) SelectLds {
  uint32_t hist[3][256];
  uint64_t u64[16];
};

// Threshold over the non-zero keys held by the block (KPT per thread; keys are distinct; the
// caller guarantees 1 <= need <= number of non-zero keys).  Returns E such that the keys >= E are
// the largest ones and number
//   exactly `need` (E is then the need-th largest key itself), or
//   between keep_min and need - 1 (E is then a bin edge), when keep_min < need and a histogram
//   pass already separates at least keep_min of the largest keys from the rest.
// MSB-first radix select that starts at the highest bit where the keys differ (the bits above it
// are shared by every key, so histogramming them would pile every key into one bin) and resolves
// up to 8 bits per pass.  Every wave scans the histogram itself and the histograms rotate over
// three buffers (pass p zeroes the buffer of pass p+2, whose last readers finished before pass p's
// barrier), so a pass costs one barrier.
template <int NT, int KPT>
__device__ uint64_t block_cut(const uint64_t (&keys)[KPT], int need, int keep_min, SelectLds &sl) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < 768; i += NT) (&sl.hist[0][0])[i] = 0;
  uint64_t mn = ~uint64_t(0), mx = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k)
    if (keys[k] != 0) { mn = umin64(mn, keys[k]); mx = umax64(mx, keys[k]); }
  mn = wave_minmax_u64<true>(mn);
  mx = wave_minmax_u64<false>(mx);
  if (lane == 0) { sl.u64[wave] = mn; sl.u64[8 + wave] = mx; }
  lds_barrier();
  mn = ~uint64_t(0); mx = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { mn = umin64(mn, sl.u64[w]); mx = umax64(mx, sl.u64[8 + w]); }
  if (mn == mx) { lds_barrier(); return mn; }
  int hi = 63 - __clzll(mn ^ mx);                 // highest bit where keys differ
  uint64_t mask = hi == 63 ? 0 : ~((uint64_t(2) << hi) - 1);
  uint64_t prefix = mn & mask;
  int got = 0;                                    // keys already known to lie above the prefix
  for (int pass = 0;; ++pass) {
    uint32_t *H = sl.hist[pass % 3];
    const int width = hi + 1 < 8 ? hi + 1 : 8;
    const int shift = hi - width + 1;
    const uint64_t dmask = (uint64_t(1) << width) - 1;
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if (keys[k] != 0 && (keys[k] & mask) == prefix) atomicAdd(&H[(keys[k] >> shift) & dmask], 1u);
    lds_barrier();
    // every wave finds the digit holding rank `need`, scanning bins from the top
    const uint4 c4 = *reinterpret_cast<const uint4 *>(&H[252 - 4 * lane]);
    const int c[4] = {int(c4.w), int(c4.z), int(c4.y), int(c4.x)};   // bins 255-4l .. 252-4l
    const int sum = c[0] + c[1] + c[2] + c[3];
    int cum = wave_incl_scan(sum, lane) - sum;
    int hit = 0, d_sel = 0, above = 0, bucket = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!hit && cum < need && need <= cum + c[j]) { hit = 1; d_sel = 255 - 4 * lane - j; above = cum; bucket = c[j]; }
      cum += c[j];
    }
    const int src = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)__ballot(hit)) - 1);
    d_sel = __builtin_amdgcn_readlane(d_sel, src);
    above = __builtin_amdgcn_readlane(above, src);
    bucket = __builtin_amdgcn_readlane(bucket, src);
    // pass p-1's buffer (= pass p+2's) was last read before this pass's barrier: clear it
    uint32_t *Hn = sl.hist[(pass + 2) % 3];
    for (int i = tid; i < 256; i += NT) Hn[i] = 0;
    if (bucket != need - above && got + above >= keep_min) {
      // enough keys lie in the bins above d_sel: cut at that bin's upper edge
      lds_barrier();
      return (prefix | (uint64_t(d_sel) << shift)) + (uint64_t(1) << shift);
    }
    got += above;
    need -= above;
    prefix |= uint64_t(d_sel) << shift;
    mask |= dmask << shift;
    if (bucket == need || shift == 0) {
      // every key of this bucket is in; the answer is the smallest of them
      uint64_t m2 = ~uint64_t(0);
#pragma unroll
      for (int k = 0; k < KPT; ++k)
        if (keys[k] != 0 && (keys[k] & mask) == prefix) m2 = umin64(m2, keys[k]);
      m2 = wave_minmax_u64<true>(m2);
      if (lane == 0) sl.u64[wave] = m2;
      lds_barrier();
      uint64_t res = ~uint64_t(0);
#pragma unroll
      for (int w = 0; w < NW; ++w) res = umin64(res, sl.u64[w]);
      lds_barrier();
      return res;
    }
    hi = shift - 1;
  }
}

// Exact rank-`need` (1 = largest) key among the block's non-zero keys.
template <int NT, int KPT>
__device__ __forceinline__ uint64_t block_select(const uint64_t (&keys)[KPT], int need, SelectLds &sl) {
  return block_cut<NT, KPT>(keys, need, need, sl);
}

// ---- kernel 1: scores and per-tile candidates ------------------------------------------------
struct alignas(16) ScoreShared {
  QueryLds ql;
  float scores[kMaxTile];
  SelectLds sel;
  int tmp[16];
};

template <int FMT, int NHB, int NT, int KPT>
__global__ void __launch_bounds__(NT) index_score_kernel(IndexArgs a) {
  __shared__ ScoreShared sh;
  const int tile_id = blockIdx.x;
  const int64_t qi = blockIdx.y;                               // query = b * Sq + s
  const int b = int(blockIdx.y / uint32_t(a.Sq)), s = int(blockIdx.y) - b * a.Sq;
  const int tile = a.plan.tile, cand = a.plan.cand;
  const int64_t e_begin = int64_t(tile_id) * tile;
  const int64_t out_slot = qi * a.plan.n_tiles + tile_id;
  const int64_t n_q = int64_t(a.B) * a.Sq;
  uint64_t *cand_keys = static_cast<uint64_t *>(a.workspace);
  uint64_t *cand_bound = cand_keys + n_q * a.plan.n_tiles * cand;
  int *cand_count = reinterpret_cast<int *>(cand_bound + n_q * a.plan.n_tiles);
  const int64_t row0 = int64_t(b) * a.N_cap + e_begin;
  // The quantised-key loads are range-checked by their buffer resources, so they are issued
  // before the visible count (which waits on two scalar loads and a division) is known.
  QueryRaw raw;
  KeyFrag<FMT> ka[batch_of<FMT>()], kb[batch_of<FMT>()];
  TileKeys<FMT> tk;
  if (FMT != 0) {
    // the query's loads go first (loads complete in issue order), then two batches of keys,
    // which stream while the query is quantised
    load_query_raw(static_cast<const uint16_t *>(a.q_idx) + qi * a.H_I * 128, a.w_idx + qi * a.H_I, a.H_I, raw);
    __builtin_amdgcn_sched_barrier(0);                       // keep the query loads first
    const int rows = int(min(int64_t(tile), a.N_cap - e_begin));
    tk = make_tile_keys<FMT>(a.k_codes, a.k_scales, row0, rows, threadIdx.x & 63);
    const int g_first = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * batch_of<FMT>();
    load_batch<FMT>(tk, g_first, threadIdx.x & 63, ka);
    load_batch<FMT>(tk, g_first + (NT / 64) * batch_of<FMT>(), threadIdx.x & 63, kb);
  }
  const int64_t t = a.q_pos0[b] + s;
  const int64_t n_vis = min(a.n_entries[b], div_count(t + 1, a.m));
  const int vis = int(max(int64_t(0), min(int64_t(tile), n_vis - e_begin)));

  if (vis == 0 && a.scores == nullptr) {                      // nothing visible in this tile
    if (threadIdx.x == 0) { cand_count[out_slot] = 0; cand_bound[out_slot] = 0; }
    return;
  }
  if (FMT == 0) {
    float *q_lds = reinterpret_cast<float *>(sh.ql.codes);    // H_I * D_I <= 2048 floats
    const float *qsrc = static_cast<const float *>(a.q_idx) + qi * a.H_I * a.D_I;
    for (int i = threadIdx.x; i < a.H_I * a.D_I; i += NT) q_lds[i] = qsrc[i];
    if (threadIdx.x < a.H_I) sh.ql.f[threadIdx.x] = a.w_idx[qi * a.H_I + threadIdx.x];
    lds_barrier();
    score_tile_f32(q_lds, sh.ql.f, a.H_I, a.D_I, static_cast<const float *>(a.k_codes), row0, tile, vis,
                   sh.scores);
  } else {
    prep_query_lds<FMT>(raw, a.H_I, sh.ql);
    lds_barrier();
    QueryFrag<NHB> qf;
    load_query_frag<FMT, NHB>(sh.ql, threadIdx.x & 63, qf);
    score_tile_mfma<FMT, NHB>(qf, ka, kb, tk, tile, vis, sh.scores);
  }
  lds_barrier();
  if (a.scores) {
    float *dst = a.scores + qi * a.N_cap;
    for (int i = threadIdx.x; i < tile; i += NT)
      if (e_begin + i < a.N_cap) dst[e_begin + i] = sh.scores[i];
  }
  // keys of this thread's KPT consecutive entries
  uint64_t keys[KPT];
  int nvalid_local = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = threadIdx.x * KPT + k;
    const bool ok = i < vis;
    keys[k] = ok ? make_key(sh.scores[i], uint32_t(e_begin + i)) : 0;
    nvalid_local += ok;
  }
  uint64_t bound = 0;
  // keep the tile's largest keys: all `cand` of them, or at least half as many when one histogram
  // pass already separates them (the merge checks every truncated tile's bound against its
  // threshold and rescans the tile when the bound is not below it)
  if (vis > cand) bound = block_cut<NT, KPT>(keys, cand, cand / 2, sh.sel);
  int mine = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) mine += (keys[k] != 0 && keys[k] >= bound);
  int total;
  int pos = block_excl_scan<NT>(mine, sh.tmp, total);
  uint64_t *dst = cand_keys + out_slot * cand;
#pragma unroll
  for (int k = 0; k < KPT; ++k)
    if (keys[k] != 0 && keys[k] >= bound) dst[pos++] = keys[k];
  if (threadIdx.x == 0) { cand_count[out_slot] = total; cand_bound[out_slot] = bound; }
  (void)nvalid_local;
}

// ---- kernel 1b (prefill): one key tile, eight queries of one sequence ------------------------
// For calls with many queries per sequence (a prefill chunk) the same keys are scored against
// consecutive queries.  Workgroup = (tile of 512 entries, 8 consecutive queries, sequence): the
// tile's quantised keys are loaded into LDS once and every wave scores them against its own query
// (quantised straight into MFMA operands, no LDS), then selects its candidates with a wave-local
// radix select -- no workgroup barrier after the tile is loaded.  Scores are bit-identical to
// index_score_kernel's (the same MFMA operands and epilogue order), so the selection is too.
constexpr int kMultiQ = 8;              // queries per workgroup, one per wave
constexpr int kMultiTile = 512;         // entries per tile

// Keep the wave's largest keys (8 per lane, distinct, 0 = absent): the same cut as block_cut --
// exactly `need` keys, or between keep_min and need - 1 when one histogram pass separates them --
// on one wave, with the wave's own 256-bin histogram in LDS and no workgroup barrier (a wave's
// LDS accesses complete in order; the fences keep the compiler from reordering them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ uint64_t wave_cut(const uint64_t (&keys)[8], int need, int keep_min, uint32_t *H) {
  const int lane = threadIdx.x & 63;
  uint64_t mn = ~uint64_t(0), mx = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (keys[k] != 0) { mn = umin64(mn, keys[k]); mx = umax64(mx, keys[k]); }
  mn = wave_minmax_u64<true>(mn);
  mx = wave_minmax_u64<false>(mx);
  if (mn == mx) return mn;
  int hi = 63 - __clzll(mn ^ mx);
  uint64_t mask = hi == 63 ? 0 : ~((uint64_t(2) << hi) - 1);
  uint64_t prefix = mn & mask;
  int got = 0;
  *reinterpret_cast<uint4 *>(&H[4 * lane]) = make_uint4(0, 0, 0, 0);
  wave_lds_sync();
  for (;;) {
    const int width = hi + 1 < 8 ? hi + 1 : 8;
    const int shift = hi - width + 1;
    const uint64_t dmask = (uint64_t(1) << width) - 1;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (keys[k] != 0 && (keys[k] & mask) == prefix) atomicAdd(&H[(keys[k] >> shift) & dmask], 1u);
    wave_lds_sync();
    const uint4 c4 = *reinterpret_cast<const uint4 *>(&H[252 - 4 * lane]);
    const int c[4] = {int(c4.w), int(c4.z), int(c4.y), int(c4.x)};   // bins 255-4l .. 252-4l
    const int sum = c[0] + c[1] + c[2] + c[3];
    int cum = wave_incl_scan(sum, lane) - sum;
    int hit = 0, d_sel = 0, above = 0, bucket = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!hit && cum < need && need <= cum + c[j]) { hit = 1; d_sel = 255 - 4 * lane - j; above = cum; bucket = c[j]; }
      cum += c[j];
    }
    const int src = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)__ballot(hit)) - 1);
    d_sel = __builtin_amdgcn_readlane(d_sel, src);
    above = __builtin_amdgcn_readlane(above, src);
    bucket = __builtin_amdgcn_readlane(bucket, src);
    *reinterpret_cast<uint4 *>(&H[252 - 4 * lane]) = make_uint4(0, 0, 0, 0);   // for the next pass
    wave_lds_sync();
    if (bucket != need - above && got + above >= keep_min)
      return (prefix | (uint64_t(d_sel) << shift)) + (uint64_t(1) << shift);
    got += above;
    need -= above;
    prefix |= uint64_t(d_sel) << shift;
    mask |= dmask << shift;
    if (bucket == need || shift == 0) {
      uint64_t m2 = ~uint64_t(0);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (keys[k] != 0 && (keys[k] & mask) == prefix) m2 = umin64(m2, keys[k]);
      return wave_minmax_u64<true>(m2);
    }
    hi = shift - 1;
  }
}

struct alignas(16) MultiShared {
  union {
    struct {
      uint8_t codes[kMultiTile * 128];    // fp8 [entry][128]; MXFP4 [entry][64]
      uint32_t scales[kMultiTile];        // fp8: row scale bits; MXFP4: the row's four e8m0 bytes
    } tile;
    QueryLds q[kMultiQ];                  // before the tile arrives: each wave's quantised query
  };
  uint32_t hist[kMultiQ][256];            // each wave's select histogram
};

// Workspace of the shared-tile path: after the candidate slots, bounds and counts (as in the
// one-query path), every query's quantised query (a QueryLds image), 16-byte aligned.
__host__ __device__ inline size_t prepared_query_offset(int64_t n_q, const IndexPlan &p) {
  const int64_t slots = n_q * p.n_tiles;
  const size_t off = size_t(slots * p.cand * 8 + slots * 8 + slots * 4);
  return (off + 255) / 256 * 256;
}

// Shared-tile path, step 0: every query quantised once (the same encoders, so the same bytes, as
// the one-query kernel's) into the workspace; the tile workgroups then copy it instead of
// re-quantising the query for each of their tiles.
template <int FMT>
__global__ void __launch_bounds__(256) index_query_prep_kernel(IndexArgs a) {
  __shared__ QueryLds ql;
  const int64_t qi = blockIdx.x;
  const int t = threadIdx.x;
  QueryRaw raw;
  load_query_raw(static_cast<const uint16_t *>(a.q_idx) + qi * a.H_I * 128, a.w_idx + qi * a.H_I, a.H_I, raw, t);
  prep_query_slot<FMT>(raw, t, a.H_I, ql);
  lds_barrier();
  constexpr int W = int(sizeof(QueryLds) / 16);
  const int64_t n_q = int64_t(a.B) * a.Sq;
  uint4 *dst = reinterpret_cast<uint4 *>(static_cast<uint8_t *>(a.workspace) + prepared_query_offset(n_q, a.plan)) +
               qi * W;
  const uint4 *src = reinterpret_cast<const uint4 *>(&ql);
  for (int i = t; i < W; i += 256) dst[i] = src[i];
}

template <int FMT, int NHB>
__global__ void __launch_bounds__(64 * kMultiQ, 2) index_score_multi_kernel(IndexArgs a) {
  __shared__ MultiShared sh;
  constexpr int NT = 64 * kMultiQ;
  constexpr int RB = FMT == 1 ? 128 : 64;                      // code bytes per entry
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile_id = blockIdx.x, b = blockIdx.z;
  const int s0 = blockIdx.y * kMultiQ;
  const int tile = a.plan.tile, cand = a.plan.cand;
  const int64_t e_begin = int64_t(tile_id) * tile;
  const int64_t row0 = int64_t(b) * a.N_cap + e_begin;
  const int rows = int(min(int64_t(tile), a.N_cap - e_begin));
  // the tile's keys, through range-checked buffer loads (rows past N_cap read zeros), go to
  // registers first; the LDS they land in holds the waves' quantised queries until then
  constexpr int LPT = kMultiTile * RB / 16 / NT;               // 16-byte loads per thread
  uint4 v[LPT];
  uint32_t sc;
  {
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(static_cast<const uint8_t *>(a.k_codes) + row0 * RB), short(0), rows * RB, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(static_cast<const uint8_t *>(a.k_scales) + row0 * 4), short(0), rows * 4, kRawBufferWord3);
#pragma unroll
    for (int l = 0; l < LPT; ++l)
      v[l] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, uint32_t((l * NT + tid) * 16), 0, 0));
    sc = __builtin_amdgcn_raw_buffer_load_b32(rs, uint32_t(tid * 4), 0, 0);
  }
  // this wave's query, already quantised by index_query_prep_kernel, copied into its LDS slot,
  // then read back as MFMA operands
  const int s = s0 + wave;
  const bool live = s < a.Sq;
  const int64_t qi = int64_t(b) * a.Sq + (live ? s : a.Sq - 1);
  {
    constexpr int W = int(sizeof(QueryLds) / 16);
    const int64_t n_q = int64_t(a.B) * a.Sq;
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(a.workspace) +
                                                       prepared_query_offset(n_q, a.plan)) + qi * W;
    uint4 *dst = reinterpret_cast<uint4 *>(&sh.q[wave]);
    for (int i = lane; i < W; i += 64) dst[i] = src[i];
  }
  wave_lds_sync();
  QueryFrag<NHB> qf;
  load_query_frag<FMT, NHB>(sh.q[wave], lane, qf);
  const int64_t t = a.q_pos0[b] + s;
  const int64_t n_vis = min(a.n_entries[b], div_count(t + 1, a.m));
  const int vis = int(max(int64_t(0), min(int64_t(tile), n_vis - e_begin)));
  lds_barrier();                                                // every wave has its query
#pragma unroll
  for (int l = 0; l < LPT; ++l) *reinterpret_cast<uint4 *>(sh.tile.codes + (l * NT + tid) * 16) = v[l];
  sh.tile.scales[tid] = sc;
  lds_barrier();                                                // the tile is in LDS
  if (!live) return;
  const int64_t n_q = int64_t(a.B) * a.Sq;
  uint64_t *cand_keys = static_cast<uint64_t *>(a.workspace);
  uint64_t *cand_bound = cand_keys + n_q * a.plan.n_tiles * cand;
  int *cand_count = reinterpret_cast<int *>(cand_bound + n_q * a.plan.n_tiles);
  const int64_t out_slot = qi * a.plan.n_tiles + tile_id;
  // scores: group j (16 entries) lands in lanes 16 (j % 4) .. + 15, slot j / 4 -- entry 64 slot + lane
  const int g = lane >> 4, r = lane & 15;
  constexpr int fmt = FMT == 1 ? 0 : 4;                        // instruction format code
  uint64_t keys[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) keys[k] = 0;
  const int ngroups = (vis + 15) >> 4;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
#pragma unroll 1
   for (int jj = 0; jj < 4; ++jj) {
    const int j = 4 * k + jj;
    if (j < ngroups) {
      const int el = 16 * j + r;
      const uint8_t *cp = sh.tile.codes + el * RB + g * (FMT == 1 ? 32 : 16);
      const uint4 x0 = *reinterpret_cast<const uint4 *>(cp);
      const uint4 x1 = FMT == 1 ? *reinterpret_cast<const uint4 *>(cp + 16) : make_uint4(0, 0, 0, 0);
      const uint32_t ksc = sh.tile.scales[el];
      const v8i bop = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      const int sb = FMT == 1 ? 127 : int((ksc >> (8 * g)) & 0xff);
      v4f c[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        c[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf.a[hb], bop, v4f{0.f, 0.f, 0.f, 0.f}, fmt, fmt, 0,
                                                                 qf.sa[hb], 0, sb);
      float acc = 0.f;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc = fmaf(qf.f[hb][v], relu(c[hb][v]), acc);
      acc = lane_group_sum(acc);
      const float score = acc * (FMT == 1 ? __uint_as_float(ksc) : 1.0f);
      if (g == jj && el < vis) keys[k] = make_key(score, uint32_t(e_begin + el));
    }
   }
  }
  uint64_t bound = 0;
  if (vis > cand) bound = wave_cut(keys, cand, cand / 2, sh.hist[wave]);
  // kept keys in ascending entry order (slot-major: entry 64 slot + lane)
  uint64_t *dst = cand_keys + out_slot * cand;
  int base = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool keep = keys[k] != 0 && keys[k] >= bound;
    const uint64_t m = __ballot(keep);
    if (keep) dst[base + __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0))] = keys[k];
    base += __popcll(m);
  }
  if (lane == 0) { cand_count[out_slot] = base; cand_bound[out_slot] = bound; }
}

// ---- kernel 2: merge ----------------------------------------------------------------------
struct alignas(16) MergeShared {
  QueryLds ql;
  float scores[kMaxTile];
  uint64_t work[kMaxK + kMaxTile];
  int counts[kMaxCand / 8];
  uint64_t bounds[kMaxCand / 8];
  SelectLds sel;
  int tmp[16];
  int flag;
};

// Sort P (a power of two) entry indices ascending in LDS.
__device__ void bitonic_sort_u32(uint32_t *v, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint32_t x = v[i], y = v[ixj];
          bool up = (i & k) == 0;
          if ((x > y) == up) { v[i] = y; v[ixj] = x; }
        }
      }
      lds_barrier();
    }
  }
}

// Exact fallback: the candidate set may miss winners hidden in tiles whose kept keys all beat
// `tau`.  Keep a working set W (the k_eff best so far) in LDS and merge in every such tile,
// re-scored from its keys.  Writes the final selection in ascending index order.
template <int FMT, int KPT>
__device__ void merge_fallback(const IndexArgs &a, MergeShared &sh, const uint64_t (&keys)[KPT], uint64_t tau,
                               int64_t qi, int b, int64_t n_vis, int k_eff, int32_t *out) {
  constexpr int NT = kMergeThreads;
  const int tid = threadIdx.x;
  const int tile = a.plan.tile, n_tiles = a.plan.n_tiles;
  int wn;
  {
    int mine = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) mine += (keys[k] != 0 && keys[k] >= tau);
    int pos = block_excl_scan<NT>(mine, sh.tmp, wn);
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if (keys[k] != 0 && keys[k] >= tau) sh.work[pos++] = keys[k];
  }
  lds_barrier();
  QueryFrag<4> qf;
  float *q_lds = reinterpret_cast<float *>(sh.ql.codes);
  if (FMT == 0) {
    const float *qsrc = static_cast<const float *>(a.q_idx) + qi * a.H_I * a.D_I;
    for (int i = tid; i < a.H_I * a.D_I; i += NT) q_lds[i] = qsrc[i];
    if (tid < a.H_I) sh.ql.f[tid] = a.w_idx[qi * a.H_I + tid];
    lds_barrier();
  } else {
    QueryRaw raw;
    load_query_raw(static_cast<const uint16_t *>(a.q_idx) + qi * a.H_I * 128, a.w_idx + qi * a.H_I, a.H_I, raw);
    prep_query_lds<FMT>(raw, a.H_I, sh.ql);
    lds_barrier();
    load_query_frag<FMT, 4>(sh.ql, tid & 63, qf);
  }
  constexpr int KW = (kMaxK + kMaxTile) / NT;
  for (int tl = 0; tl < n_tiles; ++tl) {
    const uint64_t bt = sh.bounds[tl];
    if (bt == 0 || bt <= tau) continue;                        // complete, or cannot hold winners
    const int64_t e_begin = int64_t(tl) * tile;
    const int vis = int(max(int64_t(0), min(int64_t(tile), n_vis - e_begin)));
    const int64_t row0 = int64_t(b) * a.N_cap + e_begin;
    if (FMT == 0) {
      score_tile_f32(q_lds, sh.ql.f, a.H_I, a.D_I, static_cast<const float *>(a.k_codes), row0, tile, vis,
                     sh.scores);
    } else {
      const int rows = int(min(int64_t(tile), a.N_cap - e_begin));
      const TileKeys<FMT> tk = make_tile_keys<FMT>(a.k_codes, a.k_scales, row0, rows, tid & 63);
      KeyFrag<FMT> ka[batch_of<FMT>()], kb[batch_of<FMT>()];
      const int g_first = __builtin_amdgcn_readfirstlane(tid >> 6) * batch_of<FMT>();
      load_batch<FMT>(tk, g_first, tid & 63, ka);
      load_batch<FMT>(tk, g_first + (NT / 64) * batch_of<FMT>(), tid & 63, kb);
      score_tile_mfma<FMT, 4>(qf, ka, kb, tk, tile, vis, sh.scores);
    }
    lds_barrier();
    // append the tile's entries below its bound (the ones not already candidates) and above tau
    int mine = 0;
    for (int i = tid; i < vis; i += NT) {
      const uint64_t key = make_key(sh.scores[i], uint32_t(e_begin + i));
      mine += (key < bt && key > tau);
    }
    int total;
    int pos = block_excl_scan<NT>(mine, sh.tmp, total) + wn;
    for (int i = tid; i < vis; i += NT) {
      const uint64_t key = make_key(sh.scores[i], uint32_t(e_begin + i));
      if (key < bt && key > tau) sh.work[pos++] = key;
    }
    wn += total;
    lds_barrier();
    if (wn >= k_eff) {                                          // shrink W back to the k_eff best
      uint64_t wk[KW];
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const int i = tid * KW + k;
        wk[k] = i < wn ? sh.work[i] : 0;
      }
      lds_barrier();
      tau = block_select<NT, KW>(wk, k_eff, sh.sel);
      int m2 = 0;
#pragma unroll
      for (int k = 0; k < KW; ++k) m2 += (wk[k] != 0 && wk[k] >= tau);
      int tot2;
      int p2 = block_excl_scan<NT>(m2, sh.tmp, tot2);
#pragma unroll
      for (int k = 0; k < KW; ++k)
        if (wk[k] != 0 && wk[k] >= tau) sh.work[p2++] = wk[k];
      wn = tot2;
      lds_barrier();
    }
  }
  // ascending indices
  uint32_t *idx = reinterpret_cast<uint32_t *>(sh.work);
  int P = 1;
  while (P < wn) P <<= 1;
  uint32_t tmpv[KW];
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int i = tid * KW + k;
    tmpv[k] = i < wn ? key_index(sh.work[i]) : 0xffffffffu;
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int i = tid * KW + k;
    if (i < P) idx[i] = tmpv[k];
  }
  lds_barrier();
  bitonic_sort_u32(idx, P);
  for (int i = tid; i < a.topk; i += NT) out[i] = i < wn ? int32_t(idx[i]) : -1;
}

template <int FMT, int KPT>
__global__ void __launch_bounds__(kMergeThreads) index_merge_kernel(IndexArgs a) {
  __shared__ MergeShared sh;
  constexpr int NT = kMergeThreads;
  const int tid = threadIdx.x;
  const int64_t qi = blockIdx.x;
  const int b = int(blockIdx.x / uint32_t(a.Sq)), s = int(blockIdx.x) - b * a.Sq;
  const int cand = a.plan.cand, n_tiles = a.plan.n_tiles;
  const int64_t n_q = int64_t(a.B) * a.Sq;
  const uint64_t *cand_keys = static_cast<const uint64_t *>(a.workspace);
  const uint64_t *cand_bound = cand_keys + n_q * n_tiles * cand;
  const int *cand_count = reinterpret_cast<const int *>(cand_bound + n_q * n_tiles);
  int32_t *out = a.topk_idx + qi * a.topk;

  // candidate slots and per-tile counts are loaded together; slots past a tile's count are masked
  uint64_t keys[KPT];
  const int slots = n_tiles * cand;                            // a multiple of 8
  if constexpr (KPT % 2 == 0) {
    const uint4 *src = reinterpret_cast<const uint4 *>(cand_keys + qi * slots + tid * KPT);
#pragma unroll
    for (int k = 0; k < KPT; k += 2) {
      const uint4 v = tid * KPT + k < slots ? src[k / 2] : make_uint4(0, 0, 0, 0);
      keys[k] = (uint64_t(v.y) << 32) | v.x;
      keys[k + 1] = (uint64_t(v.w) << 32) | v.z;
    }
  } else {
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int slot = tid * KPT + k;
      keys[k] = slot < slots ? cand_keys[qi * slots + slot] : 0;
    }
  }
  // per-tile counts and bounds (n_tiles <= 2 NT), held in registers until the position is known
  static_assert(kMaxCand / 8 <= 2 * NT, "two tiles' counts per thread");
  // (loaded unconditionally from a clamped slot, so no branch separates the loads from the ones above)
  int cnt[2];
  uint64_t bnd[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = min(tid + j * NT, n_tiles - 1);
    cnt[j] = cand_count[qi * n_tiles + i];
    bnd[j] = cand_bound[qi * n_tiles + i];
  }
  // the query's position is read only now, while the candidate loads are in flight
  __builtin_amdgcn_sched_barrier(0);
  const int64_t t = a.q_pos0[b] + s;
  const int64_t n_vis = min(a.n_entries[b], div_count(t + 1, a.m));
  const int k_eff = int(min(int64_t(a.topk), n_vis));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + j * NT;
    if (i < n_tiles) { sh.counts[i] = cnt[j]; sh.bounds[i] = bnd[j]; }
  }
  if (tid == 0) sh.flag = 0;
  lds_barrier();
  int nvalid_local = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int slot = tid * KPT + k;
    const int tl = slot / cand, j = slot - tl * cand;
    if (slot >= slots || j >= sh.counts[tl]) keys[k] = 0;
    nvalid_local += keys[k] != 0;
  }
  int nvalid;
  (void)block_excl_scan<NT>(nvalid_local, sh.tmp, nvalid);
  if (k_eff == 0) {
    for (int i = tid; i < a.topk; i += NT) out[i] = -1;
    return;
  }
  uint64_t tau = 0;                                            // k-th best candidate (0: need all)
  if (nvalid >= k_eff) tau = block_select<NT, KPT>(keys, k_eff, sh.sel);
  // a truncated tile whose smallest kept key beats tau may hold further winners
  for (int i = tid; i < n_tiles; i += NT)
    if (sh.bounds[i] != 0 && sh.bounds[i] > tau) sh.flag = 1;
  lds_barrier();
  if (sh.flag) {
    merge_fallback<FMT, KPT>(a, sh, keys, tau, qi, b, n_vis, k_eff, out);
    return;
  }
  int mine = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) mine += (keys[k] != 0 && keys[k] >= tau);
  int total;
  int pos = block_excl_scan<NT>(mine, sh.tmp, total);
#pragma unroll
  for (int k = 0; k < KPT; ++k)
    if (keys[k] != 0 && keys[k] >= tau) out[pos++] = int32_t(key_index(keys[k]));
  for (int i = k_eff + tid; i < a.topk; i += NT) out[i] = -1;
}

template <int FMT, int NHB>
hipError_t launch_score_t(const IndexArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.plan.multi) {
    e = launch("index_query_prep", index_query_prep_kernel<FMT>, dim3(unsigned(int64_t(a.B) * a.Sq)), dim3(256),
               stream, a);
    if (e != hipSuccess) return e;
    const dim3 mgrid(unsigned(a.plan.n_tiles), unsigned((a.Sq + kMultiQ - 1) / kMultiQ), unsigned(a.B));
    return launch("index_score", index_score_multi_kernel<FMT, NHB>, mgrid, dim3(64 * kMultiQ), stream, a);
  }
  dim3 grid(unsigned(a.plan.n_tiles), unsigned(int64_t(a.B) * a.Sq));
  switch (a.plan.tile) {
    case 64: case 128: case 256:
      e = launch("index_score", index_score_kernel<FMT, NHB, 256, 1>, grid, dim3(256), stream, a); break;
    case 512: e = launch("index_score", index_score_kernel<FMT, NHB, 256, 2>, grid, dim3(256), stream, a); break;
    case 1024: e = launch("index_score", index_score_kernel<FMT, NHB, 512, 2>, grid, dim3(512), stream, a); break;
    case 2048: e = launch("index_score", index_score_kernel<FMT, NHB, 512, 4>, grid, dim3(512), stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return e;
}

template <int FMT>
hipError_t launch_merge_t(const IndexArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  dim3 grid(unsigned(int64_t(a.B) * a.Sq));
  const int slots = a.plan.n_tiles * a.plan.cand;
  if (slots <= 512)
    e = launch("index_merge", index_merge_kernel<FMT, 1>, grid, dim3(kMergeThreads), stream, a);
  else if (slots <= 1024)
    e = launch("index_merge", index_merge_kernel<FMT, 2>, grid, dim3(kMergeThreads), stream, a);
  else if (slots <= 2048)
    e = launch("index_merge", index_merge_kernel<FMT, 4>, grid, dim3(kMergeThreads), stream, a);
  else if (slots <= 4096)
    e = launch("index_merge", index_merge_kernel<FMT, 8>, grid, dim3(kMergeThreads), stream, a);
  else
    e = launch("index_merge", index_merge_kernel<FMT, 16>, grid, dim3(kMergeThreads), stream, a);
  return e;
}

}  // namespace

IndexPlan plan_index(int64_t B, int64_t Sq, int64_t N_cap, int topk, int format) {
  IndexPlan p;
  const int64_t n_queries = B * Sq;
  // many queries per sequence (a prefill chunk) with quantised keys: tiles of 512 shared by eight
  // queries (index_score_multi_kernel)
  p.multi = (format != 0 && Sq >= kMultiQ && N_cap > kMultiTile && N_cap <= int64_t(kMaxCand / 8) * kMultiTile) ? 1 : 0;
  int tile = kMaxTile;
  if (p.multi) tile = kMultiTile;
  while (!p.multi && tile > 64 && n_queries * ((N_cap + tile - 1) / tile) < 512) tile >>= 1;
  while (!p.multi && tile > 64 && tile / 2 >= N_cap) tile >>= 1;
  p.tile = tile;
  p.n_tiles = int((N_cap + tile - 1) / tile);
  // keep ~4x the expected number of winners per tile, within the merge kernel's capacity
  int64_t want = (4 * int64_t(topk) * tile + N_cap - 1) / N_cap;
  int cand = 8;
  while (cand < want && cand < tile) cand <<= 1;
  if (cand > tile) cand = tile;
  while (int64_t(p.n_tiles) * cand > kMaxCand && cand > 8) cand >>= 1;
  p.cand = cand;
  return p;
}

size_t index_workspace_bytes(int64_t B, int64_t Sq, int64_t N_cap, int topk, int format) {
  IndexPlan p = plan_index(B, Sq, N_cap, topk, format);
  const int64_t slots = B * Sq * p.n_tiles;
  if (p.multi) return prepared_query_offset(B * Sq, p) + size_t(B * Sq) * sizeof(QueryLds) + 256;
  return size_t(slots * p.cand * 8 + slots * 8 + slots * 4 + 256);
}

hipError_t launch_index_score(const IndexArgs &a, hipStream_t stream) {
  const int nhb = a.H_I / 16;
  if (a.format == 0) return launch_score_t<0, 1>(a, stream);
  if (a.format == 1) {
    switch (nhb) {
      case 1: return launch_score_t<1, 1>(a, stream);
      case 2: return launch_score_t<1, 2>(a, stream);
      case 3: return launch_score_t<1, 3>(a, stream);
      case 4: return launch_score_t<1, 4>(a, stream);
    }
  } else {
    switch (nhb) {
      case 1: return launch_score_t<2, 1>(a, stream);
      case 2: return launch_score_t<2, 2>(a, stream);
      case 3: return launch_score_t<2, 3>(a, stream);
      case 4: return launch_score_t<2, 4>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_index_merge(const IndexArgs &a, hipStream_t stream) {
  if (a.format == 0) return launch_merge_t<0>(a, stream);
  if (a.format == 1) return launch_merge_t<1>(a, stream);
  return launch_merge_t<2>(a, stream);
}

}  // namespace csa
