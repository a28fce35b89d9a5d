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
// With quantised keys every path first encodes the query's [H_I x 128] head matrix like the keys
// (prep_query_slot: fp8 e4m3 with a per-head scale, or MXFP4 with e8m0 block scales; the head
// weight and scale are folded into one factor per head) and holds it as MFMA A-operands.  A group
// of 16 entries then costs one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 heads, the block scales
// applied by the instruction.  fp32 keys are scored by plain fp32 dot products.
// Which kernels run is fixed by plan_index:
//
//   quantised keys, fewer than eight queries per sequence or the raw scores asked for (the
//   streaming path): index_stream_kernel, grid (segments, queries).
//     A segment of up to 4,096 entries per workgroup streams through a ring of LDS chunks filled by
//     direct-to-LDS buffer loads; its scores stay in LDS and its best keys are published as
//     candidates.  The last segment workgroup of a query to finish merges them into the query's
//     top-k (arrive_last; index_merge_kernel after it when the candidates exceed what one workgroup
//     holds).
//   quantised keys, eight or more queries per sequence (a prefill chunk, the shared-tile path):
//     index_query_prep_kernel encodes every query once into the workspace, index_score_multi_kernel
//     scores one 512-entry tile against eight queries (one per wave), index_merge_kernel merges.
//   fp32 keys: index_score_kernel, one tile of up to 2,048 entries per workgroup, with the merge in
//     each query's last tile workgroup.
//
// Keeping a segment's candidates: an estimate of the score distribution (per-wave mean and mean
// absolute deviation) places four trial thresholds at normal quantiles around the wanted count;
// one pass counts the entries above each, and the kept entries' output positions come from the
// same pass.  When no threshold lands in the accepted band the bucket select over the score keys'
// order bits decides instead.  The merge selects the exact k-th best key over all candidates; a
// segment whose smallest kept key beats it may hide further winners and is re-scored by the
// merging workgroup (exact, slow, rare).
//
// Workspace (bytes, from the start; n_q = queries, S = segments or tiles per query):
//   candidate keys  n_q * S * cand * 8   (score order bits << 32 | entry index, ascending index)
//   smallest kept   n_q * S * 8
//   counts          n_q * S * 4
//   then, 256-aligned, either the arrival counters (n_q * kCounterStride ints; every merge leaves
//   its counter at zero, so a zeroed workspace stays valid across calls) or, on the shared-tile
//   path, every query's encoded image (n_q * sizeof(QueryLds)).
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
constexpr int kFusedKeys = 8;                     // candidate slots per thread of a merging tile workgroup
constexpr int kFusedSlots = 512 * kFusedKeys;

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
// The e4m3 / e2m1 codes are produced by the gfx950 conversion instructions (v_cvt_pk_fp8_f32,
// v_cvt_scalef32_pk_fp4_f32 with unit scale) from values already divided by the power-of-two
// scale (an exact division).  In the range those scales produce (|x| <= 448 for e4m3, |x| < 8 for
// e2m1) their rounding -- nearest, ties to the even code, saturating -- is that of f32_to_e4m3 /
// f32_to_e2m1 (the encoders csa_quantize_keys uses) for every bf16 input, and the GPU tests hold
// the resulting codes to the oracle's bit for bit.
template <int FMT>
__device__ __forceinline__ void prep_query_slot(const QueryRaw &raw, int t, int H_I, QueryLds &ql) {
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
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf16lo(wv[2 * k]) * inv, bf16hi(wv[2 * k]) * inv, 0, false);
      outw[k] = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(bf16lo(wv[2 * k + 1]) * inv, bf16hi(wv[2 * k + 1]) * inv, lo,
                                                         true));
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
      p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, bf16lo(wv[4 * k]) * inv, bf16hi(wv[4 * k]) * inv, 1.0f, 0);
      p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, bf16lo(wv[4 * k + 1]) * inv, bf16hi(wv[4 * k + 1]) * inv, 1.0f, 1);
      p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, bf16lo(wv[4 * k + 2]) * inv, bf16hi(wv[4 * k + 2]) * inv, 1.0f, 2);
      p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, bf16lo(wv[4 * k + 3]) * inv, bf16hi(wv[4 * k + 3]) * inv, 1.0f, 3);
      outw[k] = p;
    }
    *reinterpret_cast<uint4 *>(ql.codes + h * 64 + c * 16) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    ql.sbytes[h * 4 + c] = uint8_t(sb);
    if (c == 0) ql.f[h] = act ? wh : 0.f;
  }
}

template <int FMT>
__device__ __forceinline__ void prep_query_lds(const QueryRaw &raw, int H_I, QueryLds &ql) {
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
      const_cast<uint8_t *>(static_cast<const uint8_t *>(codes) + row0 * RB), short(0), rows * RB, kRawBufferDesc3);
  tk.scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(static_cast<const uint8_t *>(scales) + row0 * 4), short(0), rows * 4, kRawBufferDesc3);
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


// max(x, 0) for a float: non-negative floats order like their bit patterns as signed integers, and
// every negative float (and -0) is a negative integer.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

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

// Scores of a tile for the merge's exact fallback, which runs after the scoring: the query's MFMA
// operands are read from LDS for every group and one group per wave is in flight, so it needs few
// registers.  Same MFMA operands and epilogue order (heads in order, then the four values of each)
// as the streaming kernel's scorer, hence the same scores bit for bit.
template <int FMT, int NHB>
__device__ __forceinline__ void score_tile_lean(const QueryLds &ql, const TileKeys<FMT> &tk, int tile, int vis, float *s_scores) {
  constexpr int fmt = FMT == 1 ? 0 : 4;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6, ngroups = tile >> 4;
  const int g = lane >> 4, r = lane & 15;
  for (int grp = wave; grp < ngroups; grp += nwaves) {
    KeyFrag<FMT> kf;
    load_key_frag<FMT>(tk, grp, lane, kf);
    const uint4 x0 = kf.c0, x1 = FMT == 1 ? kf.c1 : make_uint4(0, 0, 0, 0);
    const v8i bop = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
    const int sb = FMT == 1 ? 127 : int((kf.s >> (8 * g)) & 0xff);
    float acc = 0.f;
#pragma unroll 1
    for (int hb = 0; hb < NHB; ++hb) {
      const int head = hb * 16 + r;
      v8i qa;
      int sa;
      if (FMT == 1) {
        const uint4 *q = reinterpret_cast<const uint4 *>(ql.codes + head * 128 + g * 32);
        const uint4 y0 = q[0], y1 = q[1];
        qa = v8i{int(y0.x), int(y0.y), int(y0.z), int(y0.w), int(y1.x), int(y1.y), int(y1.z), int(y1.w)};
        sa = 127;
      } else {
        const uint4 y0 = *reinterpret_cast<const uint4 *>(ql.codes + head * 64 + g * 16);
        qa = v8i{int(y0.x), int(y0.y), int(y0.z), int(y0.w), 0, 0, 0, 0};
        sa = ql.sbytes[head * 4 + g];
      }
      const v4f c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, bop, v4f{0.f, 0.f, 0.f, 0.f}, fmt, fmt, 0,
                                                                     sa, 0, sb);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc = fmaf(ql.f[hb * 16 + g * 4 + v], relu(c[v]), acc);
    }
    acc = lane_group_sum(acc);
    const int el = grp * 16 + r;
    const float ks = FMT == 1 ? __uint_as_float(kf.s) : 1.0f;
    if (lane < 16) s_scores[el] = el < vis ? acc * ks : -INFINITY;
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
__device__ __forceinline__ uint64_t block_cut(const uint64_t (&keys)[KPT], int need, int keep_min, SelectLds &sl) {
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

// ---- bucket select ---------------------------------------------------------------------------
// The same cut as block_cut, found from histograms of the keys' score orders (the high words, which
// order like the scores) over kBins bins: bin = (o - base) >> shift, with the shift that fits the
// orders' span into kBins bins.  The bin never decreases as the score grows, so every key of a
// higher bin is larger than every key of a lower one.  Binning the order bits is binning the scores
// on a scale that is linear inside each binade and doubles its step per binade: a few extreme
// scores (planted keys, ten times the rest) widen the span by a few binades instead of squeezing
// every other key into a handful of bins.  A pass locates the bin where the count from the top
// reaches `need`; the result is that bin's edge when it leaves at least keep_min keys above (or
// exactly `need` from it down), the exact key of rank `need` when the bin holds at most
// kSmallBucket keys (one wave ranks them), or else a second pass over the crossing bin alone;
// equal or extremely clustered scores fall to the radix select.  A bin edge is a threshold key
// (low word 0): the keys >= it are exactly the keys of the bins above, as with any other cut.
// With fewer than `need` non-zero keys the result is 0 (every key is kept).
constexpr int kBins = 2048;
constexpr int kSmallBucket = 64;

struct alignas(16) BucketLds {
  uint32_t hist[kBins];
  uint64_t list[kSmallBucket];      // keys of the crossing bin
  int part[8][kSmallBucket];        // partial ranks of the listed keys, one row per wave
  uint64_t kmin[16];
  uint32_t omin[16], omax[16];
  int wsum[16];
  int res[4];                       // crossing bin, keys above it, keys in it, keys listed
};

// Reductions over the wave whose result every lane holds: DPP inside rows of 16 lanes, then the
// gfx950 half-wave and row swaps across the four rows (no readlane round trips).
template <bool MIN>
__device__ __forceinline__ uint32_t wave_all_u32(uint32_t v) {
  auto pick = [](uint32_t x, uint32_t y) { return MIN ? min(x, y) : max(x, y); };
  v = pick(v, uint32_t(dpp<kDppQuadXor1>(int(v))));
  v = pick(v, uint32_t(dpp<kDppQuadXor2>(int(v))));
  v = pick(v, uint32_t(dpp<kDppRowHalfMirror>(int(v))));
  v = pick(v, uint32_t(dpp<kDppRowMirror>(int(v))));
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = pick(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return pick(b[0], b[1]);
}
// Inclusive prefix sum over the wave: DPP shifts inside rows, then the GFX9 row broadcasts of
// lanes 15 and 31 to the rows above them.
__device__ __forceinline__ int wave_scan_bcast(int v) {
  v += dpp<kDppRowShr + 1>(v);
  v += dpp<kDppRowShr + 2>(v);
  v += dpp<kDppRowShr + 4>(v);
  v += dpp<kDppRowShr + 8>(v);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return v;
}

template <int NT, int KPT>
__device__ __forceinline__ uint64_t block_cut_bucket(const uint64_t (&keys)[KPT], int need, int keep_min, BucketLds &bl,
                                                     SelectLds &sl) {
  constexpr int NW = NT / 64, BPT = kBins / NT;
  static_assert(BPT == 4, "four bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t omin = ~0u, omax = 0u;
  int nk = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const uint32_t o = uint32_t(keys[k] >> 32);
    omin = min(omin, keys[k] != 0 ? o : ~0u);
    omax = max(omax, o);                                      // an empty key's order is 0
    nk += keys[k] != 0;
  }
  reinterpret_cast<uint4 *>(bl.hist)[tid] = make_uint4(0, 0, 0, 0);   // NT x 4 bins = kBins
  if (tid == 0) bl.res[3] = 0;
  omin = wave_all_u32<true>(omin);
  omax = wave_all_u32<false>(omax);
  nk = wave_scan_bcast(nk);
  if (lane == 63) { bl.omin[wave] = omin; bl.omax[wave] = omax; bl.wsum[8 + wave] = nk; }
  lds_barrier();
  nk = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { omin = min(omin, bl.omin[w]); omax = max(omax, bl.omax[w]); nk += bl.wsum[8 + w]; }
  if (nk < need) return 0;                                     // fewer keys than asked: keep them all
  if (omin == omax) return block_cut<NT, KPT>(keys, need, keep_min, sl);    // one score: by index
  uint32_t base = omin, span = omax - omin;                   // the undecided keys' orders
  int rneed = need, rkeep = keep_min;                          // still to find among them
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = max(0, 32 - __clz(span) - 11);          // span >> shift < kBins
    int bin[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const uint32_t d = uint32_t(keys[k] >> 32) - base;
      bin[k] = (keys[k] != 0 && d <= span) ? int(d >> shift) : -1;
      if (bin[k] >= 0) atomicAdd(&bl.hist[bin[k]], 1u);
    }
    lds_barrier();
    // this thread's four bins, highest first, and the undecided keys in every higher bin
    const int top = kBins - 1 - tid * BPT;
    const uint4 x = reinterpret_cast<const uint4 *>(bl.hist)[(top - 3) >> 2];
    const int c0 = int(x.w), c1 = int(x.z), c2 = int(x.y), c3 = int(x.x);
    const int sum = c0 + c1 + c2 + c3;
    const int incl = wave_scan_bcast(sum);
    if (lane == 63) bl.wsum[wave] = incl;
    lds_barrier();
    int cum = incl - sum;
#pragma unroll
    for (int w = 0; w < NW; ++w) cum += w < wave ? bl.wsum[w] : 0;
    {
      const int a0 = cum, a1 = a0 + c0, a2 = a1 + c1, a3 = a2 + c2;
      const int hit = (a0 < rneed && rneed <= a1) ? 0 : (a1 < rneed && rneed <= a2) ? 1
                    : (a2 < rneed && rneed <= a3) ? 2 : (a3 < rneed && rneed <= a3 + c3) ? 3 : -1;
      if (hit >= 0) {
        bl.res[0] = top - hit;
        bl.res[1] = hit == 0 ? a0 : hit == 1 ? a1 : hit == 2 ? a2 : a3;
        bl.res[2] = hit == 0 ? c0 : hit == 1 ? c1 : hit == 2 ? c2 : c3;
      }
    }
    // the histogram is read: its readers clear their own bins for a second pass
    reinterpret_cast<uint4 *>(bl.hist)[(top - 3) >> 2] = make_uint4(0, 0, 0, 0);
    lds_barrier();
    const int bstar = bl.res[0], above = bl.res[1], cnt = bl.res[2];
    if (above >= rkeep)                                        // the bins above keep enough
      return uint64_t(base + (uint32_t(bstar + 1) << shift)) << 32;
    if (above + cnt == rneed) return uint64_t(base + (uint32_t(bstar) << shift)) << 32;
    if (cnt <= kSmallBucket) {                                 // rank the crossing bin's keys (distinct)
      // the wave's crossing keys (ballots, counted in scalar registers) get one range of the list:
      // one LDS atomic per wave
      uint64_t bal[KPT];
      int tot = 0;
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        bal[k] = __ballot(bin[k] == bstar);
        tot += __popcll(bal[k]);
      }
      if (tot) {
        int wb = 0;
        if (lane == 0) wb = atomicAdd(&bl.res[3], tot);
        wb = __builtin_amdgcn_readlane(wb, 0);
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
          const int r = __builtin_amdgcn_mbcnt_hi(uint32_t(bal[k] >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(bal[k]), 0));
          if (bin[k] == bstar) bl.list[wb + r] = keys[k];
          wb += __popcll(bal[k]);
        }
      }
      lds_barrier();
      if (cnt <= 16) {                                         // a short list: one wave ranks it
        if (wave == 0) {
          const uint64_t v = lane < cnt ? bl.list[lane] : 0;
          int rank = 0;
          for (int j = 0; j < cnt; ++j) rank += readlane64(v, j) > v;
          if (lane < cnt && rank == rneed - above - 1) bl.kmin[0] = v;
        }
        lds_barrier();
        return bl.kmin[0];
      }
      // lane l of every wave ranks listed key l against the wave's share of the list (the key of
      // rank r has exactly r listed keys above it); wave 0 adds the waves' partial ranks
      {
        constexpr int SH = kSmallBucket / NW;                  // listed keys per wave
        static_assert(NW <= 8 && SH * NW == kSmallBucket, "the list splits over the waves");
        const uint64_t v = lane < cnt ? bl.list[lane] : 0;
        int part = 0;
#pragma unroll
        for (int j = 0; j < SH; ++j) {
          const int o = wave * SH + j;
          part += (o < cnt && bl.list[o] > v) ? 1 : 0;
        }
        bl.part[wave][lane] = part;
      }
      lds_barrier();
      if (wave == 0 && lane < cnt) {
        int rank = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) rank += bl.part[w][lane];
        if (rank == rneed - above - 1) bl.kmin[0] = bl.list[lane];
      }
      lds_barrier();
      return bl.kmin[0];
    }
    if (shift == 0) break;                                     // one score in the bin: by index
    base += uint32_t(bstar) << shift;                          // narrow to the crossing bin
    span = (1u << shift) - 1;
    rneed -= above;
    rkeep -= above;
  }
  // equal or extremely clustered scores: the radix select decides (ties by index)
  return block_cut<NT, KPT>(keys, need, keep_min, sl);
}

// ---- tile cut from the score distribution --------------------------------------------------
// z with P(Z > z) = p for a standard normal Z, 0 < p <= 1/2: the rational approximation of
// Abramowitz and Stegun, Handbook of Mathematical Functions, formula 26.2.23 (|error| < 4.5e-4).
__device__ __forceinline__ float normal_upper_quantile(float p) {
  const float t = sqrtf(-2.0f * __logf(p));
  return t - (2.515517f + t * (0.802853f + t * 0.010328f)) / (1.0f + t * (1.432788f + t * (0.189269f + t * 0.001308f)));
}

// Sum over the wave's 64 lanes, in lane 63 (inclusive DPP scan, then the row broadcasts).
__device__ __forceinline__ float wave_total_f32(float v) {
  v += __int_as_float(dpp<kDppRowShr + 1>(__float_as_int(v)));
  v += __int_as_float(dpp<kDppRowShr + 2>(__float_as_int(v)));
  v += __int_as_float(dpp<kDppRowShr + 4>(__float_as_int(v)));
  v += __int_as_float(dpp<kDppRowShr + 8>(__float_as_int(v)));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return v;
}

// A tile's candidates: its entries whose scores reach a cut that keeps between cand / 2 and cand
// of them (all of them when at most cand are visible), written in entry order as keys to `dst`
// with coherent stores, then their count and the cut (0: nothing cut) for the merge.  The tile's
// scores are sums over many heads, so their upper tail is close to normal: each wave's mean and
// mean absolute deviation about it (a spread one extreme score -- a planted or duplicated key --
// barely moves) place the score ranked 3 cand / 4 near mean + z sd, sd = sqrt(pi / 2) x deviation;
// four thresholds from 0.15 sd below to 0.45 sd above it (the ReLU sums' tail is heavier than a
// normal one with the same deviation, so the range leans upward) are counted in one pass, with the
// positions every kept entry takes, and the highest threshold that keeps between cand / 2 and
// cand entries is the cut: two barriers in all.  When none does (a tail far from normal), the histogram cut decides.  Which threshold is
// taken changes only how many candidates the tile hands to the merge, never which entries win.
// Scores: KPT consecutive entries per thread in `scores` (LDS); entries past vis are ignored.
template <int NT, int KPT>
__device__ __forceinline__ void publish_candidates(const float *scores, int vis, int64_t e_begin, int cand,
                                                   uint64_t *dst, int *count_out, uint64_t *bound_out, BucketLds &bl,
                                                   SelectLds &sl, int *tmp) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 8 && NT * KPT < 65536, "per-wave sums in bl.wsum, 16-bit counts");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int keep_min = cand / 2;
  float x[KPT];
  uint32_t o[KPT];                                 // score order; 0 for an entry past vis
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = tid * KPT + k;
    x[k] = scores[i];
    o[k] = i < vis ? score_order(x[k]) : 0u;
  }
  auto key_of = [&](int k) { return (uint64_t(o[k]) << 32) | uint64_t(~uint32_t(e_begin + tid * KPT + k)); };
  uint64_t bound = 0;                              // keep the entries whose keys reach it
  int pos = 0, total = 0;
  bool done = false;
  if (vis > cand) {
    // this wave's mean, then its summed absolute deviation about that mean
    const int n_w = min(max(vis - wave * 64 * KPT, 0), 64 * KPT);
    float s1 = 0.f;
#pragma unroll
    for (int k = 0; k < KPT; ++k) s1 += o[k] != 0 ? x[k] : 0.f;
    s1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_total_f32(s1)), 63));
    const float m_w = n_w > 0 ? s1 / float(n_w) : 0.f;
    float d1 = 0.f;
#pragma unroll
    for (int k = 0; k < KPT; ++k) d1 += o[k] != 0 ? fabsf(x[k] - m_w) : 0.f;
    d1 = wave_total_f32(d1);
    if (lane == 63) bl.kmin[wave] = (uint64_t(__float_as_uint(d1)) << 32) | __float_as_uint(s1);
    lds_barrier();
    float sum = 0.f, dev = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint64_t v = bl.kmin[w];
      sum += __uint_as_float(uint32_t(v));
      dev += __uint_as_float(uint32_t(v >> 32));
    }
    const float inv_n = 1.0f / float(vis);
    const float mean = sum * inv_n, sd = 1.2533141f * dev * inv_n;
    const float z = normal_upper_quantile(fminf(0.5f, 0.5f * float(cand + keep_min) * inv_n));
    uint32_t th[4];
    const float dz[4] = {0.45f, 0.25f, 0.05f, -0.15f};         // highest threshold first
#pragma unroll
    for (int j = 0; j < 4; ++j) th[j] = score_order(fmaf(z + dz[j], sd, mean));
    // the four counts in two words (16 bits each), their wave prefixes and totals
    uint32_t c01 = 0, c23 = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      c01 += (o[k] >= th[0] ? 1u : 0u) + (o[k] >= th[1] ? 0x10000u : 0u);
      c23 += (o[k] >= th[2] ? 1u : 0u) + (o[k] >= th[3] ? 0x10000u : 0u);
    }
    const uint32_t i01 = uint32_t(wave_scan_bcast(int(c01))), i23 = uint32_t(wave_scan_bcast(int(c23)));
    if (lane == 63) { bl.wsum[wave] = int(i01); bl.wsum[8 + wave] = int(i23); }
    lds_barrier();
    uint32_t t01 = 0, t23 = 0, p01 = 0, p23 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t v01 = uint32_t(bl.wsum[w]), v23 = uint32_t(bl.wsum[8 + w]);
      t01 += v01; t23 += v23;
      if (w < wave) { p01 += v01; p23 += v23; }
    }
    const uint32_t tot[4] = {t01 & 0xffffu, t01 >> 16, t23 & 0xffffu, t23 >> 16};
    int pick = -1;
#pragma unroll
    for (int j = 3; j >= 0; --j)
      if (int(tot[j]) >= keep_min) pick = j;                   // the highest threshold keeping enough
    if (pick >= 0 && int(tot[pick]) <= cand && th[pick] != 0) {
      const uint32_t pre01 = p01 + i01 - c01, pre23 = p23 + i23 - c23;   // entries kept before mine
      const uint32_t pre = pick == 0 ? (pre01 & 0xffffu) : pick == 1 ? (pre01 >> 16)
                         : pick == 2 ? (pre23 & 0xffffu) : (pre23 >> 16);
      bound = uint64_t(th[pick]) << 32;                       // keys >= it: orders >= th[pick]
      pos = int(pre);
      total = int(tot[pick]);
      done = true;
    } else {
      uint64_t keys[KPT];
#pragma unroll
      for (int k = 0; k < KPT; ++k) keys[k] = o[k] != 0 ? key_of(k) : 0;
      bound = block_cut_bucket<NT, KPT>(keys, cand, keep_min, bl, sl);
    }
  }
  if (!done) {                                     // positions by a block scan
    int mine = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) mine += (o[k] != 0 && key_of(k) >= bound);
    pos = block_excl_scan<NT>(mine, tmp, total);
  }
#pragma unroll
  for (int k = 0; k < KPT; ++k)
    if (o[k] != 0 && key_of(k) >= bound) store_coherent(&dst[pos++], key_of(k));
  if (tid == 0) { store_coherent(count_out, total); store_coherent(bound_out, bound); }
}

// A key E such that exactly `need` of the block's non-zero keys are >= E (the rank-`need` key,
// 1 = largest, or a bin edge just below it), or 0 when there are fewer than `need` keys.
template <int NT, int KPT>
__device__ __forceinline__ uint64_t block_select(const uint64_t (&keys)[KPT], int need, BucketLds &bl, SelectLds &sl) {
  return block_cut_bucket<NT, KPT>(keys, need, need, bl, sl);
}

// ---- the merge: a query's exact top-k from its tiles' candidates -----------------------------
// Run either by the last of the query's tile workgroups to finish (one-query path: no separate
// launch) or by a merge kernel with one workgroup per query (shared-tile path).
template <int TILE>
struct alignas(16) IndexSharedT {
  QueryLds ql;                        // the query (quantised, or fp32 values and weights)
  float scores[TILE];                 // one tile's scores
  SelectLds sel;
  BucketLds bl;
  int tmp[16];
  int flag;
  int counts[kMaxCand / 8];           // per tile: candidates kept
  uint64_t bounds[kMaxCand / 8];      // per tile: smallest kept key (0: the tile kept every entry)
  uint64_t work[kMaxK + TILE];        // exact fallback: the working set
};
// the tile kernel (tiles of up to kMaxTile entries)
typedef IndexSharedT<kMaxTile> IndexShared;

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

// The query of merge workgroup `qi` into sh.ql (fp32: values and weights; otherwise quantised).
template <int FMT, int NT, class SH>
__device__ __forceinline__ void load_query_lds(const IndexArgs &a, SH &sh, int64_t qi) {
  if (FMT == 0) {
    float *q_lds = reinterpret_cast<float *>(sh.ql.codes);    // H_I * D_I <= 2048 floats
    const float *qsrc = static_cast<const float *>(a.q_idx) + qi * a.H_I * a.D_I;
    for (int i = threadIdx.x; i < a.H_I * a.D_I; i += NT) q_lds[i] = qsrc[i];
    if (int(threadIdx.x) < a.H_I) sh.ql.f[threadIdx.x] = a.w_idx[qi * a.H_I + threadIdx.x];
  } else {
    QueryRaw raw;
    load_query_raw(static_cast<const uint16_t *>(a.q_idx) + qi * a.H_I * 128, a.w_idx + qi * a.H_I, a.H_I, raw);
    prep_query_lds<FMT>(raw, a.H_I, sh.ql);
  }
  lds_barrier();
}

// Exact fallback: the candidate set may miss winners hidden in tiles whose kept keys all beat
// `tau`.  Keep a working set W (the k_eff best so far) in LDS and merge in every such tile,
// re-scored from its keys.  Writes the final selection in ascending index order.  The query must
// be in sh.ql already.
template <int FMT, int NHB, int NT, int KPT, class SH>
__device__ __forceinline__ void merge_fallback(const IndexArgs &a, SH &sh, const uint64_t (&keys)[KPT], uint64_t tau,
                               int b, int64_t n_vis, int k_eff, int32_t *out) {
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
  const float *q_lds = reinterpret_cast<const float *>(sh.ql.codes);
  constexpr int KW = int(sizeof(sh.work) / 8) / NT;          // the working set: k_eff + one tile
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
      score_tile_lean<FMT, NHB>(sh.ql, tk, tile, vis, sh.scores);
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
      tau = block_select<NT, KW>(wk, k_eff, sh.bl, sh.sel);
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

// Select query qi's top-k from the candidates of all its tiles (candidate slots of tile j at
// j * cand, ascending entry order within a tile, so slot order is entry order).  `have_query`: the
// query is already in sh.ql (the tile workgroup that scored it), needed only by the fallback.
template <int FMT, int NHB, int NT, int KPT, class SH>
__device__ __forceinline__ void merge_query(const IndexArgs &a, SH &sh, int64_t qi, int b, int s, bool have_query) {
  const int tid = threadIdx.x;
  const int cand = a.plan.cand, n_tiles = a.plan.n_tiles;
  const int cshift = __builtin_ctz(uint32_t(cand));              // cand is a power of two
  const int64_t n_q = int64_t(a.B) * a.Sq;
  const uint64_t *cand_keys = static_cast<const uint64_t *>(a.workspace);
  const uint64_t *cand_bound = cand_keys + n_q * n_tiles * cand;
  const int *cand_count = reinterpret_cast<const int *>(cand_bound + n_q * n_tiles);
  int32_t *out = a.topk_idx + qi * a.topk;

  // candidate slots and per-tile counts are loaded together; slots past a tile's count are masked
  uint64_t keys[KPT];
  const int slots = n_tiles * cand;                            // a multiple of 8
  static_assert(KPT % 2 == 0, "slots are loaded in pairs");
  {
    // coherent loads (the tile workgroups of this launch wrote them); slots past the region read 0
    const __amdgpu_buffer_rsrc_t src = coherent_region(cand_keys + qi * slots, uint32_t(slots) * 8u);
#pragma unroll
    for (int k = 0; k < KPT; k += 2) {
      const uint4 v = load_coherent16(src, uint32_t(tid * KPT + k) * 8u);
      keys[k] = (uint64_t(v.y) << 32) | v.x;
      keys[k + 1] = (uint64_t(v.w) << 32) | v.z;
    }
  }
  // per-tile counts and bounds, held in registers until the position is known (loaded from a
  // clamped slot, so no branch separates these loads from the ones above)
  constexpr int TPT = (kMaxCand / 8 + NT - 1) / NT;
  int cnt[TPT];
  uint64_t bnd[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int i = min(tid + j * NT, n_tiles - 1);
    cnt[j] = load_coherent(&cand_count[qi * n_tiles + i]);
    bnd[j] = load_coherent(&cand_bound[qi * n_tiles + i]);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int64_t t = a.q_pos0[b] + s;
  const int64_t n_vis = min(a.n_entries[b], div_count(t + 1, a.m));
  const int k_eff = int(min(int64_t(a.topk), n_vis));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int i = tid + j * NT;
    if (i < n_tiles) { sh.counts[i] = cnt[j]; sh.bounds[i] = bnd[j]; }
  }
  if (tid == 0) sh.flag = 0;
  lds_barrier();
  // (every count read first, from a clamped slot, so that one wait covers them all)
  int kc[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) kc[k] = sh.counts[min(tid * KPT + k, slots - 1) >> cshift];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int slot = tid * KPT + k;
    if (slot >= slots || (slot & (cand - 1)) >= kc[k]) keys[k] = 0;
  }
  if (k_eff == 0) {
    for (int i = tid; i < a.topk; i += NT) out[i] = -1;
    return;
  }
  // the k-th best candidate (0 when fewer than k_eff candidates: every one is kept)
  const uint64_t tau = block_select<NT, KPT>(keys, k_eff, sh.bl, sh.sel);
  // a truncated tile whose cut beats tau may hold further winners (the flag is read after the
  // output positions' scan, whose barrier publishes it)
  for (int i = tid; i < n_tiles; i += NT)
    if (sh.bounds[i] != 0 && sh.bounds[i] > tau) sh.flag = 1;
  int mine = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) mine += (keys[k] != 0 && keys[k] >= tau);
  int total;
  int pos = block_excl_scan<NT>(mine, sh.tmp, total);
  if (sh.flag) {
    if (!have_query) load_query_lds<FMT, NT>(a, sh, qi);
    merge_fallback<FMT, NHB, NT, KPT>(a, sh, keys, tau, b, n_vis, k_eff, out);
    return;
  }
#pragma unroll
  for (int k = 0; k < KPT; ++k)
    if (keys[k] != 0 && keys[k] >= tau) out[pos++] = int32_t(key_index(keys[k]));
  for (int i = k_eff + tid; i < a.topk; i += NT) out[i] = -1;
}

// Arrival counters of the one-query path: one per query (kCounterStride apart), after the
// candidate arrays.
__host__ __device__ inline size_t arrivals_offset(int64_t n_q, const IndexPlan &p) {
  const int64_t slots = n_q * p.n_tiles;
  const size_t off = size_t(slots * p.cand * 8 + slots * 8 + slots * 4);
  return (off + 255) / 256 * 256;
}

// ---- kernel 1: fp32 keys -- scores, per-tile candidates and (last tile of a query) the merge ------
// One query and one tile of up to 2,048 entries per workgroup; one thread per entry.  Every tile
// workgroup of a query publishes its candidates and counts itself in (arrive_last); the last one
// runs the merge for the query and leaves the counter at zero for the next call.
template <int NT, int KPT, int MKPT, bool FUSE>
__global__ void __launch_bounds__(NT) index_score_kernel(IndexArgs a) {
  __shared__ IndexShared sh;
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
  const int64_t t = a.q_pos0[b] + s;
  const int64_t n_vis = min(a.n_entries[b], div_count(t + 1, a.m));
  const int vis = int(max(int64_t(0), min(int64_t(tile), n_vis - e_begin)));
  // a tile with nothing visible publishes an empty candidate list (unless scores are asked for)
  const bool work = vis > 0 || a.scores != nullptr;
  if (work) {
    load_query_lds<0, NT>(a, sh, qi);
    score_tile_f32(reinterpret_cast<const float *>(sh.ql.codes), sh.ql.f, a.H_I, a.D_I,
                   static_cast<const float *>(a.k_codes), row0, tile, vis, sh.scores);
    lds_barrier();
    if (a.scores) {
      float *dst = a.scores + qi * a.N_cap;
      for (int i = threadIdx.x; i < tile; i += NT)
        if (e_begin + i < a.N_cap) dst[e_begin + i] = sh.scores[i];
    }
    publish_candidates<NT, KPT>(sh.scores, vis, e_begin, cand, cand_keys + out_slot * cand, &cand_count[out_slot],
                                &cand_bound[out_slot], sh.bl, sh.sel, sh.tmp);
  } else if (threadIdx.x == 0) {
    store_coherent(&cand_count[out_slot], 0);
    store_coherent(&cand_bound[out_slot], uint64_t(0));
  }
  if constexpr (FUSE) {
    int *arrivals = reinterpret_cast<int *>(static_cast<uint8_t *>(a.workspace) + arrivals_offset(n_q, a.plan));
    if (!arrive_last(&arrivals[qi * kCounterStride], a.plan.n_tiles, &sh.flag)) return;
    merge_query<0, 1, NT, MKPT>(a, sh, qi, b, s, work);
  }
}

// ---- kernel 1s: streaming scores of quantised keys, one query per workgroup ------------------
// One 512-thread workgroup per CU owns a contiguous segment of one query's keys (up to 4,096
// entries) and streams it through a ring of three 32 KB LDS chunks filled by direct-to-LDS
// buffer loads (range-checked: rows past the cache read as zeros): the query and the first chunk
// are requested at once, the next two chunks once the query is in, and every chunk scored frees
// its slot for the chunk two ahead.  The loads are laid out so that lane (r, g) of a scoring wave
// reads its MFMA key operand (entry r of a 16-entry group, K-chunk g) as one linear 16-byte LDS
// read.  Scores (the same MFMA operands and epilogue order as the shared-tile kernel and the
// merge's exact re-scoring, hence the same bits) stay in LDS; the segment then keeps its best
// keys like a tile, and the query's last segment workgroup to finish merges (FUSE).
//
// The LDS loads are issued from inline assembly with their LDS address in m0: the compiler then
// knows of no vector-memory load in flight and adds no waits of its own, and every wait is an
// explicit vmcnt count below (chunks complete in issue order; the query's loads are issued first).
// The compiler's LDS-DMA intrinsic would serve as well, except that the compiler cannot tell the
// ring's slots apart and waits for every chunk in flight before each LDS read.
constexpr int kStreamThreads = 512;
constexpr int kStreamSeg = 4096;                    // entries per workgroup, at most
constexpr int kRingSlots = 3;
constexpr int kChunkBytes = 32768;                  // key codes per ring slot
template <int FMT>
constexpr int chunk_entries() { return FMT == 1 ? 256 : 512; }

__device__ __forceinline__ uint32_t lds_address(const void *p) {      // p points into LDS
  const __attribute__((address_space(3))) void *l = (const __attribute__((address_space(3))) void *)(p);
  return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(l)));
}
// Lane l's 16 (4) bytes at byte offset voff of the buffer go to LDS address m0 + 16 l (4 l).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_loads() {               // at most N vector loads in flight
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Barrier for the ring: the wave's direct-to-LDS loads are complete already (explicit vmcnt
// waits); its own LDS reads complete before it (lgkmcnt(0)), so a slot read before the barrier may
// be refilled after it; the compiler-only fences keep LDS accesses from moving across it.
__device__ __forceinline__ void ring_barrier() { lds_sync(); }

struct alignas(16) StreamShared {
  union {
    struct {                                        // while streaming
      uint8_t codes[kRingSlots][kChunkBytes];
      uint32_t scales[kRingSlots][512];
    };
    struct {                                        // the merge, after the stream
      int counts[kMaxCand / 8];
      uint64_t bounds[kMaxCand / 8];
      uint64_t work[kMaxK + kStreamSeg];
    };
  };
  QueryLds ql;
  float scores[kStreamSeg];                         // before the scores: the raw bf16 query
  float qw[64];                                     // the query's head weights
  SelectLds sel;
  BucketLds bl;
  int tmp[16];
  int flag;
};

template <int FMT, int NHB, bool FUSE>
__global__ void __launch_bounds__(kStreamThreads, 1) index_stream_kernel(IndexArgs a) {
  constexpr int NT = kStreamThreads, NW = NT / 64;
  constexpr int CH = chunk_entries<FMT>();          // entries per chunk
  constexpr int RB = FMT == 1 ? 128 : 64;           // code bytes per entry
  static_assert(CH * RB == kChunkBytes, "a chunk fills one slot");
  constexpr int CODE_I = kChunkBytes / 1024 / NW;   // 16-byte-per-lane loads per wave and chunk
  constexpr int SCALE_I = CH / 64;                  // 4-byte-per-lane loads holding a chunk's scales
  constexpr int P = CODE_I + 1;                     // loads per wave and chunk
  constexpr int GPW = CH / 16 / NW;                 // 16-entry groups scored per wave and chunk
  constexpr int KPT = kStreamSeg / NT;
  constexpr int Q_I = 2;                            // the raw query: 16 KB of bf16 over 8 waves
  __shared__ StreamShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int seg_id = blockIdx.x;
  const int64_t qi = blockIdx.y;
  const int b = int(blockIdx.y / uint32_t(a.Sq)), s = int(blockIdx.y) - b * a.Sq;
  const int seg = a.plan.tile, cand = a.plan.cand;
  const int64_t e_begin = int64_t(seg_id) * seg;
  const int64_t out_slot = qi * a.plan.n_tiles + seg_id;
  const int64_t n_q = int64_t(a.B) * a.Sq;
  const int rows = int(min(int64_t(seg), a.N_cap - e_begin));
  const int nch = (rows + CH - 1) / CH;
  const int64_t row0 = int64_t(b) * a.N_cap + e_begin;
  // the position and entry count first: loaded before any asm statement, they stay scalar loads
  // (a vector load here would make the compiler wait for every direct-to-LDS load issued before
  // its use)
  const int64_t t = a.q_pos0[b] + s;
  const int64_t n_ent = a.n_entries[b];
  const __amdgpu_buffer_rsrc_t rcodes = coherent_region(static_cast<const uint8_t *>(a.k_codes) + row0 * RB,
                                                        uint32_t(rows * RB));
  const __amdgpu_buffer_rsrc_t rscales = coherent_region(static_cast<const uint8_t *>(a.k_scales) + row0 * 4,
                                                         uint32_t(rows * 4));
  // the raw query (heads x 128 bf16; heads past H_I read zeros) and its weights, first
  {
    const __amdgpu_buffer_rsrc_t rq = coherent_region(static_cast<const uint16_t *>(a.q_idx) + qi * a.H_I * 128,
                                                      uint32_t(a.H_I * 256));
    const __amdgpu_buffer_rsrc_t rw = coherent_region(a.w_idx + qi * a.H_I, uint32_t(a.H_I * 4));
#pragma unroll
    for (int i = 0; i < Q_I; ++i) {
      const int blk = wave * Q_I + i;                 // 1 KB blocks of the 16 KB query
      lds_load16(rq, uint32_t(blk * 1024 + lane * 16), lds_address(reinterpret_cast<uint8_t *>(sh.scores) + blk * 1024));
    }
    lds_load4(rw, uint32_t(lane * 4), lds_address(sh.qw));   // every wave: the same 256 bytes
  }
  // chunk c of the segment into ring slot SLOT
  auto issue = [&](int c, uint8_t *codes, uint32_t *scales) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CODE_I; ++i) {
      const int blk = wave * CODE_I + i;              // 1 KB block of the slot
      uint32_t off;
      if (FMT == 1) {                                 // block = half h of group blk / 2: bytes 16 (2 g + h)
        const int grp = blk >> 1, h = blk & 1;
        off = uint32_t((c * CH + grp * 16 + r16) * RB + (2 * g4 + h) * 16);
      } else {                                        // block = group blk: bytes 16 g of each entry
        off = uint32_t((c * CH + blk * 16 + r16) * RB + g4 * 16);
      }
      lds_load16(rcodes, off, lds_address(codes + blk * 1024));
    }
    const int j = wave % SCALE_I;                     // scale block j (fp8: two waves load each block)
    lds_load4(rscales, uint32_t((c * CH + j * 64 + lane) * 4), lds_address(scales + j * 64));
  };
  // chunk 0 goes out with the query; chunks 1 and 2 only once the query is in: every load issued
  // across the device before the query's is served before it, so the first requests are kept few
  issue(0, sh.codes[0], sh.scales[0]);
  const int64_t n_vis = min(n_ent, div_count(t + 1, a.m));
  const int vis = int(max(int64_t(0), min(int64_t(seg), n_vis - e_begin)));
  wait_loads<P>();                                  // the query (issued before chunk 0)
  ring_barrier();
  if (nch > 1) issue(1, sh.codes[1], sh.scales[1]);
  if (nch > 2) issue(2, sh.codes[2], sh.scales[2]);
  if (tid < 256) {
    QueryRaw raw;
    const int h = min(tid >> 2, a.H_I - 1), c = tid & 3;
    const uint4 *src = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(sh.scores) + h * 256 + c * 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 v = src[k];
      raw.wv[4 * k] = v.x; raw.wv[4 * k + 1] = v.y; raw.wv[4 * k + 2] = v.z; raw.wv[4 * k + 3] = v.w;
    }
    raw.w = sh.qw[h];
    prep_query_slot<FMT>(raw, tid, a.H_I, sh.ql);
  }
  ring_barrier();
  QueryFrag<NHB> qf;
  load_query_frag<FMT, NHB>(sh.ql, lane, qf);
  constexpr int fmt = FMT == 1 ? 0 : 4;               // instruction format code: 0 = fp8 e4m3, 4 = fp4 e2m1
  // scores of chunk c from a slot: the wave's GPW groups, MFMAs of the next group issued before the
  // previous group's epilogue
  auto score = [&](int c, const uint8_t *codes, const uint32_t *scales) __attribute__((always_inline)) {
    v8i bop[GPW];
    uint32_t ks[GPW];
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      const int grp = wave * GPW + u;
      uint4 x0, x1 = make_uint4(0, 0, 0, 0);
      if (FMT == 1) {
        x0 = *reinterpret_cast<const uint4 *>(codes + (2 * grp) * 1024 + lane * 16);
        x1 = *reinterpret_cast<const uint4 *>(codes + (2 * grp + 1) * 1024 + lane * 16);
      } else {
        x0 = *reinterpret_cast<const uint4 *>(codes + grp * 1024 + lane * 16);
      }
      bop[u] = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      ks[u] = scales[grp * 16 + r16];
    }
    v4f acc4[2][NHB];
    auto mfma = [&](int u, v4f (&cc)[NHB]) __attribute__((always_inline)) {
      const int sb = FMT == 1 ? 127 : int((ks[u] >> (8 * g4)) & 0xff);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        cc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf.a[hb], bop[u], v4f{0.f, 0.f, 0.f, 0.f}, fmt, fmt,
                                                                  0, qf.sa[hb], 0, sb);
    };
    mfma(0, acc4[0]);
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
      if (u + 1 < GPW) mfma(u + 1, acc4[(u + 1) & 1]);
      float acc = 0.f;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc = fmaf(qf.f[hb][v], relu(acc4[u & 1][hb][v]), acc);
      acc = lane_group_sum(acc);
      const int el = c * CH + (wave * GPW + u) * 16 + r16;
      const float kscale = FMT == 1 ? __uint_as_float(ks[u]) : 1.0f;
      if (lane < 16) sh.scores[el] = el < vis ? acc * kscale : -INFINITY;
    }
  };
  // the stream: wait for chunk c (chunks c + 1 and, for c == 0, c + 2 may be younger), then refill
  // the slot of chunk c - 1 with chunk c + 2, then score chunk c
  auto step = [&](int c, int cur) __attribute__((always_inline)) {
    if (c == 0 && nch > 2) wait_loads<2 * P>();
    else if (c + 1 < nch) wait_loads<P>();
    else wait_loads<0>();
    ring_barrier();
    const int nxt = cur == 0 ? 2 : cur - 1;          // slot of chunk c + 2 = slot of chunk c - 1
    if (c >= 1 && c + 2 < nch) issue(c + 2, sh.codes[nxt], sh.scales[nxt]);
    score(c, sh.codes[cur], sh.scales[cur]);
  };
  for (int c = 0; c < nch; c += kRingSlots) {
    step(c, 0);
    if (c + 1 < nch) step(c + 1, 1);
    if (c + 2 < nch) step(c + 2, 2);
  }
  lds_barrier();
  if (a.scores) {
    float *dst = a.scores + qi * a.N_cap;
    for (int i = tid; i < rows; i += NT) dst[e_begin + i] = i < nch * CH ? sh.scores[i] : -INFINITY;
  }
  // the segment's best keys, as a tile's
  uint64_t *cand_keys = static_cast<uint64_t *>(a.workspace);
  uint64_t *cand_bound = cand_keys + n_q * a.plan.n_tiles * cand;
  int *cand_count = reinterpret_cast<int *>(cand_bound + n_q * a.plan.n_tiles);
  publish_candidates<NT, KPT>(sh.scores, vis, e_begin, cand, cand_keys + out_slot * cand, &cand_count[out_slot],
                              &cand_bound[out_slot], sh.bl, sh.sel, sh.tmp);
  if constexpr (FUSE) {
    int *arrivals = reinterpret_cast<int *>(static_cast<uint8_t *>(a.workspace) + arrivals_offset(n_q, a.plan));
    if (!arrive_last(&arrivals[qi * kCounterStride], a.plan.n_tiles, &sh.flag)) return;
    // the ring is no longer read: the merge's arrays may take its place
    merge_query<FMT, NHB, NT, 8>(a, sh, qi, b, s, true);
  }
}

// ---- kernel 1b (prefill): one key tile, eight queries of one sequence ------------------------
// For calls with many queries per sequence (a prefill chunk) the same keys are scored against
// consecutive queries.  Workgroup = (tile of 512 entries, 8 consecutive queries, sequence): the
// tile's quantised keys are loaded into LDS once and every wave scores them against its own query
// (encoded once per call by index_query_prep_kernel; each wave copies the image into its LDS slot
// before the tile arrives and reads its MFMA operands from there), then selects its candidates
// with a wave-local radix select -- no workgroup barrier after the tile is loaded.  Scores are
// bit-identical to the streaming kernel's (the same MFMA operands and epilogue order), so the
// selection is too.
constexpr int kMultiQ = 8;              // queries per workgroup, one per wave
constexpr int kMultiTile = 512;         // entries per tile

// Keep the wave's largest keys (8 per lane, distinct, 0 = absent): the same cut as block_cut --
// exactly `need` keys, or between keep_min and need - 1 when one histogram pass separates them --
// on one wave, with the wave's own 256-bin histogram in LDS and no workgroup barrier (a wave's
// LDS accesses complete in order; the fences keep the compiler from reordering them).

__device__ __forceinline__ uint64_t wave_cut(const uint64_t (&keys)[8], int need, int keep_min, uint32_t *H) {
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
// The indexer's query encoding on its own (csa_quantize_query): one workgroup per query, the same
// prep_query_slot as every scoring path, the image copied out field by field.
template <int FMT>
__global__ void __launch_bounds__(256) query_codes_kernel(const uint16_t *q, const float *w, int H_I, uint8_t *codes,
                                                          uint8_t *scale_bytes, float *factors) {
  __shared__ QueryLds ql;
  const int64_t qi = blockIdx.x;
  const int t = threadIdx.x;
  QueryRaw raw;
  load_query_raw(q + qi * H_I * 128, w + qi * H_I, H_I, raw, t);
  prep_query_slot<FMT>(raw, t, H_I, ql);
  lds_barrier();
  constexpr int RB = FMT == 1 ? 128 : 64;                      // code bytes per head
  for (int i = t; i < H_I * RB / 16; i += 256)
    reinterpret_cast<uint4 *>(codes + qi * H_I * RB)[i] = reinterpret_cast<const uint4 *>(ql.codes)[i];
  if (FMT == 2)
    for (int i = t; i < H_I * 4; i += 256) scale_bytes[qi * H_I * 4 + i] = ql.sbytes[i];
  if (t < H_I) factors[qi * H_I + t] = ql.f[t];
}

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
        const_cast<uint8_t *>(static_cast<const uint8_t *>(a.k_codes) + row0 * RB), short(0), rows * RB, kRawBufferDesc3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(static_cast<const uint8_t *>(a.k_scales) + row0 * 4), short(0), rows * 4, kRawBufferDesc3);
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

// ---- kernel 2 (shared-tile path, very long caches): one workgroup per query merges -----------
template <int FMT, int NHB>
__global__ void __launch_bounds__(kMergeThreads) index_merge_kernel(IndexArgs a) {
  __shared__ IndexSharedT<kStreamSeg> sh;             // tiles or stream segments (the fallback rescans one)
  const int64_t qi = blockIdx.x;
  const int b = int(blockIdx.x / uint32_t(a.Sq)), s = int(blockIdx.x) - b * a.Sq;
  merge_query<FMT, NHB, kMergeThreads, kMaxCand / kMergeThreads>(a, sh, qi, b, s, false);
}

template <int FMT, int NHB>
hipError_t launch_score_t(const IndexArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.plan.multi) {
    e = launch("index_query_prep", index_query_prep_kernel<FMT>, dim3(unsigned(int64_t(a.B) * a.Sq)), dim3(256),
               stream, a);
    if (e != hipSuccess) return e;
    const dim3 mgrid(unsigned(a.plan.n_tiles), unsigned((a.Sq + kMultiQ - 1) / kMultiQ), unsigned(a.B));
    e = launch("index_score", index_score_multi_kernel<FMT, NHB>, mgrid, dim3(64 * kMultiQ), stream, a);
    if (e != hipSuccess) return e;
    return launch("index_merge", index_merge_kernel<FMT, NHB>, dim3(unsigned(int64_t(a.B) * a.Sq)),
                  dim3(kMergeThreads), stream, a);
  }
  if (a.plan.stream) {
    // one query segment per workgroup; the merge runs in the last segment workgroup of each query
    // (fused), or for more than kFusedSlots candidate slots in a merge kernel after it
    const dim3 sgrid(unsigned(a.plan.n_tiles), unsigned(int64_t(a.B) * a.Sq));
    if constexpr (FMT != 0) {
      if (a.plan.fused)
        return launch("index_score", index_stream_kernel<FMT, NHB, true>, sgrid, dim3(kStreamThreads), stream, a);
      e = launch("index_score", index_stream_kernel<FMT, NHB, false>, sgrid, dim3(kStreamThreads), stream, a);
      if (e != hipSuccess) return e;
      return launch("index_merge", index_merge_kernel<FMT, NHB>, dim3(unsigned(int64_t(a.B) * a.Sq)),
                    dim3(kMergeThreads), stream, a);
    }
    return hipErrorInvalidValue;
  }
  // one query per tile workgroup of 512 threads; the merge runs in the last tile workgroup of each
  // query (fused), or for caches of more than 4,096 candidate slots in a merge kernel after it
  if constexpr (FMT == 0) {
    dim3 grid(unsigned(a.plan.n_tiles), unsigned(int64_t(a.B) * a.Sq));
#define CSA_SCORE_LAUNCH(KPT, FUSE) \
    e = launch("index_score", index_score_kernel<512, KPT, kFusedKeys, FUSE>, grid, dim3(512), stream, a)
    const bool fuse = a.plan.fused != 0;
    switch (a.plan.tile) {
      case 64: case 128: case 256: case 512:
        if (fuse) CSA_SCORE_LAUNCH(1, true); else CSA_SCORE_LAUNCH(1, false);
        break;
      case 1024:
        if (fuse) CSA_SCORE_LAUNCH(2, true); else CSA_SCORE_LAUNCH(2, false);
        break;
      case 2048:
        if (fuse) CSA_SCORE_LAUNCH(4, true); else CSA_SCORE_LAUNCH(4, false);
        break;
      default: return hipErrorInvalidValue;
    }
#undef CSA_SCORE_LAUNCH
    if (e != hipSuccess || fuse) return e;
    return launch("index_merge", index_merge_kernel<FMT, NHB>, dim3(unsigned(int64_t(a.B) * a.Sq)),
                  dim3(kMergeThreads), stream, a);
  } else {
    return hipErrorInvalidValue;
  }
}

}  // namespace

IndexPlan plan_index(int64_t B, int64_t Sq, int64_t N_cap, int topk, int format, bool shared_tiles) {
  IndexPlan p;
  const int64_t n_queries = B * Sq;
  // many queries per sequence (a prefill chunk) with quantised keys: tiles of 512 shared by eight
  // queries (index_score_multi_kernel)
  p.multi = (shared_tiles && format != 0 && Sq >= kMultiQ && N_cap > kMultiTile &&
             N_cap <= int64_t(kMaxCand / 8) * kMultiTile) ? 1 : 0;
  // otherwise quantised keys stream through one workgroup per segment, about one workgroup per CU
  p.stream = (!p.multi && format != 0) ? 1 : 0;
  int tile;
  if (p.multi) {
    tile = kMultiTile;
  } else if (p.stream) {
    const int ch = format == 1 ? chunk_entries<1>() : chunk_entries<2>();
    const int64_t per_cu = (n_queries * N_cap + 255) / 256;
    tile = ch;
    while (tile < kStreamSeg && tile < per_cu && tile < N_cap) tile <<= 1;
  } else {
    tile = kMaxTile;
    while (tile > 64 && n_queries * ((N_cap + tile - 1) / tile) < 512) tile >>= 1;
    while (tile > 64 && tile / 2 >= N_cap) tile >>= 1;
  }
  p.tile = tile;
  p.n_tiles = int((N_cap + tile - 1) / tile);
  // keep ~4x the expected number of winners per tile, within what the merge holds: kFusedSlots in
  // the tile workgroup that merges (kFusedKeys per thread), else kMaxCand in a merge kernel
  int64_t want = (4 * int64_t(topk) * tile + N_cap - 1) / N_cap;
  int cand = 8;
  while (cand < want && cand < tile) cand <<= 1;
  if (cand > tile) cand = tile;
  p.fused = (!p.multi && int64_t(p.n_tiles) * 8 <= kFusedSlots) ? 1 : 0;
  const int64_t max_slots = p.fused ? kFusedSlots : kMaxCand;
  while (int64_t(p.n_tiles) * cand > max_slots && cand > 8) cand >>= 1;
  p.cand = cand;
  return p;
}

size_t index_workspace_bytes(int64_t B, int64_t Sq, int64_t N_cap, int topk, int format, bool shared_tiles) {
  IndexPlan p = plan_index(B, Sq, N_cap, topk, format, shared_tiles);
  if (p.multi) return prepared_query_offset(B * Sq, p) + size_t(B * Sq) * sizeof(QueryLds) + 256;
  return arrivals_offset(B * Sq, p) + size_t(B * Sq) * kCounterStride * 4 + 256;
}

hipError_t launch_query_codes(const uint16_t *q, const float *w, int64_t n, int H_I, int format, void *codes,
                              void *scale_bytes, float *factors, hipStream_t stream) {
  if (format == 1)
    return launch("query_codes", query_codes_kernel<1>, dim3(unsigned(n)), dim3(256), stream, q, w, H_I,
                  static_cast<uint8_t *>(codes), static_cast<uint8_t *>(scale_bytes), factors);
  return launch("query_codes", query_codes_kernel<2>, dim3(unsigned(n)), dim3(256), stream, q, w, H_I,
                static_cast<uint8_t *>(codes), static_cast<uint8_t *>(scale_bytes), factors);
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

}  // namespace csa
