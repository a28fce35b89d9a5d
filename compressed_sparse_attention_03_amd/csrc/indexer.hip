// Lightning indexer and top-k selector.
//
// "DeepSeek-V4: Million-Token Context" (codexsims explainer), CSA walk-through: a small attention
// head scores every compressed block against the current query and a top-k selector keeps only
// the best.  "Follow the white rabbit" (sambatista.com), indexer paragraph: about 262,000 entries
// at the longest context, the top 1,024 pass on; the pass is cheap because it uses smaller
// representations and lower-precision numbers; its work grows with the context.
//
// score[i] = sum_h w[h] * max(0, <q~_h, k~_i>)  (the form stated in csa.h).
//
// Kernel 1 (index_score): grid (tiles, queries), 4 waves.  The query's 64x128 head matrix is
// quantised once per workgroup into LDS and held as MFMA A-operands; key tiles stream from HBM
// in groups of 16 entries, each group costing one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 heads
// (fp8 e4m3, or MXFP4 with its e8m0 block scales applied by the instruction).  The tile's scores
// stay in LDS; a block radix select keeps the tile's `cand` best (score, index) keys, written in
// ascending index order together with the smallest kept key.
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

struct QueryLds {                     // quantised query of one indexer query token
  uint8_t codes[64 * 128];            // fp8: [head][128]; MXFP4: [head][64] packed
  uint8_t sbytes[64 * 4];             // MXFP4 block scales [head][4]
  float f[64];                        // per-head factor: w_h * fp8 scale (w_h for MXFP4)
};

// Quantise one query's [H_I x 128] bf16 heads into LDS.  Threads 0 .. 4*H_I-1 each own 32 values.
template <int FMT>
__device__ void prep_query_lds(const uint16_t *q, const float *w, int H_I, QueryLds &ql) {
  const int t = threadIdx.x;
  if (t < 256) {
    const bool act = t < 4 * H_I;
    const int h = t >> 2, c = t & 3;
    uint32_t wv[16];
    if (act) {
      const uint4 *src = reinterpret_cast<const uint4 *>(q + h * 128 + c * 32);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint4 v = src[k];
        wv[4 * k] = v.x; wv[4 * k + 1] = v.y; wv[4 * k + 2] = v.z; wv[4 * k + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) wv[k] = 0;
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(wv[k])), fabsf(bf16hi(wv[k]))));
    if (FMT == 1) {
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int e = e4m3_row_exp(amax);
      const float inv = ldexpf(1.0f, -e);
      if (act) {
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
        if (c == 0) ql.f[h] = w[h] * ldexpf(1.0f, e);
      }
    } else {
      const uint32_t sb = mx_scale_byte(amax);
      const float inv = ldexpf(1.0f, 127 - int(sb));
      if (act) {
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
        if (c == 0) ql.f[h] = w[h];
      }
    }
  }
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

// Key operand of one lane for the group of 16 entries starting at e0: entry e0 + (lane & 15),
// K-chunk (lane >> 4).  Rows past the allocation are clamped (their scores are discarded).
template <int FMT>
struct KeyFrag {
  v8i b;
  int sb;
  float ks;
};

template <int FMT>
__device__ __forceinline__ void load_key_frag(const uint8_t *codes, const void *scales, int64_t row,
                                              int lane, KeyFrag<FMT> &kf) {
  const int g = lane >> 4;
  if (FMT == 1) {
    const uint4 *p = reinterpret_cast<const uint4 *>(codes + row * 128 + g * 32);
    uint4 x0 = p[0], x1 = p[1];
    kf.b = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
    kf.sb = 127;
    kf.ks = static_cast<const float *>(scales)[row];
  } else {
    uint4 x0 = *reinterpret_cast<const uint4 *>(codes + row * 64 + g * 16);
    kf.b = v8i{int(x0.x), int(x0.y), int(x0.z), int(x0.w), 0, 0, 0, 0};
    uint32_t s4 = static_cast<const uint32_t *>(scales)[row];
    kf.sb = int((s4 >> (8 * g)) & 0xff);
    kf.ks = 1.0f;
  }
}

// Score of entry (e0 + lane%16) for every lane (the 4 lanes of one entry agree).
template <int FMT, int NHB>
__device__ __forceinline__ float score_group(const QueryFrag<NHB> &qf, const KeyFrag<FMT> &kf) {
  constexpr int fmt = FMT == 1 ? 0 : 4;   // instruction format code: 0 = fp8 e4m3, 4 = fp4 e2m1
  float acc = 0.f;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf.a[hb], kf.b, c, fmt, fmt, 0, qf.sa[hb], 0, kf.sb);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc += qf.f[hb][v] * fmaxf(c[v], 0.f);
  }
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  return acc * kf.ks;
}

// Score `tile` entries starting at entry e_begin into s_scores (LDS) -- quantised formats.
// Invisible entries (>= n_vis) are written as -inf.  Work is split over all waves of the block.
template <int FMT, int NHB>
__device__ void score_tile_mfma(const QueryFrag<NHB> &qf, const uint8_t *codes, const void *scales,
                                int64_t row_base, int64_t N_cap, int64_t e_begin, int tile,
                                int64_t n_vis, float *s_scores) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int ngroups = tile >> 4;
  constexpr int U = 4;
  for (int g0 = wave * U; g0 < ngroups; g0 += nwaves * U) {
    KeyFrag<FMT> kf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t e = e_begin + int64_t(g0 + u) * 16 + (lane & 15);
      int64_t row = e < N_cap ? e : N_cap - 1;
      load_key_frag<FMT>(codes, scales, row_base + row, lane, kf[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u < ngroups) {
        float s = score_group<FMT, NHB>(qf, kf[u]);
        int64_t e = e_begin + int64_t(g0 + u) * 16 + (lane & 15);
        if (lane < 16) s_scores[(g0 + u) * 16 + lane] = e < n_vis ? s : -INFINITY;
      }
    }
  }
}

// fp32 keys: one thread per entry, query heads from LDS.
__device__ void score_tile_f32(const float *q_lds, const float *w, int H_I, int D_I, const float *keys,
                               int64_t row_base, int64_t e_begin, int tile, int64_t n_vis,
                               float *s_scores) {
  for (int i = threadIdx.x; i < tile; i += blockDim.x) {
    const int64_t e = e_begin + i;
    float s = -INFINITY;
    if (e < n_vis) {
      const float4 *kr = reinterpret_cast<const float4 *>(keys + (row_base + e) * D_I);
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

// ---- block-wide helpers -----------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix over the block of one int per thread; returns (prefix, total).
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *s_tmp, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = NT / 64;
  int incl = wave_incl_scan(v, lane);
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int x = s_tmp[w];
    base += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = __shfl_xor(uint32_t(v), o, 64), hi = __shfl_xor(uint32_t(v >> 32), o, 64);
  return (uint64_t(hi) << 32) | lo;
}

// Rank-`need` (1 = largest) key among the non-zero keys held by the block (KPT per thread).
// Keys are distinct.  The caller guarantees 1 <= need <= number of non-zero keys.
template <int NT, int KPT>
__device__ uint64_t block_select(const uint64_t (&keys)[KPT], int need, uint32_t *s_hist,
                                 uint64_t *s_u64, int *s_sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix = 0, mask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if (keys[k] != 0 && (keys[k] & mask) == prefix) atomicAdd(&s_hist[(keys[k] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = int(s_hist[255 - 4 * lane - j]); sum += c[j]; }
      int cum = wave_incl_scan(sum, lane) - sum;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (cum < need && need <= cum + c[j]) {
          s_sel[0] = 255 - 4 * lane - j;
          s_sel[1] = cum;
          s_sel[2] = c[j];
        }
        cum += c[j];
      }
    }
    __syncthreads();
    const uint64_t digit = uint64_t(s_sel[0]);
    need -= s_sel[1];
    const int bucket = s_sel[2];
    prefix |= digit << shift;
    mask |= uint64_t(255) << shift;
    __syncthreads();
    if (bucket == need) {
      // every key of this bucket is in; the answer is the smallest of them
      uint64_t mn = ~uint64_t(0);
#pragma unroll
      for (int k = 0; k < KPT; ++k)
        if (keys[k] != 0 && (keys[k] & mask) == prefix && keys[k] < mn) mn = keys[k];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        uint64_t t = shfl_xor_u64(mn, o);
        mn = t < mn ? t : mn;
      }
      if (lane == 0) s_u64[wave] = mn;
      __syncthreads();
      uint64_t r = ~uint64_t(0);
      for (int w = 0; w < NT / 64; ++w) r = s_u64[w] < r ? s_u64[w] : r;
      __syncthreads();
      return r;
    }
  }
  return prefix;
}

// ---- kernel 1: scores and per-tile candidates ------------------------------------------------
struct ScoreShared {
  QueryLds ql;
  float scores[kMaxTile];
  uint32_t hist[256];
  uint64_t u64[16];
  int sel[4];
  int tmp[16];
};

template <int FMT, int NHB, int KPT>
__global__ void __launch_bounds__(256) index_score_kernel(IndexArgs a) {
  __shared__ ScoreShared sh;
  const int tile_id = blockIdx.x;
  const int64_t qi = blockIdx.y;                               // query = b * Sq + s
  const int b = int(qi / a.Sq), s = int(qi % a.Sq);
  const int tile = a.plan.tile, cand = a.plan.cand;
  const int64_t e_begin = int64_t(tile_id) * tile;
  const int64_t t = a.q_pos0[b] + s;
  const int64_t n_vis = min(a.n_entries[b], (t + 1) / a.m);
  const int64_t out_slot = qi * a.plan.n_tiles + tile_id;
  uint64_t *cand_keys = static_cast<uint64_t *>(a.workspace);
  uint64_t *cand_bound = cand_keys + int64_t(gridDim.y) * a.plan.n_tiles * cand;
  int *cand_count = reinterpret_cast<int *>(cand_bound + int64_t(gridDim.y) * a.plan.n_tiles);

  if (e_begin >= n_vis && a.scores == nullptr) {              // nothing visible in this tile
    if (threadIdx.x == 0) { cand_count[out_slot] = 0; cand_bound[out_slot] = 0; }
    return;
  }
  const int64_t row_base = int64_t(b) * a.N_cap;
  if (FMT == 0) {
    float *q_lds = reinterpret_cast<float *>(sh.ql.codes);    // H_I * D_I <= 2048 floats
    const float *qsrc = static_cast<const float *>(a.q_idx) + qi * a.H_I * a.D_I;
    for (int i = threadIdx.x; i < a.H_I * a.D_I; i += blockDim.x) q_lds[i] = qsrc[i];
    if (threadIdx.x < a.H_I) sh.ql.f[threadIdx.x] = a.w_idx[qi * a.H_I + threadIdx.x];
    __syncthreads();
    score_tile_f32(q_lds, sh.ql.f, a.H_I, a.D_I, static_cast<const float *>(a.k_codes), row_base,
                   e_begin, tile, n_vis, sh.scores);
  } else {
    prep_query_lds<FMT>(static_cast<const uint16_t *>(a.q_idx) + qi * a.H_I * 128, a.w_idx + qi * a.H_I,
                        a.H_I, sh.ql);
    __syncthreads();
    QueryFrag<NHB> qf;
    load_query_frag<FMT, NHB>(sh.ql, threadIdx.x & 63, qf);
    score_tile_mfma<FMT, NHB>(qf, static_cast<const uint8_t *>(a.k_codes), a.k_scales, row_base, a.N_cap,
                              e_begin, tile, n_vis, sh.scores);
  }
  __syncthreads();
  if (a.scores) {
    float *dst = a.scores + qi * a.N_cap;
    for (int i = threadIdx.x; i < tile; i += blockDim.x)
      if (e_begin + i < a.N_cap) dst[e_begin + i] = sh.scores[i];
  }
  // keys of this thread's KPT consecutive entries
  uint64_t keys[KPT];
  int nvalid_local = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = threadIdx.x * KPT + k;
    const int64_t e = e_begin + i;
    const bool ok = i < tile && e < n_vis;
    keys[k] = ok ? make_key(sh.scores[i], uint32_t(e)) : 0;
    nvalid_local += ok;
  }
  int nvalid;
  (void)block_excl_scan<256>(nvalid_local, sh.tmp, nvalid);
  uint64_t bound = 0;
  if (nvalid > cand) bound = block_select<256, KPT>(keys, cand, sh.hist, sh.u64, sh.sel);
  int mine = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) mine += (keys[k] != 0 && keys[k] >= bound);
  int total;
  int pos = block_excl_scan<256>(mine, sh.tmp, total);
  uint64_t *dst = cand_keys + out_slot * cand;
#pragma unroll
  for (int k = 0; k < KPT; ++k)
    if (keys[k] != 0 && keys[k] >= bound) dst[pos++] = keys[k];
  if (threadIdx.x == 0) { cand_count[out_slot] = total; cand_bound[out_slot] = bound; }
}

// ---- kernel 2: merge ----------------------------------------------------------------------
struct MergeShared {
  QueryLds ql;
  float scores[kMaxTile];
  uint64_t work[kMaxK + kMaxTile];
  int counts[kMaxCand / 8];
  uint64_t bounds[kMaxCand / 8];
  uint32_t hist[256];
  uint64_t u64[16];
  int sel[4];
  int tmp[16];
  int flag;
};

// Sort `n` (<= kMaxK, padded to a power of two P) entry indices ascending, in LDS (as keys).
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
      __syncthreads();
    }
  }
}

template <int FMT, int NHB>
__global__ void __launch_bounds__(kMergeThreads) index_merge_kernel(IndexArgs a) {
  __shared__ MergeShared sh;
  constexpr int KPT = kMaxCand / kMergeThreads;
  const int tid = threadIdx.x;
  const int64_t qi = blockIdx.x;
  const int b = int(qi / a.Sq), s = int(qi % a.Sq);
  const int tile = a.plan.tile, cand = a.plan.cand, n_tiles = a.plan.n_tiles;
  const int64_t t = a.q_pos0[b] + s;
  const int64_t n_vis = min(a.n_entries[b], (t + 1) / a.m);
  const int k_eff = int(min(int64_t(a.topk), n_vis));
  const uint64_t *cand_keys = static_cast<const uint64_t *>(a.workspace);
  const uint64_t *cand_bound = cand_keys + int64_t(gridDim.x) * n_tiles * cand;
  const int *cand_count = reinterpret_cast<const int *>(cand_bound + int64_t(gridDim.x) * n_tiles);
  int32_t *out = a.topk_idx + qi * a.topk;

  for (int i = tid; i < n_tiles; i += kMergeThreads) {
    sh.counts[i] = cand_count[qi * n_tiles + i];
    sh.bounds[i] = cand_bound[qi * n_tiles + i];
  }
  __syncthreads();
  uint64_t keys[KPT];
  int nvalid_local = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int slot = tid * KPT + k;
    const int tl = slot / cand, j = slot - tl * cand;
    uint64_t key = 0;
    if (tl < n_tiles && j < sh.counts[tl]) key = cand_keys[(qi * n_tiles + tl) * cand + j];
    keys[k] = key;
    nvalid_local += key != 0;
  }
  int nvalid;
  (void)block_excl_scan<kMergeThreads>(nvalid_local, sh.tmp, nvalid);
  if (k_eff == 0) {
    for (int i = tid; i < a.topk; i += kMergeThreads) out[i] = -1;
    return;
  }
  uint64_t tau = 0;                                            // k-th best candidate (0: need all)
  if (nvalid >= k_eff) tau = block_select<kMergeThreads, KPT>(keys, k_eff, sh.hist, sh.u64, sh.sel);
  // a truncated tile whose smallest kept key beats tau may hold further winners
  if (tid == 0) sh.flag = 0;
  __syncthreads();
  for (int i = tid; i < n_tiles; i += kMergeThreads)
    if (sh.bounds[i] != 0 && sh.bounds[i] > tau) sh.flag = 1;
  __syncthreads();
  if (!sh.flag) {
    int mine = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) mine += (keys[k] != 0 && keys[k] >= tau);
    int total;
    int pos = block_excl_scan<kMergeThreads>(mine, sh.tmp, total);
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if (keys[k] != 0 && keys[k] >= tau) out[pos++] = int32_t(key_index(keys[k]));
    for (int i = k_eff + tid; i < a.topk; i += kMergeThreads) out[i] = -1;
    return;
  }

  // ---- exact fallback: working set W (<= k_eff keys) in LDS, re-score each suspicious tile ----
  int wn;
  {
    int mine = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) mine += (keys[k] != 0 && keys[k] >= tau);
    int pos = block_excl_scan<kMergeThreads>(mine, sh.tmp, wn);
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if (keys[k] != 0 && keys[k] >= tau) sh.work[pos++] = keys[k];
  }
  __syncthreads();
  QueryFrag<NHB> qf;
  float *q_lds = reinterpret_cast<float *>(sh.ql.codes);
  if (FMT == 0) {
    const float *qsrc = static_cast<const float *>(a.q_idx) + qi * a.H_I * a.D_I;
    for (int i = tid; i < a.H_I * a.D_I; i += kMergeThreads) q_lds[i] = qsrc[i];
    if (tid < a.H_I) sh.ql.f[tid] = a.w_idx[qi * a.H_I + tid];
    __syncthreads();
  } else {
    prep_query_lds<FMT>(static_cast<const uint16_t *>(a.q_idx) + qi * a.H_I * 128, a.w_idx + qi * a.H_I,
                        a.H_I, sh.ql);
    __syncthreads();
    load_query_frag<FMT, NHB>(sh.ql, tid & 63, qf);
  }
  const int64_t row_base = int64_t(b) * a.N_cap;
  constexpr int KW = (kMaxK + kMaxTile) / kMergeThreads;
  for (int tl = 0; tl < n_tiles; ++tl) {
    const uint64_t bt = sh.bounds[tl];
    if (bt == 0 || bt <= tau) continue;                        // complete, or cannot hold winners
    const int64_t e_begin = int64_t(tl) * tile;
    if (FMT == 0)
      score_tile_f32(q_lds, sh.ql.f, a.H_I, a.D_I, static_cast<const float *>(a.k_codes), row_base,
                     e_begin, tile, n_vis, sh.scores);
    else
      score_tile_mfma<FMT, NHB>(qf, static_cast<const uint8_t *>(a.k_codes), a.k_scales, row_base,
                                a.N_cap, e_begin, tile, n_vis, sh.scores);
    __syncthreads();
    // append the tile's entries below its bound (the ones not already candidates) and above tau
    int mine = 0;
    for (int i = tid; i < tile; i += kMergeThreads) {
      const int64_t e = e_begin + i;
      if (e < n_vis) {
        uint64_t key = make_key(sh.scores[i], uint32_t(e));
        mine += (key < bt && key > tau);
      }
    }
    int total;
    int pos = block_excl_scan<kMergeThreads>(mine, sh.tmp, total) + wn;
    for (int i = tid; i < tile; i += kMergeThreads) {
      const int64_t e = e_begin + i;
      if (e < n_vis) {
        uint64_t key = make_key(sh.scores[i], uint32_t(e));
        if (key < bt && key > tau) sh.work[pos++] = key;
      }
    }
    wn += total;
    __syncthreads();
    if (wn > k_eff) {                                           // shrink W back to the k_eff best
      uint64_t wk[KW];
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const int i = tid * KW + k;
        wk[k] = i < wn ? sh.work[i] : 0;
      }
      __syncthreads();
      tau = block_select<kMergeThreads, KW>(wk, k_eff, sh.hist, sh.u64, sh.sel);
      int m2 = 0;
#pragma unroll
      for (int k = 0; k < KW; ++k) m2 += (wk[k] != 0 && wk[k] >= tau);
      int tot2;
      int p2 = block_excl_scan<kMergeThreads>(m2, sh.tmp, tot2);
#pragma unroll
      for (int k = 0; k < KW; ++k)
        if (wk[k] != 0 && wk[k] >= tau) sh.work[p2++] = wk[k];
      wn = tot2;
      __syncthreads();
    } else if (wn == k_eff && tau == 0) {
      // W just reached k_eff: its smallest key is the new threshold
      uint64_t wk[KW];
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const int i = tid * KW + k;
        wk[k] = i < wn ? sh.work[i] : 0;
      }
      __syncthreads();
      tau = block_select<kMergeThreads, KW>(wk, k_eff, sh.hist, sh.u64, sh.sel);
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
  __syncthreads();
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int i = tid * KW + k;
    if (i < P) idx[i] = tmpv[k];
  }
  __syncthreads();
  bitonic_sort_u32(idx, P);
  for (int i = tid; i < a.topk; i += kMergeThreads) out[i] = i < wn ? int32_t(idx[i]) : -1;
}

template <int FMT, int NHB>
hipError_t launch_score_t(const IndexArgs &a, hipStream_t stream) {
  dim3 grid(unsigned(a.plan.n_tiles), unsigned(int64_t(a.B) * a.Sq));
  switch (a.plan.tile / 256) {
    case 0: hipLaunchKernelGGL((index_score_kernel<FMT, NHB, 1>), grid, dim3(256), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((index_score_kernel<FMT, NHB, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((index_score_kernel<FMT, NHB, 2>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((index_score_kernel<FMT, NHB, 4>), grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((index_score_kernel<FMT, NHB, 8>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, int NHB>
hipError_t launch_merge_t(const IndexArgs &a, hipStream_t stream) {
  dim3 grid(unsigned(int64_t(a.B) * a.Sq));
  hipLaunchKernelGGL((index_merge_kernel<FMT, NHB>), grid, dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

IndexPlan plan_index(int64_t n_queries, int64_t N_cap, int topk) {
  IndexPlan p;
  int tile = kMaxTile;
  while (tile > 64 && n_queries * ((N_cap + tile - 1) / tile) < 512) tile >>= 1;
  while (tile > 64 && tile / 2 >= N_cap) tile >>= 1;
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

size_t index_workspace_bytes(int64_t n_queries, int64_t N_cap, int topk) {
  IndexPlan p = plan_index(n_queries, N_cap, topk);
  const int64_t slots = n_queries * p.n_tiles;
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
  const int nhb = a.H_I / 16;
  if (a.format == 0) return launch_merge_t<0, 1>(a, stream);
  if (a.format == 1) {
    switch (nhb) {
      case 1: return launch_merge_t<1, 1>(a, stream);
      case 2: return launch_merge_t<1, 2>(a, stream);
      case 3: return launch_merge_t<1, 3>(a, stream);
      case 4: return launch_merge_t<1, 4>(a, stream);
    }
  } else {
    switch (nhb) {
      case 1: return launch_merge_t<2, 1>(a, stream);
      case 2: return launch_merge_t<2, 2>(a, stream);
      case 3: return launch_merge_t<2, 3>(a, stream);
      case 4: return launch_merge_t<2, 4>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace csa
