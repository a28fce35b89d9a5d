// Internal launcher interface between the C-ABI front (api.cpp) and the kernel sources.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

struct CompressArgs {
  const uint16_t *c, *z, *bias, *norm_w;
  uint16_t *entries, *win_rows;
  int B, d, m, overlap, rope_dim, halo;
  int64_t n_new, pos0;
  double log2_base;
  float eps;
  // indexer keys (launch_compress_keys): pooled only, rounded to bf16 (entries: optional bf16
  // copy) and quantised into k_codes / k_scales in key_format
  int key_format;
  void *k_codes, *k_scales;
};
hipError_t launch_compress(const CompressArgs &a, hipStream_t stream);
hipError_t launch_compress_keys(const CompressArgs &a, hipStream_t stream);

// Decode-time cache maintenance: one new token per sequence (see csa_decode_append).
struct AppendArgs {
  const uint16_t *c_new, *z_new, *k_new, *bias, *norm_w;
  const int64_t *pos;
  uint16_t *tok_c, *tok_z, *win_ring, *entries;
  void *k_codes, *k_scales;
  int64_t *n_entries;
  int64_t W_cap, N_cap;
  int B, d, m, overlap, rope_dim, key_format, D_I;
  double log2_base;
  float eps;
};
hipError_t launch_append(const AppendArgs &a, hipStream_t stream);
// the indexer stream's ring and keys (d = D_I; entries: optional bf16 keys [B, N_cap, D_I])
hipError_t launch_append_keys(const AppendArgs &a, hipStream_t stream);
// both streams in one launch (a: the KV stream, d in 128..1024; ai: the indexer stream)
hipError_t launch_append_step(const AppendArgs &a, const AppendArgs &ai, hipStream_t stream);

struct QuantizeArgs {
  const uint16_t *x;
  void *codes, *scales;
  int64_t rows;
  int dim, format;
};
hipError_t launch_quantize(const QuantizeArgs &a, hipStream_t stream);

// ---- lightning indexer + top-k -------------------------------------------------------------
// The entry axis of every query is cut into tiles of `tile` entries.  The score kernel keeps, per
// tile, the `cand` best (score, index) keys; the merge selects the global top-k among all tiles'
// candidates and re-scores any tile whose candidate list might have been too short.
struct IndexPlan {
  int tile;        // entries per tile (multiple of 64)
  int cand;        // candidates kept per tile (power of two, <= tile)
  int n_tiles;     // tiles per query
  int multi;       // tiles shared by eight queries of a sequence (prefill-sized calls)
  int stream;      // quantised keys: one workgroup streams a segment of `tile` entries of a query
  int fused;       // one query per tile workgroup, merged by the query's last tile workgroup
};
// shared_tiles: allow the shared-tile path (it does not write full scores)
IndexPlan plan_index(int64_t B, int64_t Sq, int64_t N_cap, int topk, int format, bool shared_tiles);
size_t index_workspace_bytes(int64_t B, int64_t Sq, int64_t N_cap, int topk, int format, bool shared_tiles);

struct IndexArgs {
  const void *q_idx;
  const float *w_idx;
  const void *k_codes, *k_scales;
  const int64_t *n_entries, *q_pos0;
  int32_t *topk_idx;
  float *scores;
  void *workspace;
  int format, B, Sq, H_I, D_I, m, topk;
  int64_t N_cap;
  IndexPlan plan;
};
// Every kernel of the call: the score kernel (which, on the one-query path, also merges each
// query's candidates in its last tile workgroup), or on the shared-tile path the query
// quantisation, the shared-tile score kernel and the merge kernel.  The workspace must hold zeros
// where the arrival counters live before the first call; every call leaves them at zero.
hipError_t launch_index_score(const IndexArgs &a, hipStream_t stream);
// The indexer's query encoding alone (csa_quantize_query).
hipError_t launch_query_codes(const uint16_t *q, const float *w, int64_t n, int H_I, int format, void *codes,
                              void *scale_bytes, float *factors, hipStream_t stream);

// ---- grouped output projection --------------------------------------------------------------
struct ProjArgs {
  const uint16_t *o, *w;            // [M, ldo] head outputs; [G, N_g, K_g] weights
  uint16_t *y;                      // [M, ldy]
  int M, G, N_g, K_g;
  int64_t ldo, ldy;
};
hipError_t launch_oproj(const ProjArgs &a, hipStream_t stream);

// ---- core attention ------------------------------------------------------------------------
struct AttendPlan {
  int n_hb;         // head blocks of 16
  int n_splits;     // row splits per (query, head block); a function of n_rows only
  int rows_per_split;
  int n_rows;       // row-list length per query: n_sel + window
  int fused;        // one workgroup per (query, head block) merges every split (many queries)
};
AttendPlan plan_attend(int64_t n_queries, int H, int64_t n_sel, int window, int D);
size_t attend_workspace_bytes(int64_t n_queries, int H, int D, int64_t n_sel, int window);

struct AttendArgs {
  const uint16_t *q, *q_norm_w, *entries, *win_rows;
  const int32_t *topk_idx;          // CSA selection, or NULL for HCA (dense prefix)
  const int64_t *n_entries;         // HCA only
  const int64_t *win_pos0, *q_pos0;
  uint16_t *out;
  float *lse;
  void *workspace;
  int64_t N_cap, W_cap;
  int64_t n_sel;                    // CSA: topk; HCA: N_cap
  int B, Sq, H, D, rope_dim, window, m;
  float scale_log2;                 // softmax_scale * log2(e)
  double log2_base;
  float eps;
  AttendPlan plan;
};
hipError_t launch_attend(const AttendArgs &a, hipStream_t stream);
hipError_t launch_combine(const AttendArgs &a, hipStream_t stream);
// The library's scratch array for csa_attend_noalloc: its size, and its device address on the
// current device (looked up once per device).
size_t attend_scratch_bytes();
hipError_t attend_scratch(void **ptr);

// Plain streaming read of `bytes` (a positive multiple of 16) at `src` (measure.hip).
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);

// Kernel timing (api.cpp).  When timing is on, timing_events hands out a start/stop event pair
// filed under `name`; launch() then passes them in the kernel's own dispatch, so they take the
// kernel's start and end timestamps (no separate marker packets around it).
struct TimingEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
TimingEvents timing_events(const char *name);

template <typename F, typename... Args>
hipError_t launch(const char *name, F kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  const TimingEvents t = timing_events(name);
  if (t.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t.start, t.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  return hipGetLastError();
}

}  // namespace csa
