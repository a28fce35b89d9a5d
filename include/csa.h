/*
 * csa.h -- C ABI of libcsa, an MI355X (gfx950) implementation of the hybrid compressed attention
 * forward pass: CSA (compressed sparse attention) and HCA (heavily compressed attention).
 *
 * The operations follow these pages (cited by title and section):
 *   [EXPLAINER] "DeepSeek-V4: Million-Token Context" (codexsims.com explainer): the CSA
 *               walk-through (compressor, lightning indexer, top-k selector, core attention plus
 *               sliding window) and the HCA walk-through (128-token windows, dense attention).
 *   [DEVTO]     "How DeepSeek-V4 Achieves Million-Token Contexts Without Quadratic Attention
 *               Costs" (dev.to), section "Two Compression Strategies: CSA and HCA".
 *   [SUMMARY]   "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence"
 *               (paperlayer.ai summary), section 2.3 "Hybrid Attention with CSA and HCA".
 *   [RABBIT]    "Follow the white rabbit: DeepSeek V4's architecture in 3D" (sambatista.com),
 *               paragraphs on HCA, CSA, the sliding window and the lightning indexer.
 *
 * Conventions for every call:
 *   - Pointers to tensors are DEVICE pointers owned by the caller.  The library never allocates,
 *     frees or keeps a pointer after the call returns.  Scalars are passed by value; the few
 *     per-sequence integers (positions, entry counts) are device arrays of int64.
 *   - Tensors are row-major and contiguous.  bf16 tensors are passed as uint16_t bit patterns.
 *     Every tensor base pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  A call validates its
 *     arguments on the host, enqueues its kernels on `stream` and returns without synchronising.
 *   - Errors: a call returns a csa_status.  Argument errors (CSA_ERR_INVALID, CSA_ERR_UNSUPPORTED,
 *     CSA_ERR_WORKSPACE) are detected before any HIP call, so nothing is enqueued.  CSA_ERR_HIP
 *     reports a failed launch.  Faults inside a kernel surface at the caller's next
 *     synchronisation.  csa_last_error() returns a thread-local message naming the argument.
 *   - Values inside device arrays (positions, counts, indices) cannot be checked on the host
 *     without a synchronisation; out-of-range values are undefined behaviour.
 *   - Workspace is caller-provided device memory of at least the size the matching
 *     *_workspace_bytes() function returns; two calls that run concurrently must not share it.
 *     It must be zero-filled once before its first use: it holds counters through which the
 *     last workgroup of a query learns that the others are done, and every completed call leaves
 *     them at zero again (a call that was launched but did not complete -- a fault -- may leave
 *     them non-zero: zero the workspace again before reusing it).  csa_index_topk keeps its
 *     counters after its candidate arrays, at an offset that depends on B * Sq, N_cap, topk and
 *     key_format (and on whether scores are asked for): zero its workspace again before a call
 *     that differs in any of these.
 *   - Results are deterministic: fixed reduction orders, no floating-point atomics.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_INVALID = 1,     /* an argument is out of its documented range; nothing enqueued */
  CSA_ERR_UNSUPPORTED = 2, /* a valid shape or format the library has no kernel for; nothing enqueued */
  CSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required; nothing enqueued */
  CSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} csa_status;

/* Storage format of the lightning-indexer keys (and the rule used for the query). */
typedef enum csa_key_format {
  CSA_KEY_F32 = 0,      /* fp32 keys [rows, D_I]; the query is used as fp32 (no quantisation) */
  CSA_KEY_FP8_E4M3 = 1, /* e4m3 codes [rows, D_I] (uint8) + one fp32 power-of-two scale per row */
  CSA_KEY_MXFP4 = 2     /* OCP MXFP4: e2m1 codes packed two per byte [rows, D_I/2] (element 2j in
                           the low nibble) + one e8m0 scale byte per 32 values [rows, D_I/32] */
} csa_key_format;

/*
 * csa_compress -- the KV compressor.
 * [EXPLAINER] CSA walk-through: every m tokens become one entry through a learned softmax
 * weighting; [RABBIT] CSA paragraph: an entry's pooling reaches back over the preceding group as
 * well; [EXPLAINER] HCA walk-through: HCA pools disjoint runs of m' = 128 tokens; [SUMMARY] 2.3 "Other details": RMSNorm
 * on the compressed entries; [DEVTO] partial RoPE.
 *
 * For entry i and channel j the weights are a softmax over the entry's tokens of
 * z[t,j] + bias[slot(t), j]; the pooled value sum_t w[t,j] c[t,j] is RMS-normalised (weight
 * norm_w, eps) and then rotated on its last rope_dim channels at position i*m (interleaved pairs,
 * angle pos * rope_base^(-2u/rope_dim)).  With overlap the entry spans tokens (i-1)m .. (i+1)m-1;
 * bias rows 0..m-1 act on the previous group and m..2m-1 on the own group; entry 0 (no previous
 * group) takes the softmax over its own m tokens only.  Without overlap it spans i*m .. (i+1)m-1.
 *
 *   c, z     bf16 [B, halo + n_new, d]: token rows for positions pos0-halo .. pos0+n_new-1.
 *   bias     bf16 [(1+overlap)*m, d].
 *   norm_w   bf16 [d] RMSNorm weight, or NULL for ones.
 *   halo     must be m when overlap && pos0 > 0, else 0.
 *   pos0     position of the first new token; pos0 % m == 0; n_new % m == 0.
 *   entries  out bf16 [B, n_new/m, d]: entries pos0/m .. (pos0+n_new)/m - 1.
 *   win_rows out bf16 [B, n_new, d] or NULL: each new token's row RMS-normalised (norm_w) and
 *            rotated at its own position -- the rows the sliding window attends to.
 * Limits: d in {64, 128, 256, 512, 1024}; 1 <= m <= 1024; rope_dim % 4 == 0, rope_dim <= d; eps > 0.
 */
csa_status csa_compress(const uint16_t *c, const uint16_t *z, const uint16_t *bias,
                        const uint16_t *norm_w, int B, int64_t n_new, int halo, int d, int m,
                        int overlap, int rope_dim, int64_t pos0, float rope_base, float eps,
                        uint16_t *entries, uint16_t *win_rows, void *stream);

/*
 * csa_decode_append -- decode-time cache maintenance: one new token per sequence.
 * [EXPLAINER] CSA walk-through: the compressed store gains one entry per m tokens (HCA
 * walk-through: per m' = 128 tokens); [RABBIT] sliding-window paragraph: the newest tokens are
 * also kept as separate rows, and tokens of an unfinished group belong to no entry yet; [RABBIT]
 * indexer paragraph, [DEVTO] "Two Compression Strategies": the indexer keys are kept in low
 * precision (quantised when written).
 *
 * For sequence b with its new token at position t = pos[b] (tokens arrive in position order):
 *   - the token's c, z rows are kept in the compressor's token ring: rows t mod R of
 *     tok_c / tok_z [B, R, d], R = (1 + overlap) * m;
 *   - its window row (RMSNorm with norm_w, RoPE at t; as csa_compress's win_rows) is written to
 *     win_ring [B, W_cap, d] at row t mod W_cap -- the ring csa_attend / hca_attend read when
 *     given win_pos0 = NULL;
 *   - when t + 1 is a multiple of m, entry i = (t+1)/m - 1 is complete: it is pooled from the
 *     ring exactly as csa_compress defines it (bias slots, overlap, entry 0 alone), normalised,
 *     rotated at i*m and written to entries[b, i]; k_new[b] (its indexer key, bf16 [B, D_I]) is
 *     quantised by csa_quantize_keys's rule for key_format (CSA_KEY_F32: copied as fp32) into
 *     k_codes / k_scales row (b, i); n_entries[b] becomes i + 1.  Entries at i >= N_cap are
 *     dropped.  k_new NULL keeps no indexer keys (HCA).
 *   c_new, z_new  bf16 [B, d] the new token's compressor inputs.
 *   pos           device int64 [B]; a negative position leaves that sequence untouched.
 *   k_codes       [B, N_cap, D_I] fp32 | [B, N_cap, D_I] e4m3 | [B, N_cap, D_I/2] e2m1 pairs;
 *   k_scales      NULL | fp32 [B, N_cap] | e8m0 [B, N_cap, D_I/32].
 *   n_entries     device int64 [B], written when an entry completes.
 * The caches are device memory owned by the caller; the ring rows of positions before the first
 * appended token are never read when the sequence starts at position 0.
 * Limits: d in {64, 128, 256, 512, 1024}; 1 <= m <= 1024; rope_dim % 4 == 0; D_I a multiple of
 * 32 in [32, 1024]; W_cap, N_cap in [1, 2^31).
 */
csa_status csa_decode_append(const uint16_t *c_new, const uint16_t *z_new, const uint16_t *k_new,
                             const int64_t *pos, const uint16_t *bias, const uint16_t *norm_w, int B,
                             int d, int m, int overlap, int rope_dim, float rope_base, float eps,
                             uint16_t *tok_c, uint16_t *tok_z, uint16_t *win_ring, int64_t W_cap,
                             uint16_t *entries, int64_t N_cap, int key_format, int D_I, void *k_codes,
                             void *k_scales, int64_t *n_entries, void *stream);

/*
 * csa_compress_index_keys -- lightning-indexer keys produced by compression, quantised on write.
 * [EXPLAINER] CSA walk-through: the indexer rates compressed blocks, each pooled from its group of
 * tokens with learned softmax weights; [RABBIT] indexer paragraph: the indexer's operands are
 * compact and low-precision.
 *
 * A per-token indexer stream c_i with logits z_i and bias bias_i is pooled exactly as
 * csa_compress pools (same groups, overlap, bias slots, entry 0 alone), with no RMSNorm and no
 * rotation.  Each pooled key is rounded to bf16 (written to keys_out when given) and quantised by
 * csa_quantize_keys's rule for key_format (CSA_KEY_F32: stored as fp32).
 *   c_i, z_i   bf16 [B, halo + n_new, D_I]; bias_i bf16 [(1+overlap)*m, D_I]; halo, pos0, n_new as
 *              csa_compress.
 *   keys_out   bf16 [B, n_new/m, D_I] or NULL.
 *   k_codes, k_scales  the keys of entries pos0/m .. in key_format: rows [B, n_new/m] of the
 *              layouts of csa_quantize_keys (fp32: codes fp32 [B, n_new/m, D_I], scales unused).
 * Limits: D_I in {128, 256, 512, 1024}; 1 <= m <= 1024.
 */
csa_status csa_compress_index_keys(const uint16_t *c_i, const uint16_t *z_i, const uint16_t *bias_i, int B,
                                   int64_t n_new, int halo, int D_I, int m, int overlap, int64_t pos0,
                                   int key_format, uint16_t *keys_out, void *k_codes, void *k_scales,
                                   void *stream);

/*
 * csa_decode_append_index -- the indexer stream's part of decode-time cache maintenance.
 * As csa_decode_append for the per-token indexer stream: the new token's c_i, z_i rows go to
 * the stream's ring tok_c / tok_z [B, (1+overlap)*m, D_I] at row t mod ring size; when t + 1
 * completes entry i = (t+1)/m - 1 its key is pooled from the ring as csa_compress_index_keys
 * pools it, rounded to bf16 (keys_out [B, N_cap, D_I] row (b, i) when given) and quantised into
 * k_codes / k_scales row (b, i) ([B, N_cap] rows).  n_entries is left to csa_decode_append.
 * Limits as csa_compress_index_keys; pos < 0 leaves a sequence untouched.
 */
csa_status csa_decode_append_index(const uint16_t *c_i_new, const uint16_t *z_i_new, const int64_t *pos,
                                   const uint16_t *bias_i, int B, int D_I, int m, int overlap, uint16_t *tok_c,
                                   uint16_t *tok_z, int64_t N_cap, int key_format, uint16_t *keys_out,
                                   void *k_codes, void *k_scales, void *stream);

/*
 * csa_decode_append_step -- a decode step's whole cache maintenance in one launch: the KV
 * stream's part of csa_decode_append and the indexer stream's csa_decode_append_index, side by
 * side (one workgroup per sequence and stream).  [EXPLAINER] CSA walk-through: one new entry per
 * m tokens, and its indexer key, which the lightning indexer rates; [RABBIT] sliding-window and
 * indexer paragraphs.
 * The KV-stream arguments are csa_decode_append's (with no k_new: the closed entry's indexer key
 * is the indexer stream's pooled key); c_i_new, z_i_new, bias_i, D_I, tok_ci, tok_zi, key_format,
 * keys_out, k_codes, k_scales are csa_decode_append_index's (tok_c, tok_z there).  The results are
 * those of the two calls.  pos, m, overlap and N_cap are shared by both streams.
 * Limits: d in {128, 256, 512, 1024}; D_I in {128, 256, 512, 1024}; others as the two calls.
 */
csa_status csa_decode_append_step(const uint16_t *c_new, const uint16_t *z_new, const int64_t *pos,
                                  const uint16_t *bias, const uint16_t *norm_w, int B, int d, int m, int overlap,
                                  int rope_dim, float rope_base, float eps, uint16_t *tok_c, uint16_t *tok_z,
                                  uint16_t *win_ring, int64_t W_cap, uint16_t *entries, int64_t N_cap,
                                  int64_t *n_entries, const uint16_t *c_i_new, const uint16_t *z_i_new,
                                  const uint16_t *bias_i, int D_I, uint16_t *tok_ci, uint16_t *tok_zi,
                                  int key_format, uint16_t *keys_out, void *k_codes, void *k_scales, void *stream);

/*
 * csa_quantize_keys -- quantise lightning-indexer keys to their storage format (quantise on write).
 * [DEVTO] "Two Compression Strategies": the indexer runs in FP4; [RABBIT] indexer paragraph:
 * the indexer works on compact, low-precision operands.
 *
 *   x       bf16 [rows, dim] keys.
 *   format  CSA_KEY_FP8_E4M3: codes uint8 [rows, dim]; scales fp32 [rows] = 2^e, e the smallest
 *           integer with max|row| <= 448 * 2^e (clamped to [-126, 127]; 1.0 for a zero row);
 *           codes = round-to-nearest-even(x / 2^e) in e4m3, saturating at +-448.
 *           CSA_KEY_MXFP4: codes uint8 [rows, dim/2] (two e2m1 codes per byte); scales uint8
 *           [rows, dim/32] e8m0 = clamp(floor(log2 amax) - 2 + 127, 0, 254) (0 for a zero block);
 *           codes = round-to-nearest-even(x / 2^(scale-127)) in e2m1, saturating at +-6.
 *           Zero magnitudes keep the sign bit of the input.
 * Limits: dim % 32 == 0, dim <= 1024.  CSA_KEY_F32 is not a stored code format (CSA_ERR_INVALID).
 */
csa_status csa_quantize_keys(const uint16_t *x, int64_t rows, int dim, int format, void *codes,
                             void *scales, void *stream);

/*
 * csa_quantize_query -- the lightning indexer's query encoding on its own: what csa_index_topk
 * scores with, exposed so that it can be checked bit for bit.
 * [DEVTO] "Two Compression Strategies": the indexer runs in low precision (FP4); the query is put
 * in the keys' format so the products run on the low-precision matrix units.
 *
 *   q_idx     bf16 [n, H_I, 128] query heads; w_idx fp32 [n, H_I] head weights.
 *   key_format CSA_KEY_FP8_E4M3: codes uint8 [n, H_I, 128] by csa_quantize_keys's row rule (one
 *             power-of-two scale 2^e per head row); scale_bytes unused (may be NULL);
 *             factors fp32 [n, H_I] = w * 2^e.
 *             CSA_KEY_MXFP4: codes uint8 [n, H_I, 64] (two e2m1 codes per byte, element 2j in the
 *             low nibble) by csa_quantize_keys's MX rule; scale_bytes uint8 [n, H_I, 4] (e8m0 per 32
 *             values); factors fp32 [n, H_I] = w.
 * Limits: H_I in {16, 32, 48, 64}; 0 <= n <= 65535.
 */
csa_status csa_quantize_query(const uint16_t *q_idx, const float *w_idx, int64_t n, int H_I, int key_format,
                              void *codes, void *scale_bytes, float *factors, void *stream);

/*
 * csa_index_topk -- lightning-indexer scores and per-query top-k selection.
 * [EXPLAINER] CSA walk-through: a lightweight scoring head rates each compressed block for the
 * present query and only the k highest-rated blocks are kept; [RABBIT] indexer paragraph: of some
 * 262,000 entries at the longest context, 1,024 go on to attention.
 *
 * For query s of sequence b at position t = q_pos0[b] + s the visible entries are
 * i < min(n_entries[b], (t+1)/m) (an entry is usable once its last token exists).  Its score is
 *     score[i] = sum_h w_idx[b,s,h] * max(0, <q~[b,s,h,:], k~[b,i,:]>)
 * where k~ are the decoded keys and q~ the query quantised by the keys' rule (per head row for
 * fp8, per 32 values for MXFP4; unchanged for fp32).  The selection is the min(topk, visible)
 * highest scores, ties to the lower index, written in ascending index order and padded with -1.
 *
 *   q_idx      [B, Sq, H_I, D_I]: fp32 when key_format == CSA_KEY_F32, else bf16.
 *   w_idx      fp32 [B, Sq, H_I].
 *   k_codes    keys [B, N_cap, ...] in key_format (see csa_key_format); k_scales its scales
 *              (NULL for CSA_KEY_F32).
 *   n_entries  device int64 [B]: valid entries per sequence (<= N_cap).
 *   q_pos0     device int64 [B]: position of query 0 of each sequence.
 *   topk_idx   out int32 [B, Sq, topk].
 *   scores     out fp32 [B, Sq, N_cap] or NULL; when given, visible entries get their score and
 *              the rest -inf (for inspection; it adds traffic).
 * Limits: 1 <= topk <= 2048; fp8/MXFP4 need D_I == 128 and H_I in {16, 32, 48, 64}; fp32 needs
 * H_I * D_I <= 2048 with D_I % 4 == 0; 1 <= N_cap <= 2^21; m >= 1.
 * Kernels: one launch per call on the one-query-per-workgroup path (scores per tile, and the
 * top-k merge in the last tile workgroup of each query to finish); three when many queries share a
 * sequence (prefill) or a cache holds more than about a million entries.
 */
csa_status csa_index_topk(const void *q_idx, const float *w_idx, const void *k_codes,
                          const void *k_scales, int key_format, int B, int Sq, int H_I, int D_I,
                          int64_t N_cap, const int64_t *n_entries, const int64_t *q_pos0, int m,
                          int topk, int32_t *topk_idx, float *scores, void *workspace,
                          size_t workspace_bytes, void *stream);
size_t csa_index_topk_workspace_bytes(int B, int Sq, int64_t N_cap, int topk);

/*
 * csa_attend -- CSA core attention: shared-KV multi-query attention over the selected compressed
 * entries plus the sliding window, in one joint softmax.
 * [EXPLAINER] CSA walk-through: every query head's attention covers the selected entries together
 * with a window of the newest tokens; [SUMMARY] 2.3: shared-KV multi-query attention, RMSNorm on
 * the query heads before core attention; [DEVTO] partial RoPE; [RABBIT] sliding-window paragraph:
 * the window is the newest 128 tokens.
 *
 * For query s of sequence b at t = q_pos0[b] + s, every head h uses
 *     q^ = RoPE(RMSNorm(q[b,s,h,:]; q_norm_w, eps), t)
 * and the rows X = { entries[b, i] : i in topk_idx[b,s,:], i >= 0 } followed by
 * { win_rows[b, p - win_pos0[b]] : max(0, t-window+1) <= p <= t }.  K = V = the row.
 *     out[b,s,h] = sum_x softmax_x(softmax_scale * <q^, x>) x,  lse[b,s,h] = log-sum-exp (natural).
 *
 *   q          bf16 [B, Sq, H, D] raw query heads; q_norm_w bf16 [D] or NULL (ones).
 *   entries    bf16 [B, N_cap, D] compressed entries (as written by csa_compress).
 *   topk_idx   int32 [B, Sq, topk]; -1 marks an empty slot.
 *   win_rows   bf16 [B, W_cap, D] prepared rows; the caller guarantees the window's positions are
 *              inside [win_pos0[b], win_pos0[b] + W_cap).  With win_pos0 NULL, win_rows is a ring
 *              (as csa_decode_append keeps it): the row of position p is row p mod W_cap, and
 *              W_cap >= window is required.
 *   out        bf16 [B, Sq, H, D]; lse fp32 [B, Sq, H] or NULL.
 * Limits: D in {64, 128, 256, 512}; H >= 1 (heads are processed in blocks of 16);
 *         rope_dim % 4 == 0, rope_dim <= D; 1 <= window <= 4096; 1 <= topk <= 2048;
 *         N_cap + W_cap and N_cap + window below 2^31 (rows are named by 32-bit codes);
 *         B * Sq <= 65535.
 */
csa_status csa_attend(const uint16_t *q, const uint16_t *q_norm_w, const uint16_t *entries,
                      int64_t N_cap, const int32_t *topk_idx, int topk, const uint16_t *win_rows,
                      int64_t W_cap, const int64_t *win_pos0, const int64_t *q_pos0, int B, int Sq,
                      int H, int D, int rope_dim, int window, float softmax_scale, float rope_base,
                      float eps, uint16_t *out, float *lse, void *workspace,
                      size_t workspace_bytes, void *stream);
size_t csa_attend_workspace_bytes(int B, int Sq, int H, int D, int topk, int window);

/*
 * csa_attend_noalloc -- csa_attend for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same kernels, with the
 * split-K partials in a scratch array the library holds on each GPU (32 MiB, from module load until
 * the process ends) instead of a caller workspace.  Arguments and results as csa_attend.
 * The call allocates nothing.  Shapes whose partials need more than the scratch holds
 * (csa_attend_workspace_bytes() > 32 MiB) return CSA_ERR_WORKSPACE before any HIP call.  Every
 * call on a GPU uses that GPU's one scratch array: calls that overlap on one GPU (concurrent
 * streams or threads) race and must be serialised by the caller.  A call rewrites every scratch
 * byte it reads, so nothing needs clearing between calls.
 */
csa_status csa_attend_noalloc(const uint16_t *q, const uint16_t *q_norm_w, const uint16_t *entries,
                              int64_t N_cap, const int32_t *topk_idx, int topk, const uint16_t *win_rows,
                              int64_t W_cap, const int64_t *win_pos0, const int64_t *q_pos0, int B, int Sq,
                              int H, int D, int rope_dim, int window, float softmax_scale, float rope_base,
                              float eps, uint16_t *out, float *lse, void *stream);

/*
 * hca_attend -- HCA core attention: dense over every visible compressed entry plus the window.
 * [EXPLAINER] HCA walk-through: no selection step -- each query sees every compressed entry
 * (ordinary multi-query attention, over a far shorter sequence) together with a short window of
 * the newest raw tokens.
 *
 * As csa_attend with the selection replaced by entries 0 .. min(n_entries[b], (t+1)/m) - 1.
 * Limits as csa_attend; N_cap < 2^31.
 */
csa_status hca_attend(const uint16_t *q, const uint16_t *q_norm_w, const uint16_t *entries,
                      int64_t N_cap, const int64_t *n_entries, int m, const uint16_t *win_rows,
                      int64_t W_cap, const int64_t *win_pos0, const int64_t *q_pos0, int B, int Sq,
                      int H, int D, int rope_dim, int window, float softmax_scale, float rope_base,
                      float eps, uint16_t *out, float *lse, void *workspace,
                      size_t workspace_bytes, void *stream);
size_t hca_attend_workspace_bytes(int B, int Sq, int H, int D, int64_t N_cap, int window);

/*
 * csa_output_projection -- grouped output projection of the core-attention head outputs.
 * [SUMMARY] 2.3, shared-KV and output-projection paragraph: both attention types map their many
 * head outputs back to the model width through a projection split into groups, to cut that cost.
 *
 * The H heads fall into G equal groups in head order; group g's concatenated head outputs
 * (K_g = H*D/G values) are projected by its own weight w[g] [N_g, K_g] (a linear layer's
 * [out, in] layout) to N_g outputs; the groups' outputs are concatenated:
 *     y[m, g*N_g + n] = sum_k o[m, g*K_g + k] * w[g, n, k]     (fp32 accumulation)
 *   o  bf16 [M, H*D] (for example csa_attend's output [B, Sq, H, D] with M = B*Sq).
 *   w  bf16 [G, N_g, K_g].
 *   y  out bf16 [M, G*N_g].
 * Limits: H % G == 0; K_g % 256 == 0; N_g % 128 == 0; G*N_g <= 2^20.
 */
csa_status csa_output_projection(const uint16_t *o, const uint16_t *w, int M, int H, int D, int G, int N_g,
                                 uint16_t *y, void *stream);

/* Text for a status code (static storage). */
const char *csa_status_string(csa_status s);
/* Thread-local detail of the last failed call on this thread ("" if none). */
const char *csa_last_error(void);

/*
 * Kernel timing for measurement tools.  csa_timing_enable(1) clears the counters and makes every
 * later launch record a pair of HIP events on its stream; csa_timing_enable(0) stops recording.
 * csa_timing_read() waits for the recorded events and returns the summed duration (ms) and the
 * launch count for one kernel name: "compress", "compress_keys", "quantize", "decode_append",
 * "decode_append_keys", "index_query_prep", "index_score", "index_merge", "attend_split", "attend_combine", "oproj",
 * "stream_read".  Not for use while a stream is being captured into a graph.
 */
void csa_timing_enable(int on);
csa_status csa_timing_read(const char *kernel, double *total_ms, int64_t *launches);

/*
 * Bandwidth floor for measurement tools: a plain streaming read of `bytes` bytes at `src` (device,
 * 16-byte aligned; bytes a positive multiple of 16, at most 2^40), every 16-byte word loaded once
 * by 4,096 workgroups of 512 threads.  Nothing is computed from the bytes; `sink` (device, 4-byte
 * aligned, 4 bytes) is written at most once, with a value of no meaning.  Enqueued on `stream`;
 * recorded under the timing name "stream_read".  A bandwidth-bound kernel of this library is
 * compared with this read of its own byte count as well as with the device's published peak.
 * Errors: CSA_ERR_INVALID for a bad size or pointer (before any HIP call); CSA_ERR_HIP on launch.
 */
csa_status csa_measure_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
