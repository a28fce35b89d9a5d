// C-ABI front of libcsa: argument validation (before any HIP call), planning and dispatch.
// The operations and their arguments are documented in include/csa.h.
#include "../../include/csa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

csa_status fail(csa_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, ...) \
  do { if (!(cond)) return fail(CSA_ERR_INVALID, __VA_ARGS__); } while (0)
#define REQUIRE_PTR(p) \
  do { \
    if ((p) == nullptr) return fail(CSA_ERR_INVALID, "%s must not be NULL", #p); \
    if (!aligned16(p)) return fail(CSA_ERR_INVALID, "%s must be 16-byte aligned", #p); \
  } while (0)
#define REQUIRE_PTR_OR_NULL(p) \
  do { if ((p) != nullptr && !aligned16(p)) return fail(CSA_ERR_INVALID, "%s must be 16-byte aligned", #p); } while (0)

csa_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_last_error.clear();
  return CSA_OK;
}

// ---- kernel timing ---------------------------------------------------------------------------
struct TimedLaunch {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimedLaunch> g_pending;
std::vector<std::pair<std::string, std::pair<double, int64_t>>> g_totals;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  (void)hipEventCreate(&e);
  return e;
}

}  // namespace

namespace csa {
TimingEvents timing_events(const char *name) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing) return {};
  TimedLaunch t{name, take_event(), take_event()};
  if (!t.start || !t.stop) return {};
  g_pending.push_back(t);
  return {t.start, t.stop};
}
}  // namespace csa

extern "C" {

const char *csa_status_string(csa_status s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported shape or format";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *csa_last_error(void) { return g_last_error.c_str(); }

void csa_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto &t : g_pending) { g_event_pool.push_back(t.start); g_event_pool.push_back(t.stop); }
  g_pending.clear();
  g_totals.clear();
  g_timing = on != 0;
}

csa_status csa_timing_read(const char *kernel, double *total_ms, int64_t *launches) {
  if (!kernel || !total_ms || !launches) return fail(CSA_ERR_INVALID, "NULL argument");
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto &t : g_pending) {
    if (hipEventSynchronize(t.stop) != hipSuccess) return fail(CSA_ERR_HIP, "event sync failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) return fail(CSA_ERR_HIP, "elapsed time failed");
    bool found = false;
    for (auto &tot : g_totals)
      if (tot.first == t.name) { tot.second.first += ms; tot.second.second += 1; found = true; }
    if (!found) g_totals.push_back({t.name, {double(ms), 1}});
    g_event_pool.push_back(t.start);
    g_event_pool.push_back(t.stop);
  }
  g_pending.clear();
  *total_ms = 0.0;
  *launches = 0;
  for (auto &tot : g_totals)
    if (tot.first == kernel) { *total_ms = tot.second.first; *launches = tot.second.second; }
  return CSA_OK;
}

// ---------------------------------------------------------------------------------------------
csa_status csa_compress(const uint16_t *c, const uint16_t *z, const uint16_t *bias,
                        const uint16_t *norm_w, int B, int64_t n_new, int halo, int d, int m,
                        int overlap, int rope_dim, int64_t pos0, float rope_base, float eps,
                        uint16_t *entries, uint16_t *win_rows, void *stream) {
  REQUIRE(B >= 0, "B must be >= 0");
  REQUIRE(n_new >= 0, "n_new must be >= 0");
  REQUIRE(d == 64 || d == 128 || d == 256 || d == 512 || d == 1024, "d must be one of 64, 128, 256, 512, 1024");
  REQUIRE(m >= 1 && m <= 1024, "m must be in [1, 1024]");
  REQUIRE(overlap == 0 || overlap == 1, "overlap must be 0 or 1");
  REQUIRE(rope_dim >= 0 && rope_dim <= d && rope_dim % 4 == 0, "rope_dim must be a multiple of 4 in [0, d]");
  REQUIRE(pos0 >= 0 && pos0 % m == 0, "pos0 must be a non-negative multiple of m");
  REQUIRE(n_new % m == 0, "n_new must be a multiple of m");
  REQUIRE(halo == ((overlap && pos0 > 0) ? m : 0), "halo must be m when overlap && pos0 > 0, else 0");
  REQUIRE(eps > 0.f && std::isfinite(eps), "eps must be positive");
  REQUIRE(rope_base > 1.f && std::isfinite(rope_base), "rope_base must be > 1");
  REQUIRE(n_new / m <= 2147483647LL && B <= 65535, "too many entries or sequences");
  if (B == 0 || n_new == 0) return CSA_OK;
  REQUIRE_PTR(c); REQUIRE_PTR(z); REQUIRE_PTR(bias); REQUIRE_PTR(entries);
  REQUIRE_PTR_OR_NULL(norm_w); REQUIRE_PTR_OR_NULL(win_rows);
  csa::CompressArgs a{c, z, bias, norm_w, entries, win_rows, B, d, m, overlap, rope_dim, halo,
                      n_new, pos0, std::log2(double(rope_base)), eps};
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = csa::launch_compress(a, st);
  return launched(e, "compress launch");
}

csa_status csa_decode_append(const uint16_t *c_new, const uint16_t *z_new, const uint16_t *k_new,
                             const int64_t *pos, const uint16_t *bias, const uint16_t *norm_w, int B,
                             int d, int m, int overlap, int rope_dim, float rope_base, float eps,
                             uint16_t *tok_c, uint16_t *tok_z, uint16_t *win_ring, int64_t W_cap,
                             uint16_t *entries, int64_t N_cap, int key_format, int D_I, void *k_codes,
                             void *k_scales, int64_t *n_entries, void *stream) {
  REQUIRE(B >= 0 && B <= 65535, "B must be in [0, 65535]");
  REQUIRE(d == 64 || d == 128 || d == 256 || d == 512 || d == 1024, "d must be one of 64, 128, 256, 512, 1024");
  REQUIRE(m >= 1 && m <= 1024, "m must be in [1, 1024]");
  REQUIRE(overlap == 0 || overlap == 1, "overlap must be 0 or 1");
  REQUIRE(rope_dim >= 0 && rope_dim <= d && rope_dim % 4 == 0, "rope_dim must be a multiple of 4 in [0, d]");
  REQUIRE(eps > 0.f && std::isfinite(eps), "eps must be positive");
  REQUIRE(rope_base > 1.f && std::isfinite(rope_base), "rope_base must be > 1");
  REQUIRE(W_cap >= 1 && W_cap < (int64_t(1) << 31), "W_cap must be in [1, 2^31)");
  REQUIRE(N_cap >= 1 && N_cap < (int64_t(1) << 31), "N_cap must be in [1, 2^31)");
  if (k_new) {
    REQUIRE(key_format == CSA_KEY_F32 || key_format == CSA_KEY_FP8_E4M3 || key_format == CSA_KEY_MXFP4,
            "unknown key_format %d", key_format);
    REQUIRE(D_I >= 32 && D_I <= 1024 && D_I % 32 == 0, "D_I must be a multiple of 32 in [32, 1024]");
  }
  if (B == 0) return CSA_OK;
  REQUIRE_PTR(c_new); REQUIRE_PTR(z_new); REQUIRE_PTR(pos); REQUIRE_PTR(bias); REQUIRE_PTR_OR_NULL(norm_w);
  REQUIRE_PTR(tok_c); REQUIRE_PTR(tok_z); REQUIRE_PTR(win_ring); REQUIRE_PTR(entries); REQUIRE_PTR(n_entries);
  REQUIRE_PTR_OR_NULL(k_new);
  if (k_new) {
    REQUIRE_PTR(k_codes);
    if (key_format != CSA_KEY_F32) REQUIRE_PTR(k_scales);
  }
  csa::AppendArgs a{};
  a.c_new = c_new; a.z_new = z_new; a.k_new = k_new; a.bias = bias; a.norm_w = norm_w; a.pos = pos;
  a.tok_c = tok_c; a.tok_z = tok_z; a.win_ring = win_ring; a.entries = entries;
  a.k_codes = k_codes; a.k_scales = k_scales; a.n_entries = n_entries; a.W_cap = W_cap; a.N_cap = N_cap;
  a.B = B; a.d = d; a.m = m; a.overlap = overlap; a.rope_dim = rope_dim; a.key_format = key_format;
  a.D_I = D_I; a.log2_base = std::log2(double(rope_base)); a.eps = eps;
  hipError_t e = csa::launch_append(a, static_cast<hipStream_t>(stream));
  return launched(e, "decode_append launch");
}

static csa_status check_key_cache(int D_I, int key_format, void *k_codes, void *k_scales) {
  if (!(D_I == 128 || D_I == 256 || D_I == 512 || D_I == 1024))
    return fail(CSA_ERR_UNSUPPORTED, "D_I must be one of 128, 256, 512, 1024 (got %d)", D_I);
  REQUIRE(key_format == CSA_KEY_F32 || key_format == CSA_KEY_FP8_E4M3 || key_format == CSA_KEY_MXFP4,
          "unknown key_format %d", key_format);
  REQUIRE_PTR(k_codes);
  if (key_format != CSA_KEY_F32) REQUIRE_PTR(k_scales);
  return CSA_OK;
}

csa_status csa_compress_index_keys(const uint16_t *c_i, const uint16_t *z_i, const uint16_t *bias_i, int B,
                                   int64_t n_new, int halo, int D_I, int m, int overlap, int64_t pos0,
                                   int key_format, uint16_t *keys_out, void *k_codes, void *k_scales,
                                   void *stream) {
  REQUIRE(B >= 0 && B <= 65535, "B must be in [0, 65535]");
  REQUIRE(n_new >= 0, "n_new must be >= 0");
  REQUIRE(m >= 1 && m <= 1024, "m must be in [1, 1024]");
  REQUIRE(overlap == 0 || overlap == 1, "overlap must be 0 or 1");
  REQUIRE(pos0 >= 0 && pos0 % m == 0, "pos0 must be a non-negative multiple of m");
  REQUIRE(n_new % m == 0, "n_new must be a multiple of m");
  REQUIRE(halo == ((overlap && pos0 > 0) ? m : 0), "halo must be m when overlap && pos0 > 0, else 0");
  REQUIRE(n_new / m <= 2147483647LL, "too many entries");
  if (B == 0 || n_new == 0) return CSA_OK;
  csa_status s = check_key_cache(D_I, key_format, k_codes, k_scales);
  if (s != CSA_OK) return s;
  REQUIRE_PTR(c_i); REQUIRE_PTR(z_i); REQUIRE_PTR(bias_i); REQUIRE_PTR_OR_NULL(keys_out);
  csa::CompressArgs a{};
  a.c = c_i; a.z = z_i; a.bias = bias_i; a.norm_w = nullptr; a.entries = keys_out; a.win_rows = nullptr;
  a.B = B; a.d = D_I; a.m = m; a.overlap = overlap; a.rope_dim = 0; a.halo = halo; a.n_new = n_new;
  a.pos0 = pos0; a.log2_base = 1.0; a.eps = 1e-6f; a.key_format = key_format; a.k_codes = k_codes;
  a.k_scales = k_scales;
  hipError_t e = csa::launch_compress_keys(a, static_cast<hipStream_t>(stream));
  return launched(e, "compress_index_keys launch");
}

csa_status csa_decode_append_index(const uint16_t *c_i_new, const uint16_t *z_i_new, const int64_t *pos,
                                   const uint16_t *bias_i, int B, int D_I, int m, int overlap, uint16_t *tok_c,
                                   uint16_t *tok_z, int64_t N_cap, int key_format, uint16_t *keys_out,
                                   void *k_codes, void *k_scales, void *stream) {
  REQUIRE(B >= 0 && B <= 65535, "B must be in [0, 65535]");
  REQUIRE(m >= 1 && m <= 1024, "m must be in [1, 1024]");
  REQUIRE(overlap == 0 || overlap == 1, "overlap must be 0 or 1");
  REQUIRE(N_cap >= 1 && N_cap < (int64_t(1) << 31), "N_cap must be in [1, 2^31)");
  if (B == 0) return CSA_OK;
  csa_status s = check_key_cache(D_I, key_format, k_codes, k_scales);
  if (s != CSA_OK) return s;
  REQUIRE_PTR(c_i_new); REQUIRE_PTR(z_i_new); REQUIRE_PTR(pos); REQUIRE_PTR(bias_i);
  REQUIRE_PTR(tok_c); REQUIRE_PTR(tok_z); REQUIRE_PTR_OR_NULL(keys_out);
  csa::AppendArgs a{};
  a.c_new = c_i_new; a.z_new = z_i_new; a.k_new = nullptr; a.bias = bias_i; a.norm_w = nullptr; a.pos = pos;
  a.tok_c = tok_c; a.tok_z = tok_z; a.win_ring = nullptr; a.entries = keys_out; a.k_codes = k_codes;
  a.k_scales = k_scales; a.n_entries = nullptr; a.W_cap = 1; a.N_cap = N_cap; a.B = B; a.d = D_I; a.m = m;
  a.overlap = overlap; a.rope_dim = 0; a.key_format = key_format; a.D_I = D_I; a.log2_base = 1.0;
  a.eps = 1e-6f;
  hipError_t e = csa::launch_append_keys(a, static_cast<hipStream_t>(stream));
  return launched(e, "decode_append_index launch");
}

csa_status csa_decode_append_step(const uint16_t *c_new, const uint16_t *z_new, const int64_t *pos,
                                  const uint16_t *bias, const uint16_t *norm_w, int B, int d, int m, int overlap,
                                  int rope_dim, float rope_base, float eps, uint16_t *tok_c, uint16_t *tok_z,
                                  uint16_t *win_ring, int64_t W_cap, uint16_t *entries, int64_t N_cap,
                                  int64_t *n_entries, const uint16_t *c_i_new, const uint16_t *z_i_new,
                                  const uint16_t *bias_i, int D_I, uint16_t *tok_ci, uint16_t *tok_zi,
                                  int key_format, uint16_t *keys_out, void *k_codes, void *k_scales, void *stream) {
  REQUIRE(B >= 0 && B <= 65535, "B must be in [0, 65535]");
  if (!(d == 128 || d == 256 || d == 512 || d == 1024))
    return fail(CSA_ERR_UNSUPPORTED, "d must be one of 128, 256, 512, 1024 (got %d)", d);
  REQUIRE(m >= 1 && m <= 1024, "m must be in [1, 1024]");
  REQUIRE(overlap == 0 || overlap == 1, "overlap must be 0 or 1");
  REQUIRE(rope_dim >= 0 && rope_dim <= d && rope_dim % 4 == 0, "rope_dim must be a multiple of 4 in [0, d]");
  REQUIRE(eps > 0.f && std::isfinite(eps), "eps must be positive");
  REQUIRE(rope_base > 1.f && std::isfinite(rope_base), "rope_base must be > 1");
  REQUIRE(W_cap >= 1 && W_cap < (int64_t(1) << 31), "W_cap must be in [1, 2^31)");
  REQUIRE(N_cap >= 1 && N_cap < (int64_t(1) << 31), "N_cap must be in [1, 2^31)");
  if (B == 0) return CSA_OK;
  csa_status s = check_key_cache(D_I, key_format, k_codes, k_scales);
  if (s != CSA_OK) return s;
  REQUIRE_PTR(c_new); REQUIRE_PTR(z_new); REQUIRE_PTR(pos); REQUIRE_PTR(bias); REQUIRE_PTR_OR_NULL(norm_w);
  REQUIRE_PTR(tok_c); REQUIRE_PTR(tok_z); REQUIRE_PTR(win_ring); REQUIRE_PTR(entries); REQUIRE_PTR(n_entries);
  REQUIRE_PTR(c_i_new); REQUIRE_PTR(z_i_new); REQUIRE_PTR(bias_i); REQUIRE_PTR(tok_ci); REQUIRE_PTR(tok_zi);
  REQUIRE_PTR_OR_NULL(keys_out);
  csa::AppendArgs a{};
  a.c_new = c_new; a.z_new = z_new; a.k_new = nullptr; a.bias = bias; a.norm_w = norm_w; a.pos = pos;
  a.tok_c = tok_c; a.tok_z = tok_z; a.win_ring = win_ring; a.entries = entries; a.k_codes = nullptr;
  a.k_scales = nullptr; a.n_entries = n_entries; a.W_cap = W_cap; a.N_cap = N_cap; a.B = B; a.d = d; a.m = m;
  a.overlap = overlap; a.rope_dim = rope_dim; a.key_format = key_format; a.D_I = D_I;
  a.log2_base = std::log2(double(rope_base)); a.eps = eps;
  csa::AppendArgs ai{};
  ai.c_new = c_i_new; ai.z_new = z_i_new; ai.k_new = nullptr; ai.bias = bias_i; ai.norm_w = nullptr; ai.pos = pos;
  ai.tok_c = tok_ci; ai.tok_z = tok_zi; ai.win_ring = nullptr; ai.entries = keys_out; ai.k_codes = k_codes;
  ai.k_scales = k_scales; ai.n_entries = nullptr; ai.W_cap = 1; ai.N_cap = N_cap; ai.B = B; ai.d = D_I; ai.m = m;
  ai.overlap = overlap; ai.rope_dim = 0; ai.key_format = key_format; ai.D_I = D_I; ai.log2_base = 1.0;
  ai.eps = 1e-6f;
  hipError_t e = csa::launch_append_step(a, ai, static_cast<hipStream_t>(stream));
  return launched(e, "decode_append_step launch");
}

csa_status csa_output_projection(const uint16_t *o, const uint16_t *w, int M, int H, int D, int G, int N_g,
                                 uint16_t *y, void *stream) {
  REQUIRE(M >= 0 && M <= (1 << 24), "M must be in [0, 2^24]");
  REQUIRE(H >= 1 && D >= 1 && G >= 1 && H % G == 0, "H must be a positive multiple of G");
  const int64_t K_g = int64_t(H) * D / G;
  if (K_g % 256 != 0 || K_g > (1 << 20) || N_g % 128 != 0 || N_g < 128 || int64_t(G) * N_g > (1 << 20))
    return fail(CSA_ERR_UNSUPPORTED, "need (H*D/G) %% 256 == 0 and N_g %% 128 == 0 (got K_g %lld, N_g %d)",
                (long long)K_g, N_g);
  if (M == 0) return CSA_OK;
  REQUIRE_PTR(o); REQUIRE_PTR(w); REQUIRE_PTR(y);
  csa::ProjArgs a{o, w, y, M, G, N_g, int(K_g), int64_t(H) * D, int64_t(G) * N_g};
  hipError_t e = csa::launch_oproj(a, static_cast<hipStream_t>(stream));
  return launched(e, "output projection launch");
}

csa_status csa_measure_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream) {
  REQUIRE(bytes > 0 && bytes % 16 == 0, "bytes must be a positive multiple of 16");
  REQUIRE(bytes <= (int64_t(1) << 40), "bytes must be <= 2^40");
  REQUIRE_PTR(src);
  REQUIRE(sink != nullptr && (reinterpret_cast<uintptr_t>(sink) & 3u) == 0, "sink must be a 4-byte aligned pointer");
  hipError_t e = csa::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream));
  return launched(e, "stream read launch");
}

csa_status csa_quantize_keys(const uint16_t *x, int64_t rows, int dim, int format, void *codes,
                             void *scales, void *stream) {
  REQUIRE(format == CSA_KEY_FP8_E4M3 || format == CSA_KEY_MXFP4, "format must be CSA_KEY_FP8_E4M3 or CSA_KEY_MXFP4");
  REQUIRE(rows >= 0, "rows must be >= 0");
  REQUIRE(dim > 0 && dim % 32 == 0 && dim <= 1024, "dim must be a multiple of 32 in [32, 1024]");
  REQUIRE(rows <= (int64_t(1) << 34), "too many rows");
  if (rows == 0) return CSA_OK;
  REQUIRE_PTR(x); REQUIRE_PTR(codes); REQUIRE_PTR(scales);
  csa::QuantizeArgs a{x, codes, scales, rows, dim, format};
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = csa::launch_quantize(a, st);
  return launched(e, "quantize launch");
}

csa_status csa_quantize_query(const uint16_t *q_idx, const float *w_idx, int64_t n, int H_I, int key_format,
                              void *codes, void *scale_bytes, float *factors, void *stream) {
  REQUIRE(key_format == CSA_KEY_FP8_E4M3 || key_format == CSA_KEY_MXFP4,
          "key_format must be CSA_KEY_FP8_E4M3 or CSA_KEY_MXFP4");
  REQUIRE(H_I == 16 || H_I == 32 || H_I == 48 || H_I == 64, "H_I must be one of 16, 32, 48, 64");
  REQUIRE(n >= 0 && n <= 65535, "n must be in [0, 65535]");
  if (n == 0) return CSA_OK;
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w_idx); REQUIRE_PTR(codes); REQUIRE_PTR(factors);
  if (key_format == CSA_KEY_MXFP4) REQUIRE_PTR(scale_bytes);
  hipError_t e = csa::launch_query_codes(q_idx, w_idx, n, H_I, key_format, codes, scale_bytes, factors,
                                         static_cast<hipStream_t>(stream));
  return launched(e, "quantize_query launch");
}

size_t csa_index_topk_workspace_bytes(int B, int Sq, int64_t N_cap, int topk) {
  if (B <= 0 || Sq <= 0 || N_cap <= 0 || topk <= 0) return 256;
  // the largest of the plans (tiles shared by several queries, one query per segment or per
  // tile): the plan depends on the key format and on whether full scores are asked for
  size_t n = csa::index_workspace_bytes(B, Sq, N_cap, topk, CSA_KEY_F32, false);
  for (int f : {CSA_KEY_FP8_E4M3, CSA_KEY_MXFP4})
    for (bool shared : {true, false}) n = std::max(n, csa::index_workspace_bytes(B, Sq, N_cap, topk, f, shared));
  return n;
}

csa_status csa_index_topk(const void *q_idx, const float *w_idx, const void *k_codes,
                          const void *k_scales, int key_format, int B, int Sq, int H_I, int D_I,
                          int64_t N_cap, const int64_t *n_entries, const int64_t *q_pos0, int m,
                          int topk, int32_t *topk_idx, float *scores, void *workspace,
                          size_t workspace_bytes, void *stream) {
  REQUIRE(key_format == CSA_KEY_F32 || key_format == CSA_KEY_FP8_E4M3 || key_format == CSA_KEY_MXFP4,
          "unknown key_format %d", key_format);
  REQUIRE(B >= 0 && Sq >= 0, "B and Sq must be >= 0");
  REQUIRE(topk >= 1 && topk <= 2048, "topk must be in [1, 2048]");
  REQUIRE(m >= 1, "m must be >= 1");
  REQUIRE(N_cap >= 1 && N_cap <= (int64_t(1) << 21), "N_cap must be in [1, 2097152]");
  REQUIRE(int64_t(B) * Sq <= 65535, "B * Sq must be <= 65535");
  if (key_format == CSA_KEY_F32) {
    REQUIRE(H_I >= 1 && H_I <= 64, "H_I must be in [1, 64] for fp32 keys");
    REQUIRE(D_I >= 4 && D_I % 4 == 0 && H_I * D_I <= 2048, "fp32 keys need D_I % 4 == 0 and H_I * D_I <= 2048");
  } else {
    if (D_I != 128) return fail(CSA_ERR_UNSUPPORTED, "quantised keys need D_I == 128 (got %d)", D_I);
    if (!(H_I == 16 || H_I == 32 || H_I == 48 || H_I == 64))
      return fail(CSA_ERR_UNSUPPORTED, "quantised keys need H_I in {16, 32, 48, 64} (got %d)", H_I);
  }
  if (B == 0 || Sq == 0) return CSA_OK;
  REQUIRE_PTR(q_idx); REQUIRE_PTR(w_idx); REQUIRE_PTR(k_codes); REQUIRE_PTR(n_entries);
  REQUIRE_PTR(q_pos0); REQUIRE_PTR(topk_idx);
  if (key_format != CSA_KEY_F32) REQUIRE_PTR(k_scales);
  REQUIRE_PTR_OR_NULL(scores);
  // full scores are written by the one-query-per-workgroup kernels only (no shared tiles)
  const bool shared = scores == nullptr;
  const size_t need = csa::index_workspace_bytes(B, Sq, N_cap, topk, key_format, shared);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "index_topk needs %zu workspace bytes, got %zu", need, workspace_bytes);
  REQUIRE_PTR(workspace);
  csa::IndexArgs a{};
  a.q_idx = q_idx; a.w_idx = w_idx; a.k_codes = k_codes; a.k_scales = k_scales;
  a.n_entries = n_entries; a.q_pos0 = q_pos0; a.topk_idx = topk_idx; a.scores = scores;
  a.workspace = workspace; a.format = key_format; a.B = B; a.Sq = Sq; a.H_I = H_I; a.D_I = D_I;
  a.m = m; a.topk = topk; a.N_cap = N_cap;
  a.plan = csa::plan_index(B, Sq, N_cap, topk, key_format, shared);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = csa::launch_index_score(a, st);
  return launched(e, "index_topk launch");
}

static csa_status check_attend_common(const uint16_t *q, const uint16_t *q_norm_w, const uint16_t *entries,
                                      int64_t N_cap, const uint16_t *win_rows, int64_t W_cap,
                                      const int64_t *win_pos0, const int64_t *q_pos0, int B, int Sq, int H,
                                      int D, int rope_dim, int window, float softmax_scale, float rope_base,
                                      float eps, uint16_t *out, float *lse) {
  REQUIRE(B >= 0 && Sq >= 0, "B and Sq must be >= 0");
  REQUIRE(H >= 1 && H <= 1024, "H must be in [1, 1024]");
  if (!(D == 64 || D == 128 || D == 256 || D == 512)) return fail(CSA_ERR_UNSUPPORTED, "D must be one of 64, 128, 256, 512");
  REQUIRE(rope_dim >= 0 && rope_dim <= D && rope_dim % 4 == 0, "rope_dim must be a multiple of 4 in [0, D]");
  REQUIRE(window >= 1 && window <= 4096, "window must be in [1, 4096]");
  REQUIRE(N_cap >= 1 && N_cap < (int64_t(1) << 31), "N_cap must be in [1, 2^31)");
  REQUIRE(W_cap >= 1 && N_cap + W_cap < (int64_t(1) << 31), "W_cap must be >= 1 and N_cap + W_cap < 2^31");
  REQUIRE(N_cap + window < (int64_t(1) << 31), "N_cap + window must be < 2^31");
  REQUIRE(std::isfinite(softmax_scale) && softmax_scale > 0.f, "softmax_scale must be positive");
  REQUIRE(eps > 0.f && std::isfinite(eps), "eps must be positive");
  REQUIRE(rope_base > 1.f && std::isfinite(rope_base), "rope_base must be > 1");
  REQUIRE(int64_t(B) * Sq <= 65535, "B * Sq must be <= 65535");
  if (B == 0 || Sq == 0) return CSA_OK;
  REQUIRE_PTR(q); REQUIRE_PTR(entries); REQUIRE_PTR(win_rows); REQUIRE_PTR_OR_NULL(win_pos0);
  REQUIRE_PTR(q_pos0); REQUIRE_PTR(out); REQUIRE_PTR_OR_NULL(q_norm_w); REQUIRE_PTR_OR_NULL(lse);
  // win_pos0 NULL: win_rows is a ring holding position p at row p mod W_cap (csa_decode_append)
  REQUIRE(win_pos0 != nullptr || W_cap >= window, "a window ring (win_pos0 NULL) needs W_cap >= window");
  return CSA_OK;
}

static csa_status run_attend(csa::AttendArgs &a, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = csa::launch_attend(a, st);
  if (e != hipSuccess) return launched(e, "attend launch");
  if (a.plan.n_splits > 1 && !a.plan.fused) e = csa::launch_combine(a, st);
  return launched(e, "combine launch");
}

size_t csa_attend_workspace_bytes(int B, int Sq, int H, int D, int topk, int window) {
  if (B <= 0 || Sq <= 0 || H <= 0 || D <= 0 || topk <= 0 || window <= 0) return 256;
  return csa::attend_workspace_bytes(int64_t(B) * Sq, H, D, topk, window);
}

size_t hca_attend_workspace_bytes(int B, int Sq, int H, int D, int64_t N_cap, int window) {
  if (B <= 0 || Sq <= 0 || H <= 0 || D <= 0 || N_cap <= 0 || window <= 0) return 256;
  return csa::attend_workspace_bytes(int64_t(B) * Sq, H, D, N_cap, window);
}

csa_status csa_attend(const uint16_t *q, const uint16_t *q_norm_w, const uint16_t *entries,
                      int64_t N_cap, const int32_t *topk_idx, int topk, const uint16_t *win_rows,
                      int64_t W_cap, const int64_t *win_pos0, const int64_t *q_pos0, int B, int Sq,
                      int H, int D, int rope_dim, int window, float softmax_scale, float rope_base,
                      float eps, uint16_t *out, float *lse, void *workspace,
                      size_t workspace_bytes, void *stream) {
  csa_status s = check_attend_common(q, q_norm_w, entries, N_cap, win_rows, W_cap, win_pos0, q_pos0, B,
                                     Sq, H, D, rope_dim, window, softmax_scale, rope_base, eps, out, lse);
  if (s != CSA_OK || B == 0 || Sq == 0) return s;
  REQUIRE(topk >= 1 && topk <= 2048, "topk must be in [1, 2048]");
  REQUIRE_PTR(topk_idx);
  const size_t need = csa::attend_workspace_bytes(int64_t(B) * Sq, H, D, topk, window);
  if (need > 256 && (workspace == nullptr || workspace_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "csa_attend needs %zu workspace bytes, got %zu", need, workspace_bytes);
  REQUIRE_PTR_OR_NULL(workspace);
  csa::AttendArgs a{};
  a.q = q; a.q_norm_w = q_norm_w; a.entries = entries; a.win_rows = win_rows; a.topk_idx = topk_idx;
  a.n_entries = nullptr; a.win_pos0 = win_pos0; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  a.workspace = workspace; a.N_cap = N_cap; a.W_cap = W_cap; a.n_sel = topk; a.B = B; a.Sq = Sq;
  a.H = H; a.D = D; a.rope_dim = rope_dim; a.window = window; a.m = 1;
  a.scale_log2 = softmax_scale * 1.4426950408889634f; a.log2_base = std::log2(double(rope_base));
  a.eps = eps;
  a.plan = csa::plan_attend(int64_t(B) * Sq, H, topk, window, D);
  return run_attend(a, stream);
}

csa_status csa_attend_noalloc(const uint16_t *q, const uint16_t *q_norm_w, const uint16_t *entries,
                              int64_t N_cap, const int32_t *topk_idx, int topk, const uint16_t *win_rows,
                              int64_t W_cap, const int64_t *win_pos0, const int64_t *q_pos0, int B, int Sq,
                              int H, int D, int rope_dim, int window, float softmax_scale, float rope_base,
                              float eps, uint16_t *out, float *lse, void *stream) {
  csa_status s = check_attend_common(q, q_norm_w, entries, N_cap, win_rows, W_cap, win_pos0, q_pos0, B,
                                     Sq, H, D, rope_dim, window, softmax_scale, rope_base, eps, out, lse);
  if (s != CSA_OK || B == 0 || Sq == 0) return s;
  REQUIRE(topk >= 1 && topk <= 2048, "topk must be in [1, 2048]");
  REQUIRE_PTR(topk_idx);
  const size_t need = csa::attend_workspace_bytes(int64_t(B) * Sq, H, D, topk, window);
  if (need > csa::attend_scratch_bytes())
    return fail(CSA_ERR_WORKSPACE, "csa_attend_noalloc needs %zu scratch bytes for this shape; its scratch holds %zu",
                need, csa::attend_scratch_bytes());
  void *ws = nullptr;
  hipError_t e = csa::attend_scratch(&ws);
  if (e != hipSuccess) return fail(CSA_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
  csa::AttendArgs a{};
  a.q = q; a.q_norm_w = q_norm_w; a.entries = entries; a.win_rows = win_rows; a.topk_idx = topk_idx;
  a.n_entries = nullptr; a.win_pos0 = win_pos0; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  a.workspace = ws; a.N_cap = N_cap; a.W_cap = W_cap; a.n_sel = topk; a.B = B; a.Sq = Sq;
  a.H = H; a.D = D; a.rope_dim = rope_dim; a.window = window; a.m = 1;
  a.scale_log2 = softmax_scale * 1.4426950408889634f; a.log2_base = std::log2(double(rope_base));
  a.eps = eps;
  a.plan = csa::plan_attend(int64_t(B) * Sq, H, topk, window, D);
  return run_attend(a, stream);
}

csa_status hca_attend(const uint16_t *q, const uint16_t *q_norm_w, const uint16_t *entries,
                      int64_t N_cap, const int64_t *n_entries, int m, const uint16_t *win_rows,
                      int64_t W_cap, const int64_t *win_pos0, const int64_t *q_pos0, int B, int Sq,
                      int H, int D, int rope_dim, int window, float softmax_scale, float rope_base,
                      float eps, uint16_t *out, float *lse, void *workspace,
                      size_t workspace_bytes, void *stream) {
  csa_status s = check_attend_common(q, q_norm_w, entries, N_cap, win_rows, W_cap, win_pos0, q_pos0, B,
                                     Sq, H, D, rope_dim, window, softmax_scale, rope_base, eps, out, lse);
  if (s != CSA_OK || B == 0 || Sq == 0) return s;
  REQUIRE(m >= 1, "m must be >= 1");
  REQUIRE_PTR(n_entries);
  const size_t need = csa::attend_workspace_bytes(int64_t(B) * Sq, H, D, N_cap, window);
  if (need > 256 && (workspace == nullptr || workspace_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "hca_attend needs %zu workspace bytes, got %zu", need, workspace_bytes);
  REQUIRE_PTR_OR_NULL(workspace);
  csa::AttendArgs a{};
  a.q = q; a.q_norm_w = q_norm_w; a.entries = entries; a.win_rows = win_rows; a.topk_idx = nullptr;
  a.n_entries = n_entries; a.win_pos0 = win_pos0; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  a.workspace = workspace; a.N_cap = N_cap; a.W_cap = W_cap; a.n_sel = N_cap; a.B = B; a.Sq = Sq;
  a.H = H; a.D = D; a.rope_dim = rope_dim; a.window = window; a.m = m;
  a.scale_log2 = softmax_scale * 1.4426950408889634f; a.log2_base = std::log2(double(rope_base));
  a.eps = eps;
  a.plan = csa::plan_attend(int64_t(B) * Sq, H, N_cap, window, D);
  return run_attend(a, stream);
}

}  // extern "C"
