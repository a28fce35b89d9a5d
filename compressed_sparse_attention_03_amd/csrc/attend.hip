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

// Waves per workgroup: each wave owns D/NW channels (at least 32).
template <int D>
constexpr int waves_of() { return D >= 128 ? 4 : D / 32; }

template <int D>
__global__ void __launch_bounds__(64 * waves_of<D>()) attend_split_kernel(AttendArgs a, int64_t n_queries) {
  constexpr int NW = waves_of<D>();
  constexpr int NT = 64 * NW;
  constexpr int QD = D / NW;          // channels owned by one wave
  constexpr int NSQ = QD / 32;        // its 32-channel steps
  constexpr int QCH = D / 32;         // prologue: threads per head (32 channels each)
  constexpr int RING = 4;             // 16-row chunks in flight per wave
  __shared__ __align__(16) uint16_t s_q[16 * D];
  __shared__ int s_row[kMaxRowsPerSplit];
  __shared__ float s_cs[256], s_sn[256];
  __shared__ __align__(16) float s_part[2][NW][64][4];   // partial S^T per wave, per lane
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
  const int ch0 = wave * QD;          // first channel of this wave

  // ---- prologue.  The raw q chunk (and norm weights) of this thread are loaded first: loads
  // complete in issue order, so anything issued later (the row prefetch) does not delay them.
  const bool qthread = tid < 16 * QCH;
  const int qh = tid / QCH, qc = tid % QCH;
  const int qhead = hb * 16 + qh;
  uint4 qraw[4], wraw[4];
  if (qthread) {
    const uint4 *src = reinterpret_cast<const uint4 *>(a.q + (qi * a.H + (qhead < a.H ? qhead : 0)) * D + 32 * qc);
    const uint4 *wsrc = reinterpret_cast<const uint4 *>(a.q_norm_w ? a.q_norm_w + 32 * qc : a.q + 32 * qc);
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

  // ring of row fragments: lane (r, g) holds row r of the chunk, channels ch0 + 32s + 8g .. +7
  Frag8 ring[RING][NSQ];
  int codes[RING];
  // Loads are unconditional (an empty slot reads entry row 0, which exists and is finite; its
  // softmax weight is exactly 0): branch-free code lets the compiler wait only for the chunk in use
  // instead of every outstanding load.
  auto issue = [&](int c, int slot) {
    const int i = c * 16 + r;
    const int code = (c < n_chunks && i < nr) ? s_row[i] : -1;
    codes[slot] = code;
    const uint16_t *rp = code < 0 ? ent_b
                                  : (code < a.N_cap ? ent_b + int64_t(code) * D : win_b + (int64_t(code) - a.N_cap) * D);
#pragma unroll
    for (int s = 0; s < NSQ; ++s) ring[slot][s].u = *reinterpret_cast<const uint4 *>(rp + ch0 + 32 * s + 8 * g);
  };
#pragma unroll
  for (int c = 0; c < RING - 1; ++c) issue(c, c);

  // q^ = RoPE(RMSNorm(q)) * scale * log2(e) for the 16 heads, into LDS
  if (qthread) {
    {
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
      uint4 *dst = reinterpret_cast<uint4 *>(s_q + h * D + 32 * c);
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
  }
  __syncthreads();
  Frag8 qf[NSQ];
#pragma unroll
  for (int s = 0; s < NSQ; ++s) qf[s].u = *reinterpret_cast<const uint4 *>(s_q + r * D + ch0 + 32 * s + 8 * g);

  // identity fragment for the V transposes: element j of lane (n, g) is 1 iff n = 4g + j
  v4s ident;
#pragma unroll
  for (int j = 0; j < 4; ++j) ident[j] = ((r >> 2) == g && (r & 3) == j) ? short(0x3f80) : short(0);

  v4f o[2 * NSQ];
#pragma unroll
  for (int k = 0; k < 2 * NSQ; ++k) o[k] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // one chunk: all waves sum their partial S^T through LDS, update the (identical) softmax state
  // and accumulate their channels of O.  `slot` is a compile-time ring position after unrolling.
  auto chunk = [&](int c, int slot) {
    const uint64_t vmask = __ballot(codes[slot] >= 0);
    v4f st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSQ; ++s) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[slot][s].b, qf[s].b, st, 0, 0, 0);
    *reinterpret_cast<v4f *>(&s_part[c & 1][wave][lane][0]) = st;
    __syncthreads();
    v4f full = *reinterpret_cast<const v4f *>(&s_part[c & 1][0][lane][0]);
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const v4f x = *reinterpret_cast<const v4f *>(&s_part[c & 1][w][lane][0]);
      full[0] += x[0]; full[1] += x[1]; full[2] += x[2]; full[3] += x[3];
    }
    float sv[4], cmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = ((vmask >> (4 * g + v)) & 1) ? full[v] : -INFINITY;
      cmax = fmaxf(cmax, sv[v]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    // lazy running max: rescale only when some head's max grew past the slack
    const bool grow = cmax > m_run + kRescaleSlack || (m_run == -INFINITY && cmax != -INFINITY);
    if (__any(grow)) {
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      float av[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
      for (int k = 0; k < 2 * NSQ; ++k) {
#pragma unroll
        for (int v = 0; v < 4; ++v) o[k][v] *= av[v];
      }
    }
    float p[4], psum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = (sv[v] == -INFINITY) ? 0.f : exp2f(sv[v] - m_run);
      psum += p[v];
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;
    const v4s pf = pack4(p[0], p[1], p[2], p[3]);
#pragma unroll
    for (int s = 0; s < NSQ; ++s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4f vt = {0.f, 0.f, 0.f, 0.f};
        vt = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ring[slot][s].h[h], ident, vt, 0, 0, 0);
        const v4s vb = pack4(vt[0], vt[1], vt[2], vt[3]);     // exact: the values are bf16
        o[2 * s + h] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pf, vb, o[2 * s + h], 0, 0, 0);
      }
    }
  };
  for (int c0 = 0; c0 < n_chunks; c0 += RING) {
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      if (c0 + k < n_chunks) {
        issue(c0 + k + RING - 1, (k + RING - 1) % RING);    // keep RING-1 chunks ahead in flight
        chunk(c0 + k, k);
      }
    }
  }

  // ---- every wave holds the same (m, l) and its own channels of O: normalise and write -------
  // O element (block 2s+h, v) of lane (r, g): head 4g+v, channel ch0 + 32s + 8(r>>2) + 4h + (r&3)
  float lv[4], mv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { lv[v] = __shfl(l_run, 4 * g + v, 64); mv[v] = __shfl(m_run, 4 * g + v, 64); }
  const bool direct = a.plan.n_splits == 1;
  float *po = static_cast<float *>(a.workspace);
  float *plse = po + n_queries * a.H * a.plan.n_splits * D;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int gh = hb * 16 + 4 * g + v;
    if (gh >= a.H) continue;
    const float invL = lv[v] > 0.f ? 1.0f / lv[v] : 0.f;
#pragma unroll
    for (int s = 0; s < NSQ; ++s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = ch0 + 32 * s + 8 * (r >> 2) + 4 * h + (r & 3);
        const float x = o[2 * s + h][v] * invL;
        if (direct) a.out[(qi * a.H + gh) * D + ch] = __builtin_bit_cast(uint16_t, __bf16(x));
        else po[((qi * a.H + gh) * a.plan.n_splits + split) * int64_t(D) + ch] = x;
      }
    }
    if (wave == 0 && r == 0) {
      const float lse2 = lv[v] > 0.f ? mv[v] + log2f(lv[v]) : -INFINITY;
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
  const int64_t qh = blockIdx.x;                  // query * H + head
  const int ns = a.plan.n_splits;
  const float *po = static_cast<const float *>(a.workspace) + qh * ns * int64_t(D);
  const float *plse = static_cast<const float *>(a.workspace) + n_queries * a.H * ns * int64_t(D) + qh * ns;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, plse[s]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int ch = threadIdx.x * 4;
  for (int s = 0; s < ns; ++s) {
    const float ls = plse[s];
    const float wgt = (ls == -INFINITY) ? 0.f : exp2f(ls - M);
    L += wgt;
    const float4 x = *reinterpret_cast<const float4 *>(po + s * int64_t(D) + ch);
    acc.x += wgt * x.x; acc.y += wgt * x.y; acc.z += wgt * x.z; acc.w += wgt * x.w;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  uint16_t *dst = a.out + qh * D + ch;
  *reinterpret_cast<v4s *>(dst) = pack4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse && threadIdx.x == 0) a.lse[qh] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

}  // namespace

AttendPlan plan_attend(int64_t n_queries, int H, int64_t n_sel, int window) {
  AttendPlan p;
  p.n_hb = (H + 15) / 16;
  p.n_rows = int(n_sel + window);
  const int64_t pairs = n_queries * p.n_hb;
  int64_t splits = (512 + pairs - 1) / pairs;
  const int64_t max_splits = (p.n_rows + 127) / 128;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t rps = (p.n_rows + splits - 1) / splits;
  rps = (rps + 15) / 16 * 16;
  if (rps > kMaxRowsPerSplit) rps = kMaxRowsPerSplit;
  p.rows_per_split = int(rps);
  p.n_splits = int((p.n_rows + rps - 1) / rps);
  return p;
}

size_t attend_workspace_bytes(int64_t n_queries, int H, int D, int64_t n_sel, int window) {
  AttendPlan p = plan_attend(n_queries, H, n_sel, window);
  if (p.n_splits == 1) return 256;
  return size_t(n_queries * H * p.n_splits * (int64_t(D) + 1) * 4 + 256);
}

hipError_t launch_attend(const AttendArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  const int64_t nq = int64_t(a.B) * a.Sq;
  const int64_t pairs = nq * a.plan.n_splits;
  dim3 grid(unsigned(((pairs + 7) / 8) * 8 * a.plan.n_hb));
  switch (a.D) {
    case 64: e = launch("attend_split", attend_split_kernel<64>, grid, dim3(64 * waves_of<64>()), stream, a, nq); break;
    case 128: e = launch("attend_split", attend_split_kernel<128>, grid, dim3(64 * waves_of<128>()), stream, a, nq); break;
    case 256: e = launch("attend_split", attend_split_kernel<256>, grid, dim3(64 * waves_of<256>()), stream, a, nq); break;
    case 512: e = launch("attend_split", attend_split_kernel<512>, grid, dim3(64 * waves_of<512>()), stream, a, nq); break;
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
