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

__device__ __forceinline__ v4s pack4(float a, float b, float c, float d) {
  uint32_t lo = pack_bf16x2(a, b), hi = pack_bf16x2(c, d);
  v4s r;
  r[0] = short(lo & 0xffff); r[1] = short(lo >> 16); r[2] = short(hi & 0xffff); r[3] = short(hi >> 16);
  return r;
}

// Row pointer for slot `ri` of the query's row list, or nullptr when the slot is empty.
__device__ __forceinline__ const uint16_t *row_ptr(const AttendArgs &a, int64_t qi, int b, int64_t t,
                                                  int64_t n_vis, int64_t ri) {
  if (ri < a.n_sel) {
    int64_t e;
    if (a.topk_idx) {
      e = a.topk_idx[qi * a.n_sel + ri];
      if (e < 0 || e >= a.N_cap) return nullptr;
    } else {
      e = ri;
      if (e >= n_vis) return nullptr;
    }
    return a.entries + (int64_t(b) * a.N_cap + e) * a.D;
  }
  const int64_t w = ri - a.n_sel;
  if (w >= a.window) return nullptr;
  const int64_t p = t - a.window + 1 + w;                  // window position
  if (p < 0) return nullptr;
  const int64_t wr = p - a.win_pos0[b];
  if (wr < 0 || wr >= a.W_cap) return nullptr;
  return a.win_rows + (int64_t(b) * a.W_cap + wr) * a.D;
}

template <int D>
__global__ void __launch_bounds__(256) attend_split_kernel(AttendArgs a) {
  constexpr int NS = D / 32;          // 32-channel steps
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int split = blockIdx.x, hb = blockIdx.y;
  const int64_t qi = blockIdx.z;
  const int b = int(qi / a.Sq), s_idx = int(qi % a.Sq);
  const int64_t t = a.q_pos0[b] + s_idx;
  const int64_t n_vis = a.topk_idx ? 0 : min(a.n_entries[b], (t + 1) / a.m);
  const int head = hb * 16 + r;
  const bool head_ok = head < a.H;

  // ---- q^ = RoPE(RMSNorm(q)) * scale * log2(e), as B operands: lane holds channels 32s+8g..+7
  Frag8 qf[NS];
  {
    float qv[NS][8];
    const uint16_t *qrow = a.q + (qi * a.H + (head_ok ? head : 0)) * D;
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint4 w = head_ok ? *reinterpret_cast<const uint4 *>(qrow + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);
      qv[s][0] = bf16lo(w.x); qv[s][1] = bf16hi(w.x); qv[s][2] = bf16lo(w.y); qv[s][3] = bf16hi(w.y);
      qv[s][4] = bf16lo(w.z); qv[s][5] = bf16hi(w.z); qv[s][6] = bf16lo(w.w); qv[s][7] = bf16hi(w.w);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += qv[s][j] * qv[s][j];
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = rsqrtf(ss / float(D) + a.eps) * a.scale_log2;
    const int rope0 = D - a.rope_dim;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ch = 32 * s + 8 * g + j;
        qv[s][j] *= inv * (a.q_norm_w ? bf16_to_f32(a.q_norm_w[ch]) : 1.0f);
      }
      if (32 * s + 8 * g + 8 > rope0) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int ch = 32 * s + 8 * g + j;
          if (ch >= rope0) {
            float cs, sn;
            rope_cos_sin(t, (ch - rope0) >> 1, a.rope_dim, a.log2_base, &cs, &sn);
            const float x0 = qv[s][j], x1 = qv[s][j + 1];
            qv[s][j] = x0 * cs - x1 * sn;
            qv[s][j + 1] = x0 * sn + x1 * cs;
          }
        }
      }
      qf[s].u = make_uint4(pack_bf16x2(qv[s][0], qv[s][1]), pack_bf16x2(qv[s][2], qv[s][3]),
                           pack_bf16x2(qv[s][4], qv[s][5]), pack_bf16x2(qv[s][6], qv[s][7]));
    }
  }
  // identity fragment for the V transposes: element j of lane (n, g) is 1 iff n = 4g + j
  v4s ident;
#pragma unroll
  for (int j = 0; j < 4; ++j) ident[j] = ((r >> 2) == g && (r & 3) == j) ? short(0x3f80) : short(0);

  v4f o[2 * NS];
#pragma unroll
  for (int k = 0; k < 2 * NS; ++k) o[k] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t r0 = int64_t(split) * a.plan.rows_per_split;
  const int64_t r1 = min(int64_t(a.plan.n_rows), r0 + a.plan.rows_per_split);
  const int n_chunks = int((r1 - r0 + 15) / 16);
  Frag8 kv[NS];
  const uint16_t *rp = nullptr;
  int c = wave;
  if (c < n_chunks) {
    const int64_t ri = r0 + int64_t(c) * 16 + r;
    rp = ri < r1 ? row_ptr(a, qi, b, t, n_vis, ri) : nullptr;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      kv[s].u = rp ? *reinterpret_cast<const uint4 *>(rp + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);
  }
  for (; c < n_chunks; c += 4) {
    // row validity of the 16 rows of this chunk (lane r holds row r)
    const uint64_t vmask = __ballot(rp != nullptr);
    // prefetch the next chunk of this wave
    Frag8 nx[NS];
    const uint16_t *np = nullptr;
    const int cn = c + 4;
    if (cn < n_chunks) {
      const int64_t ri = r0 + int64_t(cn) * 16 + r;
      np = ri < r1 ? row_ptr(a, qi, b, t, n_vis, ri) : nullptr;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        nx[s].u = np ? *reinterpret_cast<const uint4 *>(np + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);
    }
    // S^T: lane (r, g) element v = <q^_head(r), row 4g+v>
    v4f st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[s].b, qf[s].b, st, 0, 0, 0);
    float sv[4], cmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = ((vmask >> (4 * g + v)) & 1) ? st[v] : -INFINITY;
      cmax = fmaxf(cmax, sv[v]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    float p[4], psum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = (sv[v] == -INFINITY) ? 0.f : exp2f(sv[v] - m_new);
      psum += p[v];
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // O rows are heads 4g+v: fetch their rescale factors from lanes 4g+v
    float av[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
    for (int k = 0; k < 2 * NS; ++k) {
#pragma unroll
      for (int v = 0; v < 4; ++v) o[k][v] *= av[v];
    }
    const v4s pf = pack4(p[0], p[1], p[2], p[3]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4f vt = {0.f, 0.f, 0.f, 0.f};
        vt = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kv[s].h[h], ident, vt, 0, 0, 0);
        const v4s vb = pack4(vt[0], vt[1], vt[2], vt[3]);
        o[2 * s + h] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pf, vb, o[2 * s + h], 0, 0, 0);
      }
    }
    if (cn < n_chunks) {
#pragma unroll
      for (int s = 0; s < NS; ++s) kv[s] = nx[s];
      rp = np;
    }
  }

  // ---- merge the four waves --------------------------------------------------------------
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ float s_o[16][D];
  if (lane < 16) { s_m[wave][r] = m_run; s_l[wave][r] = l_run; }
  __syncthreads();
  float cw[4];                           // this wave's weight for heads 4g+v
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = 4 * g + v;
    const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    const float mw = s_m[wave][h];
    cw[v] = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
  }
  // O element (block 2s+h, v) of lane (r, g): head 4g+v, channel 32s + 8(r>>2) + 4h + (r&3)
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ch = 32 * s + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float x = o[2 * s + h][v] * cw[v];
            if (w == 0) s_o[4 * g + v][ch] = x; else s_o[4 * g + v][ch] += x;
          }
        }
      }
    }
    __syncthreads();
  }
  // normalise and write: the partial of this slice, or the final output when there is one slice
  const bool direct = a.plan.n_splits == 1;
  for (int i = threadIdx.x; i < 16 * D / 4; i += 256) {
    const int h = i / (D / 4), ch = (i % (D / 4)) * 4;
    const int gh = hb * 16 + h;
    if (gh >= a.H) continue;
    float L = 0.f, M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
#pragma unroll
    for (int w = 0; w < 4; ++w) L += (s_m[w][h] == -INFINITY) ? 0.f : s_l[w][h] * exp2f(s_m[w][h] - M);
    const float invL = L > 0.f ? 1.0f / L : 0.f;
    const float4 x = make_float4(s_o[h][ch] * invL, s_o[h][ch + 1] * invL, s_o[h][ch + 2] * invL,
                                 s_o[h][ch + 3] * invL);
    if (direct) {
      uint16_t *dst = a.out + (qi * a.H + gh) * D + ch;
      *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
      if (a.lse && ch == 0) a.lse[qi * a.H + gh] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
    } else {
      float *po = static_cast<float *>(a.workspace) +
                  ((qi * a.H + gh) * a.plan.n_splits + split) * int64_t(D);
      *reinterpret_cast<float4 *>(po + ch) = x;
      if (ch == 0) {
        float *plse = static_cast<float *>(a.workspace) +
                      int64_t(gridDim.z) * a.H * a.plan.n_splits * D;
        plse[(qi * a.H + gh) * a.plan.n_splits + split] = L > 0.f ? M + log2f(L) : -INFINITY;
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
  *reinterpret_cast<uint2 *>(dst) =
      make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
  if (a.lse && threadIdx.x == 0) a.lse[qh] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

}  // namespace

AttendPlan plan_attend(int64_t n_queries, int H, int64_t n_sel, int window) {
  AttendPlan p;
  p.n_hb = (H + 15) / 16;
  p.n_rows = int(n_sel + window);
  const int64_t pairs = n_queries * p.n_hb;
  int64_t splits = (256 + pairs - 1) / pairs;
  const int64_t max_splits = (p.n_rows + 63) / 64;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t rps = (p.n_rows + splits - 1) / splits;
  rps = (rps + 63) / 64 * 64;
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
  dim3 grid(unsigned(a.plan.n_splits), unsigned(a.plan.n_hb), unsigned(int64_t(a.B) * a.Sq));
  switch (a.D) {
    case 64: hipLaunchKernelGGL(attend_split_kernel<64>, grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(attend_split_kernel<128>, grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(attend_split_kernel<256>, grid, dim3(256), 0, stream, a); break;
    case 512: hipLaunchKernelGGL(attend_split_kernel<512>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const AttendArgs &a, hipStream_t stream) {
  if (a.plan.n_splits == 1) return hipSuccess;
  const int64_t nq = int64_t(a.B) * a.Sq;
  dim3 grid(unsigned(nq * a.H));
  switch (a.D) {
    case 64: hipLaunchKernelGGL(attend_combine_kernel<64>, grid, dim3(16), 0, stream, a, nq); break;
    case 128: hipLaunchKernelGGL(attend_combine_kernel<128>, grid, dim3(32), 0, stream, a, nq); break;
    case 256: hipLaunchKernelGGL(attend_combine_kernel<256>, grid, dim3(64), 0, stream, a, nq); break;
    case 512: hipLaunchKernelGGL(attend_combine_kernel<512>, grid, dim3(128), 0, stream, a, nq); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa
