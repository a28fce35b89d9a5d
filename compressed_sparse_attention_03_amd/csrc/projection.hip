// Grouped output projection after core attention.
//
// "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence" (paperlayer summary),
// section 2.3, shared-KV and output-projection paragraph: both attention types map their many head
// outputs back to the model width through a projection split into groups, to cut that cost.
//
// y[m, g N_g + n] = sum_k o[m, g K_g + k] * w[g, n, k]: the heads fall into G groups; each group's
// concatenated head outputs (K_g = H D / G values) go through its own weight [N_g, K_g] (stored
// as a linear layer stores it: one row of K_g inputs per output).  bf16 in, fp32 accumulation on
// v_mfma_f32_16x16x32_bf16, bf16 out; no atomics (deterministic).
//
// Decode (M <= 16 tokens): the weights are streamed once -- a workgroup owns 16 output columns,
// its eight waves take an eighth of K each with eight 32-wide steps of loads in flight, and the
// partial sums are added in wave order through LDS.
// Larger M: a 128 x 128 output tile per workgroup, K in steps of 64 through double-buffered LDS
// (rows padded to 144 bytes so the 16 rows one fragment read touches fall in different banks);
// each wave computes a 64 x 64 quarter as 4 x 4 MFMA tiles.
#include "common.h"
#include "internal.h"

namespace csa {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));   // converted with v_cvt_pk_bf16_f32 (round to nearest even)
union F8 {
  uint4 u;
  v8bf b;
};

constexpr int kSmallWaves = 8;   // waves per workgroup of the small-M kernel; each takes 1/8 of K

__global__ void __launch_bounds__(64 * kSmallWaves) oproj_small_kernel(ProjArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16;                          // first output column of the workgroup
  const int g = n0 / a.N_g;
  const int K = a.K_g, kq = K / kSmallWaves;
  const int k_begin = wave * kq, k_end = k_begin + kq;
  // A operand: token row i (rows past M read the last row and are zeroed); B: weight row of
  // output column n0 + i; lane (i, q) takes the 8 values 8q .. 8q+7 of every 32-wide step
  const bool live = i < a.M;
  const uint16_t *arow = a.o + int64_t(live ? i : a.M - 1) * a.ldo + int64_t(g) * K + 8 * q;
  const uint16_t *brow = a.w + (int64_t(g) * a.N_g + (n0 - g * a.N_g) + i) * K + 8 * q;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;
  int k = k_begin;
  for (; k + 32 * U <= k_end; k += 32 * U) {
    F8 fa[U], fb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      fa[u].u = *reinterpret_cast<const uint4 *>(arow + k + 32 * u);
      fb[u].u = *reinterpret_cast<const uint4 *>(brow + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live) fa[u].u = make_uint4(0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[u].b, fb[u].b, acc, 0, 0, 0);
    }
  }
  for (; k < k_end; k += 32) {
    F8 fa, fb;
    fa.u = *reinterpret_cast<const uint4 *>(arow + k);
    fb.u = *reinterpret_cast<const uint4 *>(brow + k);
    if (!live) fa.u = make_uint4(0, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.b, fb.b, acc, 0, 0, 0);
  }
  __shared__ float4 red[kSmallWaves][64];
  red[wave][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  lds_barrier();
  if (wave != 0) return;
  float4 s = red[0][lane];
#pragma unroll
  for (int w = 1; w < kSmallWaves; ++w) {
    const float4 x = red[w][lane];
    s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
  }
  // lane (i, q) holds rows 4q .. 4q+3 of output column n0 + i
  const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (4 * q + r < a.M) a.y[int64_t(4 * q + r) * a.ldy + n0 + i] = f32_to_bf16(v[r]);
}

constexpr int kTile = 128;       // output tile rows and columns per workgroup
constexpr int kStep = 64;        // K per LDS stage
constexpr int kRowB = kStep + 8; // LDS row stride in bf16 (8 values of padding)

__global__ void __launch_bounds__(256) oproj_tiled_kernel(ProjArgs a) {
  __shared__ __align__(16) uint16_t s_a[2][kTile * kRowB];
  __shared__ __align__(16) uint16_t s_b[2][kTile * kRowB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;                   // the wave's 64 x 64 quarter
  const int64_t m0 = int64_t(blockIdx.y) * kTile;
  const int n0 = blockIdx.x * kTile;
  const int g = n0 / a.N_g;
  const int K = a.K_g;
  // global -> LDS: thread tid moves half (tid & 1) of row tid / 2 of the 64-wide step -- 64 bytes of
  // a token row (A) and of a weight row (B); the 256 threads cover all 128 rows of both
  const int lr = tid >> 1, lh = tid & 1;                     // rows 0..127, half 0/1 of 128 bytes
  const int64_t am = min(m0 + lr, int64_t(a.M) - 1);        // rows past M repeat the last (not stored)
  const uint16_t *ga = a.o + am * a.ldo + int64_t(g) * K + 32 * lh;
  const uint16_t *gb = a.w + (int64_t(g) * a.N_g + (n0 - g * a.N_g) + lr) * K + 32 * lh;
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;               // the next step's rows (named: no spill)
  auto load = [&](int k) __attribute__((always_inline)) {
    ra0 = *reinterpret_cast<const uint4 *>(ga + k);
    ra1 = *reinterpret_cast<const uint4 *>(ga + k + 8);
    ra2 = *reinterpret_cast<const uint4 *>(ga + k + 16);
    ra3 = *reinterpret_cast<const uint4 *>(ga + k + 24);
    rb0 = *reinterpret_cast<const uint4 *>(gb + k);
    rb1 = *reinterpret_cast<const uint4 *>(gb + k + 8);
    rb2 = *reinterpret_cast<const uint4 *>(gb + k + 16);
    rb3 = *reinterpret_cast<const uint4 *>(gb + k + 24);
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    uint4 *da = reinterpret_cast<uint4 *>(s_a[buf] + lr * kRowB + 32 * lh);
    uint4 *db = reinterpret_cast<uint4 *>(s_b[buf] + lr * kRowB + 32 * lh);
    da[0] = ra0; da[1] = ra1; da[2] = ra2; da[3] = ra3;
    db[0] = rb0; db[1] = rb1; db[2] = rb2; db[3] = rb3;
  };
  v4f acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = v4f{0.f, 0.f, 0.f, 0.f};
  const int steps = K / kStep;
  load(0);
  store(0);
  lds_barrier();
  for (int t = 0; t < steps; ++t) {
    const int buf = t & 1;
    if (t + 1 < steps) load(kStep * (t + 1));                // in flight while this step computes
#pragma unroll
    for (int kk = 0; kk < kStep; kk += 32) {
      F8 fa[4], fb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        fa[x].u = *reinterpret_cast<const uint4 *>(s_a[buf] + (wm * 64 + x * 16 + i) * kRowB + kk + 8 * q);
        fb[x].u = *reinterpret_cast<const uint4 *>(s_b[buf] + (wn * 64 + x * 16 + i) * kRowB + kk + 8 * q);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[x].b, fb[y].b, acc[x][y], 0, 0, 0);
    }
    if (t + 1 < steps) store(buf ^ 1);                       // the other buffer: last read a step ago
    lds_barrier();
  }
  // tile (x, y), lane (i, q): rows 4q .. 4q+3 of its 16, column i of its 16
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + x * 16 + 4 * q + r;
        if (m < a.M) a.y[m * a.ldy + n0 + wn * 64 + y * 16 + i] = f32_to_bf16(acc[x][y][r]);
      }
}

// Large M: a 256 x 256 output tile per workgroup (one per CU at 4,096 x 4,096), four waves of
// 128 x 128 each.  A wave's 8 x 8 accumulator tiles (256 values a lane) stay in accumulation
// registers until the end -- nothing but the MFMAs touches them -- so per 32-wide K step a wave
// reads 16 fragments from LDS for 64 MFMAs (twice the reuse of the 128-tile kernel, which is
// LDS-bound).  The products are taken as Y^T tiles (weight rows as the A operand, token rows as B),
// so a lane ends with four consecutive output columns of one token: one 8-byte store each.
// Global -> LDS: load l of thread tid is the 16-byte piece (tid % 8) of tile row 32 l + tid / 8, so
// one instruction reads eight whole 128-byte row segments.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBig = 256;         // output tile rows and columns per workgroup
constexpr int kBigStep = 64;      // K per LDS stage
constexpr int kBigRow = kBigStep + 8;

__global__ void __launch_bounds__(256, 1) oproj_big_kernel(ProjArgs a) {
  __shared__ __align__(16) uint16_t s_a[2][kBig * kBigRow];   // token rows
  __shared__ __align__(16) uint16_t s_b[2][kBig * kBigRow];   // weight rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;                     // the wave's 128 x 128 quarter
  // Workgroup -> tile.  Workgroups go to the 8 XCDs round-robin by linear id; when the groups
  // divide evenly, XCD x takes every tile of groups x, x + 8, ..., so a group's weights stay in one
  // L2, and the column tiles that share a token tile get neighbouring ids (same XCD, launched
  // together: the token tile is fetched once).
  const int n_sub = a.N_g / kBig, m_tiles = (a.M + kBig - 1) / kBig;
  const int L = blockIdx.x;
  int g, sub, mt;
  if (a.G % 8 == 0) {
    const int x = L & 7, j = L >> 3;
    g = x + 8 * (j / (n_sub * m_tiles));
    const int rest = j % (n_sub * m_tiles);
    mt = rest / n_sub;
    sub = rest % n_sub;
  } else {
    g = L / (n_sub * m_tiles);
    const int rest = L % (n_sub * m_tiles);
    mt = rest / n_sub;
    sub = rest % n_sub;
  }
  const int64_t m0 = int64_t(mt) * kBig;
  const int n0 = g * a.N_g + sub * kBig;
  const int K = a.K_g;
  const int lrow = tid >> 3, lp = tid & 7;
  const uint16_t *ga0 = a.o + int64_t(g) * K + 8 * lp;
  const uint16_t *gb0 = a.w + (int64_t(g) * a.N_g + (n0 - g * a.N_g) + lrow) * K + 8 * lp;
  u32x4 ra[8], rb[8];
  auto load = [&](int k) __attribute__((always_inline)) {
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const int64_t m = min(m0 + 32 * l + lrow, int64_t(a.M) - 1);  // rows past M repeat the last (not stored)
      ra[l] = *reinterpret_cast<const u32x4 *>(ga0 + m * a.ldo + k);
      rb[l] = *reinterpret_cast<const u32x4 *>(gb0 + int64_t(32 * l) * K + k);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      *reinterpret_cast<u32x4 *>(s_a[buf] + (32 * l + lrow) * kBigRow + 8 * lp) = ra[l];
      *reinterpret_cast<u32x4 *>(s_b[buf] + (32 * l + lrow) * kBigRow + 8 * lp) = rb[l];
    }
  };
  v4f acc[8][8];                                               // [weight tile y][token tile x]
#pragma unroll
  for (int y = 0; y < 8; ++y)
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[y][x] = v4f{0.f, 0.f, 0.f, 0.f};
  const int steps = K / kBigStep;
  load(0);
  store(0);
  lds_barrier();
  for (int t = 0; t < steps; ++t) {
    const int buf = t & 1;
    if (t + 1 < steps) load(kBigStep * (t + 1));               // in flight while this step computes
#pragma unroll 1
    for (int kk = 0; kk < kBigStep; kk += 32) {
      F8 fa[8];
#pragma unroll
      for (int x = 0; x < 8; ++x)
        fa[x].u = *reinterpret_cast<const uint4 *>(s_a[buf] + (wm * 128 + x * 16 + i) * kBigRow + kk + 8 * q);
#pragma unroll
      for (int y = 0; y < 8; ++y) {
        F8 fb;
        fb.u = *reinterpret_cast<const uint4 *>(s_b[buf] + (wn * 128 + y * 16 + i) * kBigRow + kk + 8 * q);
#pragma unroll
        for (int x = 0; x < 8; ++x)
          acc[y][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb.b, fa[x].b, acc[y][x], 0, 0, 0);
      }
    }
    if (t + 1 < steps) store(buf ^ 1);                          // the other buffer: last read a step ago
    lds_barrier();
  }
  // tile (y, x), lane (i, q): token row 16 x + i, output columns 16 y + 4 q .. +3
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int64_t m = m0 + wm * 128 + x * 16 + i;
    if (m < a.M) {
      uint16_t *dst = a.y + m * a.ldy + n0 + wn * 128 + 4 * q;
#pragma unroll
      for (int y = 0; y < 8; ++y) {
        *reinterpret_cast<v4bf *>(dst + 16 * y) =
            v4bf{__bf16(acc[y][x][0]), __bf16(acc[y][x][1]), __bf16(acc[y][x][2]), __bf16(acc[y][x][3])};
      }
    }
  }
}

}  // namespace

hipError_t launch_oproj(const ProjArgs &a, hipStream_t stream) {
  const int n_total = a.G * a.N_g;
  if (a.M <= 16)
    return launch("oproj", oproj_small_kernel, dim3(unsigned(n_total / 16)), dim3(64 * kSmallWaves), stream, a);
  if (a.M >= 512 && a.N_g % kBig == 0) {
    const dim3 grid(unsigned(int64_t(n_total / kBig) * ((a.M + kBig - 1) / kBig)));
    return launch("oproj", oproj_big_kernel, grid, dim3(256), stream, a);
  }
  const dim3 grid(unsigned(n_total / kTile), unsigned((a.M + kTile - 1) / kTile));
  return launch("oproj", oproj_tiled_kernel, grid, dim3(256), stream, a);
}

}  // namespace csa
