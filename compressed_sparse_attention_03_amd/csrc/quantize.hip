// Quantise-on-write of lightning-indexer keys (fp8 e4m3 with a power-of-two row scale, or OCP
// MXFP4).  "How DeepSeek-V4 Achieves Million-Token Contexts..." (dev.to), "Two Compression
// Strategies": the indexer runs in FP4; "Follow the white rabbit" (sambatista.com), indexer
// paragraph: the indexer works on compact, low-precision operands.
//
// One wave per row, each lane owns 32/64-aligned runs of the row; integer-exact rules stated in
// csa.h.
#include "common.h"
#include "internal.h"

namespace csa {
namespace {

// fp8: one wave per row; lane j covers channels [j*dim/64 ...] in runs of 8 (dim <= 512) or a
// strided loop otherwise.
__global__ void __launch_bounds__(256) quantize_fp8_kernel(const uint16_t *x, uint8_t *codes,
                                                           float *scales, int64_t rows, int dim) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t *xr = x + row * dim;
  float amax = 0.f;
  for (int c = lane; c < dim; c += 64) amax = fmaxf(amax, fabsf(bf16_to_f32(xr[c])));
  amax = wave_max(amax);
  const int e = e4m3_row_exp(amax);
  const float inv = ldexpf(1.0f, -e);                       // exact power of two
  for (int c = lane * 4; c < dim; c += 256) {
    uint2 w = *reinterpret_cast<const uint2 *>(xr + c);
    uint32_t b0 = f32_to_e4m3(bf16lo(w.x) * inv), b1 = f32_to_e4m3(bf16hi(w.x) * inv);
    uint32_t b2 = f32_to_e4m3(bf16lo(w.y) * inv), b3 = f32_to_e4m3(bf16hi(w.y) * inv);
    *reinterpret_cast<uint32_t *>(codes + row * dim + c) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }
  if (lane == 0) scales[row] = ldexpf(1.0f, e);
}

// MXFP4: one thread per block of 32 values.
__global__ void __launch_bounds__(256) quantize_mxfp4_kernel(const uint16_t *x, uint8_t *codes,
                                                             uint8_t *scales, int64_t n_blocks) {
  const int64_t blk = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (blk >= n_blocks) return;
  const uint4 *src = reinterpret_cast<const uint4 *>(x + blk * 32);
  uint32_t w[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 v = src[q];
    w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(w[q])), fabsf(bf16hi(w[q]))));
  const uint32_t sb = mx_scale_byte(amax);
  const float inv = ldexpf(1.0f, 127 - int(sb));
  uint32_t out[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t lo = f32_to_e2m1(bf16lo(w[4 * q + k]) * inv);
      uint32_t hi = f32_to_e2m1(bf16hi(w[4 * q + k]) * inv);
      packed |= (lo | (hi << 4)) << (8 * k);
    }
    out[q] = packed;
  }
  *reinterpret_cast<uint4 *>(codes + blk * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  scales[blk] = uint8_t(sb);
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs &a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.rows == 0) return hipSuccess;
  if (a.format == 1) {
    dim3 grid(unsigned((a.rows + 3) / 4));
    e = launch("quantize", quantize_fp8_kernel, grid, dim3(256), stream, a.x,
                       static_cast<uint8_t *>(a.codes), static_cast<float *>(a.scales), a.rows, a.dim);
  } else {
    const int64_t nb = a.rows * (a.dim / 32);
    dim3 grid(unsigned((nb + 255) / 256));
    e = launch("quantize", quantize_mxfp4_kernel, grid, dim3(256), stream, a.x,
                       static_cast<uint8_t *>(a.codes), static_cast<uint8_t *>(a.scales), nb);
  }
  return e;
}

}  // namespace csa
