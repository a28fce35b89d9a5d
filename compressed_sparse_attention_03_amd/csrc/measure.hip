// A plain streaming read: the bandwidth a bandwidth-bound kernel of this library can hope for on
// the device it runs on, measured the same way (HIP events carried in the dispatch).  Every 16-byte
// word of one buffer is read once, in order, by 4,096 workgroups of 512 threads, four loads in
// flight per thread; the words are folded into a checksum that is stored only when it equals a
// constant, so the compiler keeps the loads and almost nothing is written.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace csa {
namespace {

typedef unsigned int w4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 4;
constexpr int kReadGroups = 4096;
constexpr uint32_t kNever = 0x9e3779b9u;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const w4 *__restrict__ src, int64_t n_words,
                                                                   int64_t per_group, uint32_t *__restrict__ sink) {
  const int64_t begin = int64_t(blockIdx.x) * per_group;
  const int64_t end = begin + per_group < n_words ? begin + per_group : n_words;
  uint32_t acc = 0;
  for (int64_t i = begin + threadIdx.x; i < end; i += int64_t(kReadThreads) * kReadUnroll) {
    w4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t j = i + int64_t(u) * kReadThreads;
      v[u] = j < end ? src[j] : w4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kNever) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream) {
  const int64_t n_words = bytes / 16;
  int64_t groups = (n_words + kReadThreads - 1) / kReadThreads;
  if (groups > kReadGroups) groups = kReadGroups;
  const int64_t per_group = (n_words + groups - 1) / groups;
  return launch("stream_read", stream_read_kernel, dim3(unsigned(groups)), dim3(kReadThreads), stream,
                reinterpret_cast<const w4 *>(src), n_words, per_group, sink);
}

}  // namespace csa
