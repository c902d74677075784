// Measurement aid: a plain streaming read of a device buffer, the HBM read
// ceiling the scan's roofline fraction is compared against.  Every 16-byte
// word is loaded once with the non-temporal policy the scan's plane loads
// use; the words are folded into a value that is stored only if it equals a
// constant no input is expected to produce, so no load can be removed and
// almost nothing is written.

#include "fathom_internal.h"

namespace fathom {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const v4u* __restrict__ src, int64_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * kStreamThreads;
  int64_t i = int64_t(blockIdx.x) * kStreamThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    v4u v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const v4u v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

int stream_read_blocks() { return 256 * 8; }

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(stream_read_blocks()), dim3(kStreamThreads), 0, stream,
                     static_cast<const v4u*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace fathom
