// Per-query bit allocation kernel: one wavefront per query (the rule and its
// closed form are described with allocate_query_wave).
#include "allocate_wave.h"

namespace fathom {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(kWavesPerBlock * 64) void allocate_kernel(
    const float* __restrict__ q, int num_q, int group, const float* __restrict__ var, int budget,
    uint8_t* __restrict__ alloc) {
  const int lane = threadIdx.x & 63;
  const int qi = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (qi >= num_q) return;                 // uniform per wavefront
  const int h = qi / group;
  const uint2 b = allocate_query_wave(q + int64_t(qi) * kD, var + int64_t(h) * kD, budget);
  const uint16_t pair = static_cast<uint16_t>(b.x | (b.y << 8));
  *reinterpret_cast<uint16_t*>(alloc + int64_t(qi) * kD + 2 * lane) = pair;
}

}  // namespace

hipError_t launch_allocate(const float* q, int num_q, int group, const float* var, int budget,
                           uint8_t* alloc, hipStream_t stream) {
  const int blocks = (num_q + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(allocate_kernel, dim3(blocks), dim3(kWavesPerBlock * 64), 0, stream, q, num_q,
                     group, var, budget, alloc);
  return hipGetLastError();
}

}  // namespace fathom
