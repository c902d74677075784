// Per-query bit allocation kernel: one wavefront per query (the rule and its
// closed form are described with allocate_query_wave).
#include "allocate_wave.h"
#include "fathom.h"

namespace fathom {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(kWavesPerBlock * 64) void allocate_kernel(
    const float* __restrict__ q, int num_q, int group, const float* __restrict__ var, int budget,
    uint8_t* __restrict__ alloc) {
  __shared__ uint32_t scratch[kWavesPerBlock][64];   // per wavefront, for the rank selection
  const int lane = threadIdx.x & 63;
  const int qi = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (qi >= num_q) return;                 // uniform per wavefront
  const int h = qi / group;
  const uint2 b = allocate_query_wave(q + int64_t(qi) * kD, var + int64_t(h) * kD, budget, &scratch[threadIdx.x >> 6][0]);
  const uint16_t pair = static_cast<uint16_t>(b.x | (b.y << 8));
  *reinterpret_cast<uint16_t*>(alloc + int64_t(qi) * kD + 2 * lane) = pair;
}

// Fixed-depth control reads: one wavefront per query ranks its channels by
// |q_c| (descending, ties to the lower index) and gives the leading ones the
// budget -- one plane each on top of a uniform depth (uniform), or whole
// 4-plane channels (top channels).  Lane l owns channels 2l and 2l + 1.
__global__ __launch_bounds__(kWavesPerBlock * 64) void control_allocate_kernel(
    const float* __restrict__ q, int num_q, int mode, int budget, uint8_t* __restrict__ alloc) {
  __shared__ uint32_t mag[kWavesPerBlock][kD];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qi = blockIdx.x * kWavesPerBlock + w;
  if (qi >= num_q) return;                 // uniform per wavefront (no barrier below)
  const float2 qv = *reinterpret_cast<const float2*>(q + int64_t(qi) * kD + 2 * lane);
  // |q| as bits: for non-negative floats the bit pattern orders like the value
  const uint32_t a0 = __float_as_uint(fabsf(qv.x)), a1 = __float_as_uint(fabsf(qv.y));
  mag[w][2 * lane] = a0;
  mag[w][2 * lane + 1] = a1;
  __builtin_amdgcn_wave_barrier();
  const int c0 = 2 * lane, c1 = c0 + 1;
  int r0 = 0, r1 = 0;   // channels ordered before c0, c1
  for (int i = 0; i < kD; i += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(&mag[w][i]);
    const uint32_t m[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r0 += (m[e] > a0 || (m[e] == a0 && i + e < c0)) ? 1 : 0;
      r1 += (m[e] > a1 || (m[e] == a1 && i + e < c1)) ? 1 : 0;
    }
  }
  int b0, b1;
  if (mode == FATHOM_CONTROL_TOP_CHANNELS) {
    const int r = budget / kPlanes, rem = budget % kPlanes;
    b0 = r0 < r ? kPlanes : (r0 == r ? rem : 0);
    b1 = r1 < r ? kPlanes : (r1 == r ? rem : 0);
  } else {
    const int base = budget / kD, rem = budget % kD;
    b0 = base + (r0 < rem ? 1 : 0);
    b1 = base + (r1 < rem ? 1 : 0);
  }
  const uint16_t pair = static_cast<uint16_t>(b0 | (b1 << 8));
  *reinterpret_cast<uint16_t*>(alloc + int64_t(qi) * kD + 2 * lane) = pair;
}

}  // namespace

hipError_t launch_control_allocate(const float* q, int num_q, int mode, int budget, uint8_t* alloc,
                                   hipStream_t stream) {
  const int blocks = (num_q + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(control_allocate_kernel, dim3(blocks), dim3(kWavesPerBlock * 64), 0, stream, q, num_q,
                     mode, budget, alloc);
  return hipGetLastError();
}

hipError_t launch_allocate(const float* q, int num_q, int group, const float* var, int budget,
                           uint8_t* alloc, hipStream_t stream) {
  const int blocks = (num_q + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(allocate_kernel, dim3(blocks), dim3(kWavesPerBlock * 64), 0, stream, q, num_q,
                     group, var, budget, alloc);
  return hipGetLastError();
}

}  // namespace fathom
