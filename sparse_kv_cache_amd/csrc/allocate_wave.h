// Per-query bit allocation by reverse water-filling, computed by one
// wavefront (lane l owns channels 2l and 2l + 1 of the d = 128).
//
// "Fathom Makes KV-Cache Scans Query-Adaptive for Long-Context Decoding",
// para 3: a total bit budget is spread over the channels of each query by a
// reverse water-filling rule with a closed-form solution.  "Fathom: Per-Query
// Read Depth for Sparse Decoding over Offloaded KV Caches", abstract s2-s3:
// the weights are the variance-weighted importances of the query's channels.
//
// Channel c of query q has importance w_c = fl32(fl32(q_c^2) var_c); reading
// plane j of it (j = 0..3) is worth w_c 4^-j.  The B most valuable candidates
// (c, j) form the allocation.  In closed form: with the water level theta =
// the B-th largest ordering key bits(w_c) - j 2^24, channel c takes every
// plane whose key exceeds theta, and the candidates equal to theta (at most
// one per channel) are filled in ascending channel order until sum b_c = B.
// theta is found by bisection on the int32 key with wavefront ballot counts.
#ifndef FATHOM_ALLOCATE_WAVE_H
#define FATHOM_ALLOCATE_WAVE_H

#include "fathom_internal.h"

namespace fathom {
namespace alloc_detail {

constexpr int kKeyStep = 1 << 24;

__device__ inline int wave_count(bool pred) { return __popcll(__ballot(pred)); }

__device__ inline int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  return __popcll(mask & below);
}

}  // namespace alloc_detail

// Allocation of one query: q_row and var_row are its d = 128 query values and
// its KV head's channel variances.  Returns (b_{2l}, b_{2l+1}) for lane l.
// Every lane of the wavefront must call it (ballots).
__device__ inline uint2 allocate_query_wave(const float* __restrict__ q_row, const float* __restrict__ var_row,
                                            int budget) {
  using namespace alloc_detail;
  const int lane = threadIdx.x & 63;
  const int c0 = 2 * lane;
  const float2 qv = *reinterpret_cast<const float2*>(q_row + c0);
  const float2 vv = *reinterpret_cast<const float2*>(var_row + c0);
  const float w0 = __fmul_rn(__fmul_rn(qv.x, qv.x), vv.x);
  const float w1 = __fmul_rn(__fmul_rn(qv.y, qv.y), vv.y);
  const int k0 = __float_as_int(w0);       // w >= 0, so the bit pattern orders like the value
  const int k1 = __float_as_int(w1);
  // count of candidates with key >= t
  auto count_ge = [&](long long t) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) {
      cnt += wave_count(static_cast<long long>(k0) - j * kKeyStep >= t);
      cnt += wave_count(static_cast<long long>(k1) - j * kKeyStep >= t);
    }
    return cnt;
  };
  int b0 = 0, b1 = 0;
  if (budget >= kPlanes * kD) {
    b0 = b1 = kPlanes;
  } else if (budget > 0) {
    long long lo = -3ll * kKeyStep;        // count_ge(lo) = 4d >= budget
    long long hi = 0x7f800001ll;           // above every finite key: count_ge(hi) = 0
    while (hi - lo > 1) {
      const long long mid = lo + (hi - lo) / 2;
      if (count_ge(mid) >= budget) lo = mid; else hi = mid;
    }
    const long long theta = lo;            // the budget-th largest key
    int gt0 = 0, gt1 = 0;
    bool tie0 = false, tie1 = false;
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) {
      const long long a = static_cast<long long>(k0) - j * kKeyStep;
      const long long b = static_cast<long long>(k1) - j * kKeyStep;
      gt0 += a > theta;
      gt1 += b > theta;
      tie0 |= a == theta;
      tie1 |= b == theta;
    }
    int total_gt = 0;
    for (int j = 1; j <= kPlanes; ++j) total_gt += j * (wave_count(gt0 == j) + wave_count(gt1 == j));
    const int need = budget - total_gt;    // candidates taken from the tie at theta
    const uint64_t t0 = __ballot(tie0), t1 = __ballot(tie1);
    const int rank0 = lanes_below(t0) + lanes_below(t1);   // ties in channels < c0
    const int rank1 = rank0 + (tie0 ? 1 : 0);
    b0 = gt0 + ((tie0 && rank0 < need) ? 1 : 0);
    b1 = gt1 + ((tie1 && rank1 < need) ? 1 : 0);
  }
  return make_uint2(static_cast<uint32_t>(b0), static_cast<uint32_t>(b1));
}

}  // namespace fathom

#endif  // FATHOM_ALLOCATE_WAVE_H
