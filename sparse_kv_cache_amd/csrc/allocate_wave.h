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
// theta is found by a search on the int32 key with wavefront counts.
#ifndef FATHOM_ALLOCATE_WAVE_H
#define FATHOM_ALLOCATE_WAVE_H

#include "fathom_internal.h"
#include "wave_ops.h"

namespace fathom {
namespace alloc_detail {

constexpr int kKeyStep = 1 << 24;

__device__ inline int wave_count(bool pred) { return __popcll(__ballot(pred)); }

// Sum over the wavefront's 64 lanes, returned to every lane (DPP row shifts
// give each row's inclusive prefix, row broadcasts carry it across rows).
__device__ inline uint32_t wave_sum_u32(uint32_t v) {
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

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
  // The search runs on u = key - kKeyLo, which is >= 0 for every candidate
  // key and below 2^32, so all of it is 32-bit unsigned arithmetic.
  // Candidates of channel c with u >= t: the keys k_c - j 2^24 (j = 0..3)
  // are evenly spaced, so that is min(4, (u_c - t) / 2^24 + 1) when u_c >= t.
  constexpr uint32_t kKeyLo = static_cast<uint32_t>(-3 * kKeyStep);   // -3 2^24 as a bit pattern
  const uint32_t u0 = static_cast<uint32_t>(k0) - kKeyLo, u1 = static_cast<uint32_t>(k1) - kKeyLo;
  auto cnt1 = [](uint32_t u, uint32_t t) -> uint32_t { return u >= t ? min(4u, ((u - t) >> 24) + 1u) : 0u; };
  int b0 = 0, b1 = 0;
  if (budget >= kPlanes * kD) {
    b0 = b1 = kPlanes;
  } else if (budget > 0) {
    // Search for the budget-th largest key with three probes per round:
    // their counts (each <= 4d = 512 < 2^10) are packed into one word, so one
    // wavefront sum serves all three.  Invariant: count(lo) >= budget >
    // count(hi).  The start bracket comes from the lanes' larger keys in
    // descending order, M_1 >= M_2 >= ...: with r = ceil(budget / 4), the r
    // lanes whose larger key is >= M_r each have a channel with all four
    // candidates >= M_r - 3 2^24, so that key counts >= 4r >= budget; and
    // fewer than r' = ceil(r / 2) lanes hold a key above M_r', at most two
    // channels each, so M_r' + 1 counts <= 8 (r' - 1) < budget.
    const uint32_t B = static_cast<uint32_t>(budget);
    const int r = (budget + 3) / 4, r2 = (r + 1) / 2;   // r in 1..128, r2 in 1..64
    const uint32_t msort = wave_sort_desc(static_cast<uint32_t>(max(k0, k1)));   // keys are >= 0
    const uint32_t m_r = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(msort), min(r, 64) - 1));
    const uint32_t m_r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(msort), r2 - 1));
    uint32_t lo = r <= 64 ? m_r : 0u;                      // key M_r - 3 2^24 (else -3 2^24: count 4d)
    uint32_t hi = m_r2 + 1u - kKeyLo;                      // key M_r' + 1
    while (hi - lo > 1u) {
      const uint32_t step = max(1u, (hi - lo) / 4u);
      const uint32_t t1 = min(lo + step, hi - 1u);
      const uint32_t t2 = min(t1 + step, hi - 1u);
      const uint32_t t3 = min(t2 + step, hi - 1u);
      uint32_t packed = (cnt1(u0, t1) + cnt1(u1, t1)) | ((cnt1(u0, t2) + cnt1(u1, t2)) << 10) |
                        ((cnt1(u0, t3) + cnt1(u1, t3)) << 20);
      packed = wave_sum_u32(packed);
      const uint32_t c1 = packed & 1023u, c2 = (packed >> 10) & 1023u, c3 = packed >> 20;
      if (c3 >= B) {
        lo = t3;
      } else if (c2 >= B) {
        lo = t2;
        hi = t3;
      } else if (c1 >= B) {
        lo = t1;
        hi = t2;
      } else {
        hi = t1;
      }
    }
    const long long theta = static_cast<long long>(static_cast<int>(lo + kKeyLo));   // the budget-th largest key
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
