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
// theta is found in two stages: a search on the key's top byte with
// wavefront counts, then a rank selection on the low 24 bits of the channels
// whose count still changes inside that byte.
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

// r-th largest (1 <= r <= 64, r <= number of present values) of the
// wavefront's values v0, v1 (0 marks an absent value): the r-th largest lane
// maximum L has at least r values at or above it; when at most 64 do, they
// are compacted one per lane through scratch (64 words of LDS private to the
// wavefront) and sorted; otherwise a bisection with three probes per round
// finds the rank.
__device__ inline uint32_t rth_largest2(uint32_t v0, uint32_t v1, uint32_t r, uint32_t* scratch) {
  const int lane = threadIdx.x & 63;
  const uint32_t L = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(wave_sort_desc(max(v0, v1))), static_cast<int>(r) - 1));
  const uint64_t b0 = __ballot(v0 >= L), b1 = __ballot(v1 >= L);
  const uint32_t c = static_cast<uint32_t>(__popcll(b0) + __popcll(b1));
  if (L != 0u && c <= 64u) {   // uniform
    if (v0 >= L) scratch[lanes_below(b0)] = v0;
    if (v1 >= L) scratch[__popcll(b0) + lanes_below(b1)] = v1;
    __builtin_amdgcn_wave_barrier();
    const uint32_t x = static_cast<uint32_t>(lane) < c ? scratch[lane] : 0u;
    return static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(wave_sort_desc(x)), static_cast<int>(r) - 1));
  }
  // invariant: count(>= lo) >= r > count(>= hi); counts <= 128 fit 10 bits
  uint32_t lo = 0u, hi = 0xffffffffu;
  while (hi - lo > 1u) {
    const uint32_t step = max(1u, (hi - lo) / 4u);
    const uint32_t t1 = min(lo + step, hi - 1u);
    const uint32_t t2 = min(t1 + step, hi - 1u);
    const uint32_t t3 = min(t2 + step, hi - 1u);
    auto cnt = [&](uint32_t t) { return (v0 >= t ? 1u : 0u) + (v1 >= t ? 1u : 0u); };
    const uint32_t packed = wave_sum_u32(cnt(t1) | (cnt(t2) << 10) | (cnt(t3) << 20));
    if ((packed >> 20) >= r) {
      lo = t3;
    } else if (((packed >> 10) & 1023u) >= r) {
      lo = t2;
      hi = t3;
    } else if ((packed & 1023u) >= r) {
      lo = t1;
      hi = t2;
    } else {
      hi = t1;
    }
  }
  return lo;
}

}  // namespace alloc_detail

// Allocation of one query: q_row and var_row are its d = 128 query values and
// its KV head's channel variances.  Returns (b_{2l}, b_{2l+1}) for lane l.
// Every lane of the wavefront must call it (ballots).
__device__ inline uint2 allocate_query_wave(const float* __restrict__ q_row, const float* __restrict__ var_row,
                                            int budget, uint32_t* scratch) {
  using namespace alloc_detail;
  const int lane = threadIdx.x & 63;
  const int c0 = 2 * lane;
  const float2 qv = *reinterpret_cast<const float2*>(q_row + c0);
  const float2 vv = *reinterpret_cast<const float2*>(var_row + c0);
  // A variance is >= 0.  A weight that is not a positive number (a negative,
  // -0 or NaN var_c) is read as +0, so every weight is +0, positive or +inf
  // and its bit pattern orders like its value.
  float w0 = __fmul_rn(__fmul_rn(qv.x, qv.x), vv.x);
  float w1 = __fmul_rn(__fmul_rn(qv.y, qv.y), vv.y);
  w0 = w0 > 0.0f ? w0 : 0.0f;
  w1 = w1 > 0.0f ? w1 : 0.0f;
  const int k0 = __float_as_int(w0);
  const int k1 = __float_as_int(w1);
  // The search runs on u = key - kKeyLo, which is >= 3 2^24 for every
  // channel's top key (and >= 0 for every candidate) and below 2^32, so all
  // of it is 32-bit unsigned arithmetic.
  constexpr uint32_t kKeyLo = static_cast<uint32_t>(-3 * kKeyStep);   // -3 2^24 as a bit pattern
  const uint32_t u0 = static_cast<uint32_t>(k0) - kKeyLo, u1 = static_cast<uint32_t>(k1) - kKeyLo;
  int b0 = 0, b1 = 0;
  if (budget >= kPlanes * kD) {
    b0 = b1 = kPlanes;
  } else if (budget > 0) {
    // The budget-th largest candidate key, in two stages on u = U 2^24 + f
    // (U the top byte, f the low 24 bits).  Channel c's candidates are
    // u_c - j 2^24 (j = 0..3), so at t = T 2^24 it counts
    // clamp(U_c - T + 1, 0, 4).  Stage 1 finds the largest T whose count is
    // >= budget (three probes per round share one packed wavefront sum;
    // count(0) = 4d since every U_c >= 3, count(256) = 0).  Inside
    // [T 2^24, (T + 1) 2^24) only channels with a_c = U_c - T + 1 in 1..4
    // change count, each by one once t passes T 2^24 + f_c.  With
    // m = count(T 2^24) - budget, the key is therefore T 2^24 plus the
    // (m + 1)-th smallest f_c over those s channels (m < s, else the count
    // at (T + 1) 2^24 would still reach the budget).  Stage 2 takes that
    // rank from whichever end of the s values it is nearer, so it is <= 64.
    const uint32_t B = static_cast<uint32_t>(budget);
    const int U0 = static_cast<int>(u0 >> 24), U1 = static_cast<int>(u1 >> 24);
    auto chi = [](int U, int T) -> uint32_t { return static_cast<uint32_t>(min(4, max(0, U - T + 1))); };
    int tlo = 0, thi = 256;
    uint32_t clo = 4u * kD;   // count(tlo 2^24)
    while (thi - tlo > 1) {
      const int step = max(1, (thi - tlo) / 4);
      const int t1 = min(tlo + step, thi - 1);
      const int t2 = min(t1 + step, thi - 1);
      const int t3 = min(t2 + step, thi - 1);
      uint32_t packed = (chi(U0, t1) + chi(U1, t1)) | ((chi(U0, t2) + chi(U1, t2)) << 10) |
                        ((chi(U0, t3) + chi(U1, t3)) << 20);
      packed = wave_sum_u32(packed);
      const uint32_t n1 = packed & 1023u, n2 = (packed >> 10) & 1023u, n3 = packed >> 20;
      if (n3 >= B) {
        tlo = t3;
        clo = n3;
      } else if (n2 >= B) {
        tlo = t2;
        clo = n2;
        thi = t3;
      } else if (n1 >= B) {
        tlo = t1;
        clo = n1;
        thi = t2;
      } else {
        thi = t1;
      }
    }
    const bool s0 = U0 - tlo + 1 >= 1 && U0 - tlo + 1 <= 4, s1 = U1 - tlo + 1 >= 1 && U1 - tlo + 1 <= 4;
    const uint32_t f0 = u0 & (kKeyStep - 1u), f1 = u1 & (kKeyStep - 1u);
    const uint32_t m = clo - B;
    const uint32_t sc = static_cast<uint32_t>(wave_count(s0) + wave_count(s1));
    uint32_t fsel;
    if (m + 1u <= sc - m) {   // uniform: (m + 1)-th smallest = (m + 1)-th largest of 2^24 - f
      fsel = kKeyStep - rth_largest2(s0 ? kKeyStep - f0 : 0u, s1 ? kKeyStep - f1 : 0u, m + 1u, scratch);
    } else {                  // (s - m)-th largest of f + 1
      fsel = rth_largest2(s0 ? f0 + 1u : 0u, s1 ? f1 + 1u : 0u, sc - m, scratch) - 1u;
    }
    const uint32_t lo = static_cast<uint32_t>(tlo) * kKeyStep + fsel;   // the budget-th largest u
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
