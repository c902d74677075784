// Plane-prefix key scan with fused top-k (gfx950).
//
// "Fathom Makes KV-Cache Scans Query-Adaptive for Long-Context Decoding",
// paras 1-2, and "Fathom: Per-Query Read Depth for Sparse Decoding over
// Offloaded KV Caches", abstract s1-s3: every decode step ranks all n keys
// for a top-k, and each query reads only the first b_qc bit planes of each
// channel c.  With the planes MSB-first, the b-plane prefix of a channel is
// its b-bit quantized value, so the partially dequantized dot product is
//
//   s_q(i) = C_q + sum_c sum_{j < b_qc} q_c step_c 2^(3-j) bit_{c,j}(i),
//   C_q    = sum_c q_c (lo_c + step_c 2^(3-b_qc))      (bin-centre offsets).
//
// Launch sequence per call (all on the caller's stream):
//   1. scan_sample_kernel    exact scores of up to 8 sampled 1024-key blocks
//                            per KV head (lane = key);
//   2. scan_threshold_kernel per query, a radix select on the sample picks a
//                            score theta expected to leave ~2k keys above it;
//   3. scan_main_kernel      every key of every head: workgroup = (KV head,
//                            query chunk, 256 plane words), lane = one 32-key
//                            word; reads the union of the chunk's plane
//                            prefixes once, accumulates all its queries, and
//                            appends keys scoring >= theta to a per-query
//                            candidate list;
//   4. scan_merge_kernel     per query, sorts the candidates in LDS and emits
//                            the top-k.  If the candidate list holds fewer
//                            than k keys or overflowed, the workgroup instead
//                            recomputes the query's scores and selects the
//                            exact top-k by radix select (ties by index).
// Every kernel accumulates a query's planes in the same order (channel asc,
// plane asc), so the three score paths produce identical fp32 values.

#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kScanThreads = 256;
constexpr int kMaxUnion = kD * kPlanes;
constexpr int kMergeThreads = 1024;
constexpr int kThresholdThreads = 256;
constexpr int kPrefetch = 4;

struct ScanArgs {
  const uint32_t* planes;
  const float* lo;
  const float* step;
  const float* q;
  const uint8_t* alloc;
  int64_t n;
  int64_t ldw;
  int nwords;         // ceil(n / 32)
  int group;          // query heads per KV head
  int cph;            // query chunks of this launch per KV head
  int qoff;           // first query of chunk 0 within its head
  float* theta;
  uint32_t* count;
  float* sample;
  uint2* cand;
  float* all_scores;
  int sample_stride;  // distance between sampled blocks, in 1024-key blocks
};

template <int GQ>
struct UnionLds {
  float w[kMaxUnion][GQ];       // q_c step_c 2^(3-j); 0 where the query skips the plane
  double cpart[GQ][kD];
  uint16_t row[kMaxUnion];      // plane row c*4 + j, in (c asc, j asc) order
  uint8_t mask[kMaxUnion];      // bit g: query g of the chunk reads the plane
  int off[kD];
  float C[GQ];
  float theta[GQ];
  int U;
};

__device__ inline int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  return __popcll(mask & below);
}

__device__ inline double pow2_3_minus(int b) {
  // 2^(3 - b) for b in 0..4
  return b == 0 ? 8.0 : b == 1 ? 4.0 : b == 2 ? 2.0 : b == 3 ? 1.0 : 0.5;
}

// Builds the union plane list of a query chunk (queries q0 .. q0+GQ-1 on
// KV head h), the per-plane weights and the score offsets C_q.
// Needs blockDim.x >= kD; ends with __syncthreads().
template <int GQ>
__device__ void build_union(const ScanArgs& a, int h, int q0, UnionLds<GQ>& s) {
  const int t = threadIdx.x;
  int u = 0, bq[GQ];
  float qv[GQ], st = 0.0f;
  if (t < kD) {
    const float lo = a.lo[h * kD + t];
    st = a.step[h * kD + t];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      bq[g] = min(static_cast<int>(a.alloc[int64_t(q0 + g) * kD + t]), kPlanes);
      qv[g] = a.q[int64_t(q0 + g) * kD + t];
      u = max(u, bq[g]);
      s.cpart[g][t] = static_cast<double>(qv[g]) *
                      (static_cast<double>(lo) + static_cast<double>(st) * pow2_3_minus(bq[g]));
    }
  }
  // exclusive prefix sum of u over channels (wave 0: two channels per lane)
  __shared__ int s_u[kD];
  if (t < kD) s_u[t] = u;
  __syncthreads();
  if (t < 64) {
    const int v0 = s_u[2 * t], v1 = s_u[2 * t + 1];
    int incl = v0 + v1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (t >= d) incl += o;
    }
    const int excl = incl - v0 - v1;
    s.off[2 * t] = excl;
    s.off[2 * t + 1] = excl + v0;
    if (t == 63) s.U = incl;
  }
  __syncthreads();
  if (t < kD) {
    const int o = s.off[t];
    for (int j = 0; j < u; ++j) {
      uint32_t m = 0;
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const bool on = j < bq[g];
        m |= on ? (1u << g) : 0u;
        s.w[o + j][g] = on ? __fmul_rn(qv[g], st) * static_cast<float>(8 >> j) : 0.0f;
      }
      s.row[o + j] = static_cast<uint16_t>(t * kPlanes + j);
      s.mask[o + j] = static_cast<uint8_t>(m);
    }
  }
  __syncthreads();
  if (t < GQ) {
    double c = 0.0;
    for (int i = 0; i < kD; ++i) c += s.cpart[t][i];
    s.C[t] = static_cast<float>(c);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ sample

template <int GQ>
__global__ __launch_bounds__(kScanThreads) void scan_sample_kernel(ScanArgs a) {
  __shared__ UnionLds<GQ> s;
  const int h = blockIdx.y / a.cph;
  const int q0 = h * a.group + a.qoff + (blockIdx.y % a.cph) * kQueryChunk;
  build_union<GQ>(a, h, q0, s);

  const int sbi = blockIdx.x >> 2;
  const int local = (blockIdx.x & 3) * kScanThreads + threadIdx.x;   // 0..1023
  const int64_t key = int64_t(sbi) * a.sample_stride * kSampleBlockKeys + local;
  const bool valid = key < a.n;
  const uint32_t* base = a.planes + int64_t(h) * kD * kPlanes * a.ldw + (valid ? (key >> 5) : 0);
  const int bit = static_cast<int>(key & 31);
  float acc[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g) acc[g] = 0.0f;
  const int U = s.U;
  for (int p = 0; p < U; ++p) {
    const uint32_t x = valid ? base[int64_t(s.row[p]) * a.ldw] : 0u;
    const float f = static_cast<float>((x >> bit) & 1u);
    const uint32_t m = s.mask[p];
#pragma unroll
    for (int g = 0; g < GQ; ++g)
      if (m & (1u << g)) acc[g] = fmaf(f, s.w[p][g], acc[g]);
  }
#pragma unroll
  for (int g = 0; g < GQ; ++g)
    a.sample[int64_t(q0 + g) * kSampleMaxKeys + sbi * kSampleBlockKeys + local] =
        valid ? acc[g] + s.C[g] : -INFINITY;
}

// --------------------------------------------------------------- threshold

// Radix select of the r-th largest of `count` ordered keys held in LDS.
// All threads of the block call it; returns the ordered key.
__device__ uint32_t block_select_kth(const uint32_t* vals, int count, uint32_t r, uint32_t* hist,
                                     uint32_t* s_scalar) {
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < count; i += blockDim.x) {
      const uint32_t v = vals[i];
      if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t cum = 0;
      int sel = 0;
      for (int bin = 255; bin >= 0; --bin) {
        if (cum + hist[bin] >= r) { sel = bin; break; }
        cum += hist[bin];
      }
      s_scalar[0] = static_cast<uint32_t>(sel);
      s_scalar[1] = r - cum;
    }
    __syncthreads();
    prefix |= s_scalar[0] << shift;
    pmask |= 255u << shift;
    r = s_scalar[1];
    __syncthreads();
  }
  return prefix;
}

__global__ __launch_bounds__(kThresholdThreads) void scan_threshold_kernel(
    const float* __restrict__ sample, int stot, uint32_t rsel, float* __restrict__ theta,
    uint32_t* __restrict__ count) {
  __shared__ uint32_t vals[kSampleMaxKeys];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_scalar[2];
  const int q = blockIdx.x;
  for (int i = threadIdx.x; i < stot; i += blockDim.x)
    vals[i] = float_to_ordered(sample[int64_t(q) * kSampleMaxKeys + i]);
  __syncthreads();
  const uint32_t key = block_select_kth(vals, stot, rsel, hist, s_scalar);
  if (threadIdx.x == 0) {
    theta[q] = ordered_to_float(key);
    count[q] = 0u;
  }
}

// -------------------------------------------------------------------- main

template <int GQ, uint32_t M>
__device__ __forceinline__ void accumulate_masked(uint32_t x, const float (&wv)[GQ],
                                                  float (&acc)[32][GQ]) {
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const float f = static_cast<float>((x >> b) & 1u);
#pragma unroll
    for (int g = 0; g < GQ; ++g)
      if (M & (1u << g)) acc[b][g] = fmaf(f, wv[g], acc[b][g]);
  }
}

template <int GQ, uint32_t M = 1>
__device__ __forceinline__ void accumulate(uint32_t m, uint32_t x, const float (&wv)[GQ],
                                           float (&acc)[32][GQ]) {
  if constexpr (M < (1u << GQ)) {
    if (m == M) {
      accumulate_masked<GQ, M>(x, wv, acc);
      return;
    }
    accumulate<GQ, M + 1>(m, x, wv, acc);
  }
}

template <int GQ>
__global__ __launch_bounds__(kScanThreads) void scan_main_kernel(ScanArgs a) {
  __shared__ UnionLds<GQ> s;
  const int h = blockIdx.y / a.cph;
  const int q0 = h * a.group + a.qoff + (blockIdx.y % a.cph) * kQueryChunk;
  if (threadIdx.x < GQ) s.theta[threadIdx.x] = a.theta[q0 + threadIdx.x];
  build_union<GQ>(a, h, q0, s);

  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kScanThreads + threadIdx.x;
  const bool active = w < a.nwords;
  const uint32_t* base = a.planes + int64_t(h) * kD * kPlanes * a.ldw + (active ? w : 0);
  const int U = s.U;

  float acc[32][GQ];
#pragma unroll
  for (int b = 0; b < 32; ++b)
#pragma unroll
    for (int g = 0; g < GQ; ++g) acc[b][g] = 0.0f;

  uint32_t ring[kPrefetch];
#pragma unroll
  for (int r = 0; r < kPrefetch; ++r)
    ring[r] = (r < U && active) ? base[int64_t(s.row[r]) * a.ldw] : 0u;

  for (int p0 = 0; p0 < U; p0 += kPrefetch) {
#pragma unroll
    for (int r = 0; r < kPrefetch; ++r) {
      const int p = p0 + r;
      if (p < U) {
        const uint32_t x = ring[r];
        const int pn = p + kPrefetch;
        ring[r] = (pn < U && active) ? base[int64_t(s.row[pn]) * a.ldw] : 0u;
        const uint32_t m = __builtin_amdgcn_readfirstlane(s.mask[p]);
        float wv[GQ];
#pragma unroll
        for (int g = 0; g < GQ; ++g) wv[g] = s.w[p][g];
        accumulate<GQ>(m, x, wv, acc);
      }
    }
  }

  // epilogue: finish scores, optional dump, threshold filter + append
  const int64_t key0 = int64_t(w) * 32;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const int64_t i = key0 + b;
    const bool valid = active && i < a.n;
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const float sc = acc[b][g] + s.C[g];
      if (a.all_scores && valid) a.all_scores[int64_t(q0 + g) * a.n + i] = sc;
      const bool pass = valid && sc >= s.theta[g];
      const uint64_t bal = __ballot(pass);
      if (bal) {
        const int leader = __builtin_ctzll(bal);
        uint32_t slot0 = 0;
        if (lane == leader) slot0 = atomicAdd(&a.count[q0 + g], static_cast<uint32_t>(__popcll(bal)));
        slot0 = __builtin_amdgcn_readlane(slot0, leader);
        if (pass) {
          const uint32_t slot = slot0 + lanes_below(bal);
          if (slot < static_cast<uint32_t>(kCandCap))
            a.cand[int64_t(q0 + g) * kCandCap + slot] =
                make_uint2(__float_as_uint(sc), static_cast<uint32_t>(i));
        }
      }
    }
  }
}

// ------------------------------------------------------------------- merge

__device__ inline unsigned long long sort_key(float score, uint32_t idx) {
  return (static_cast<unsigned long long>(float_to_ordered(score)) << 32) | static_cast<uint32_t>(~idx);
}

// Descending bitonic sort of N (power of two) 64-bit keys in LDS.
__device__ void bitonic_sort_desc(unsigned long long* keys, unsigned N) {
  for (unsigned size = 2; size <= N; size <<= 1) {
    for (unsigned stride = size >> 1; stride > 0; stride >>= 1) {
      for (unsigned t = threadIdx.x; t < N / 2; t += blockDim.x) {
        const unsigned lo_i = 2 * t - (t & (stride - 1));
        const unsigned hi_i = lo_i + stride;
        const bool desc = (lo_i & size) == 0;
        const unsigned long long x = keys[lo_i], y = keys[hi_i];
        if ((x < y) == desc) {
          keys[lo_i] = y;
          keys[hi_i] = x;
        }
      }
      __syncthreads();
    }
  }
}

struct QueryLds {
  float w[kD][kPlanes];
  uint8_t b[kD];
  double cpart[kD];
  float C;
};

// Score of key i for one query: same plane order and fp32 operations as the
// chunked kernels, so the value is bit-identical to theirs.
__device__ inline float query_score(const uint32_t* head_planes, int64_t ldw, const QueryLds& s,
                                    int64_t i) {
  const uint32_t* base = head_planes + (i >> 5);
  const int bit = static_cast<int>(i & 31);
  float acc = 0.0f;
  for (int c = 0; c < kD; ++c) {
    const int bc = s.b[c];
    for (int j = 0; j < bc; ++j) {
      const uint32_t x = base[int64_t(c * kPlanes + j) * ldw];
      acc = fmaf(static_cast<float>((x >> bit) & 1u), s.w[c][j], acc);
    }
  }
  return acc + s.C;
}

__global__ __launch_bounds__(kMergeThreads) void scan_merge_kernel(ScanArgs a, int k,
                                                                   int32_t* __restrict__ out_idx,
                                                                   float* __restrict__ out_score) {
  __shared__ unsigned long long keys[kCandCap];
  __shared__ QueryLds qs;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_scalar[4];
  __shared__ uint32_t s_wave[kMergeThreads / 64];
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t cnt = a.count[q];
  unsigned N;

  if (cnt >= static_cast<uint32_t>(k) && cnt <= static_cast<uint32_t>(kCandCap)) {
    N = 2;
    while (N < cnt) N <<= 1;
    for (unsigned i = tid; i < N; i += blockDim.x) {
      if (i < cnt) {
        const uint2 e = a.cand[int64_t(q) * kCandCap + i];
        keys[i] = sort_key(__uint_as_float(e.x), e.y);
      } else {
        keys[i] = 0ull;
      }
    }
    __syncthreads();
  } else {
    // exact fallback: radix select over recomputed scores
    const int h = q / a.group;
    const uint32_t* head_planes = a.planes + int64_t(h) * kD * kPlanes * a.ldw;
    if (tid < kD) {
      const float lo = a.lo[h * kD + tid], st = a.step[h * kD + tid];
      const float qv = a.q[int64_t(q) * kD + tid];
      const int bc = min(static_cast<int>(a.alloc[int64_t(q) * kD + tid]), kPlanes);
      qs.b[tid] = static_cast<uint8_t>(bc);
      for (int j = 0; j < kPlanes; ++j) qs.w[tid][j] = __fmul_rn(qv, st) * static_cast<float>(8 >> j);
      qs.cpart[tid] = static_cast<double>(qv) *
                      (static_cast<double>(lo) + static_cast<double>(st) * pow2_3_minus(bc));
    }
    __syncthreads();
    if (tid == 0) {
      double c = 0.0;
      for (int i = 0; i < kD; ++i) c += qs.cpart[i];
      qs.C = static_cast<float>(c);
    }
    __syncthreads();
    uint32_t prefix = 0, pmask = 0, r = static_cast<uint32_t>(k);
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
      __syncthreads();
      for (int64_t i = tid; i < a.n; i += blockDim.x) {
        const uint32_t v = float_to_ordered(query_score(head_planes, a.ldw, qs, i));
        if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t cum = 0;
        int sel = 0;
        for (int bin = 255; bin >= 0; --bin) {
          if (cum + hist[bin] >= r) { sel = bin; break; }
          cum += hist[bin];
        }
        s_scalar[0] = static_cast<uint32_t>(sel);
        s_scalar[1] = r - cum;
      }
      __syncthreads();
      prefix |= s_scalar[0] << shift;
      pmask |= 255u << shift;
      r = s_scalar[1];
      __syncthreads();
    }
    const uint32_t kth = prefix;                 // ordered score of the k-th key
    const uint32_t n_gt = static_cast<uint32_t>(k) - r;   // keys strictly above it
    if (tid == 0) s_scalar[2] = 0;               // gt slots used
    __syncthreads();
    uint32_t eq_taken = 0;
    const int lane = tid & 63, wave = tid >> 6;
    for (int64_t base = 0; base < a.n; base += blockDim.x) {
      const int64_t i = base + tid;
      const bool valid = i < a.n;
      const uint32_t v = valid ? float_to_ordered(query_score(head_planes, a.ldw, qs, i)) : 0u;
      const bool gt = valid && v > kth;
      const bool eq = valid && v == kth;
      if (gt) {
        const uint32_t slot = atomicAdd(&s_scalar[2], 1u);
        keys[slot] = (static_cast<unsigned long long>(v) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(i));
      }
      const uint64_t bal = __ballot(eq);
      if (lane == 0) s_wave[wave] = static_cast<uint32_t>(__popcll(bal));
      __syncthreads();
      uint32_t before = 0, total = 0;
      for (int wv = 0; wv < static_cast<int>(blockDim.x / 64); ++wv) {
        const uint32_t c = s_wave[wv];
        before += wv < wave ? c : 0u;
        total += c;
      }
      if (eq) {
        const uint32_t rank = eq_taken + before + static_cast<uint32_t>(lanes_below(bal));
        if (rank < r)
          keys[n_gt + rank] = (static_cast<unsigned long long>(v) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(i));
      }
      eq_taken += total;
      __syncthreads();
    }
    N = 2;
    while (N < static_cast<unsigned>(k)) N <<= 1;
    for (unsigned i = k + tid; i < N; i += blockDim.x) keys[i] = 0ull;
    __syncthreads();
  }
  bitonic_sort_desc(keys, N);
  for (int i = tid; i < k; i += blockDim.x) {
    const unsigned long long e = keys[i];
    out_idx[int64_t(q) * k + i] = static_cast<int32_t>(~static_cast<uint32_t>(e));
    out_score[int64_t(q) * k + i] = ordered_to_float(static_cast<uint32_t>(e >> 32));
  }
}

template <int GQ>
hipError_t launch_chunk_class(const ScanArgs& a, int H, int nsb, const ScanTiming* timing,
                              bool sample_phase, hipStream_t stream) {
  if (sample_phase) {
    hipLaunchKernelGGL(scan_sample_kernel<GQ>, dim3(nsb * 4, H * a.cph), dim3(kScanThreads), 0, stream, a);
  } else {
    const int tiles = (a.nwords + kScanThreads - 1) / kScanThreads;
    hipLaunchKernelGGL(scan_main_kernel<GQ>, dim3(tiles, H * a.cph), dim3(kScanThreads), 0, stream, a);
  }
  (void)timing;
  return hipGetLastError();
}

hipError_t launch_class(int gq, const ScanArgs& a, int H, int nsb, const ScanTiming* timing,
                        bool sample_phase, hipStream_t stream) {
  switch (gq) {
    case 1: return launch_chunk_class<1>(a, H, nsb, timing, sample_phase, stream);
    case 2: return launch_chunk_class<2>(a, H, nsb, timing, sample_phase, stream);
    case 3: return launch_chunk_class<3>(a, H, nsb, timing, sample_phase, stream);
    default: return launch_chunk_class<4>(a, H, nsb, timing, sample_phase, stream);
  }
}

}  // namespace

hipError_t launch_scan_topk(const uint32_t* planes, const float* lo, const float* step, int H,
                            int64_t n, int64_t ldw, const float* q, const uint8_t* alloc, int num_q,
                            int group, int k, int32_t* out_idx, float* out_score,
                            float* all_scores, const ScanWorkspace& ws, const ScanTiming* timing,
                            hipStream_t stream) {
  ScanArgs a{};
  a.planes = planes;
  a.lo = lo;
  a.step = step;
  a.q = q;
  a.alloc = alloc;
  a.n = n;
  a.ldw = ldw;
  a.nwords = static_cast<int>((n + 31) / 32);
  a.group = group;
  a.theta = ws.theta;
  a.count = ws.count;
  a.sample = ws.sample;
  a.cand = ws.cand;
  a.all_scores = all_scores;

  // sampled blocks: up to 8 blocks of 1024 keys spread evenly over the head
  const int64_t nblocks = (n + kSampleBlockKeys - 1) / kSampleBlockKeys;
  const int nsb = static_cast<int>(nblocks < kSampleMaxBlocks ? nblocks : kSampleMaxBlocks);
  const int64_t stride = nblocks / nsb;
  a.sample_stride = static_cast<int>(stride);
  int64_t svalid = 0;
  for (int i = 0; i < nsb; ++i) {
    const int64_t start = int64_t(i) * stride * kSampleBlockKeys;
    const int64_t left = n - start;
    svalid += left < kSampleBlockKeys ? left : kSampleBlockKeys;
  }
  // rank in the sample whose score should leave about 2k keys above it in the
  // whole head; at least 16 sampled keys above it so the estimate is stable
  int64_t rsel = (2 * int64_t(k) * svalid + n - 1) / n;
  const int64_t rmin = svalid < 16 ? svalid : 16;
  if (rsel < rmin) rsel = rmin;
  if (rsel > svalid) rsel = svalid;

  const int full = group / kQueryChunk;
  const int rest = group % kQueryChunk;

  for (int phase = 0; phase < 2; ++phase) {
    const bool sample_phase = phase == 0;
    if (!sample_phase && timing && timing->start) (void)hipEventRecord(timing->start, stream);
    if (full > 0) {
      ScanArgs b = a;
      b.cph = full;
      b.qoff = 0;
      hipError_t e = launch_class(kQueryChunk, b, H, nsb, timing, sample_phase, stream);
      if (e != hipSuccess) return e;
    }
    if (rest > 0) {
      ScanArgs b = a;
      b.cph = 1;
      b.qoff = full * kQueryChunk;
      hipError_t e = launch_class(rest, b, H, nsb, timing, sample_phase, stream);
      if (e != hipSuccess) return e;
    }
    if (!sample_phase && timing && timing->stop) (void)hipEventRecord(timing->stop, stream);
    if (sample_phase) {
      hipLaunchKernelGGL(scan_threshold_kernel, dim3(num_q), dim3(kThresholdThreads), 0, stream,
                         ws.sample, nsb * kSampleBlockKeys, static_cast<uint32_t>(rsel), ws.theta,
                         ws.count);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(scan_merge_kernel, dim3(num_q), dim3(kMergeThreads), 0, stream, a, k, out_idx,
                     out_score);
  return hipGetLastError();
}

}  // namespace fathom
