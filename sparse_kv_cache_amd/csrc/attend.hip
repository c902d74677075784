// Attention over the selected keys: the decode step that follows the top-k
// scan ("Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
// Caches", title and abstract s1: the scan ranks the keys for a top-k step;
// "Fathom Makes KV-Cache Scans Query-Adaptive for Long-Context Decoding",
// second findings bullet: attention error).  For query q with selected key
// rows i in idx[q]:
//   p_i = exp(scale q.k_i - m),  o = sum_i p_i v_i / sum_i p_i,
// with K and V rows in bf16 (the serving stack's cache) read from HBM or, as
// device-visible pinned host memory, across PCIe.
//
// Split form: the k selected rows of a query are cut into chunks of
// kAttChunk; one workgroup per (chunk, query) gathers its K and V rows once
// (K for the scores, V staged in LDS for the weighted sum) and writes the
// chunk's partial (max m_s, sum l_s, o_s); a second kernel combines the
// chunks of each query: M = max_s m_s, o = sum_s e^(m_s - M) o_s /
// sum_s e^(m_s - M) l_s.  All arithmetic is fp32.
#include "fathom_internal.h"
#include "wave_ops.h"

#include <cmath>

namespace fathom {
namespace {

constexpr int kAttThreads = 256;                   // two threads per selected row
constexpr int kAttChunk = kAttThreads / 2;         // selected rows per workgroup
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kHalf = kD / 2;                      // channels per thread in the score

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

struct AttendArgs {
  const uint16_t* krows;   // bf16 rows: head h, key i at krows[h * stride_head + i * stride_token]
  const uint16_t* vrows;
  int64_t stride_head, stride_token;
  int64_t n;
  const float* q;          // [Q][kD]
  const int32_t* idx;      // [Q][k]
  int group, topk, nsplit;
  float scale;
  float* part;             // [Q][nsplit][kD + 2]: o_s, m_s, l_s
  float* out;              // [Q][kD]
};

__global__ __launch_bounds__(kAttThreads) void attend_partial_kernel(AttendArgs a) {
  __shared__ float qs[kD];
  __shared__ uint32_t vs[kAttChunk][kHalf + 1];    // bf16 pairs; +1 word against bank conflicts
  __shared__ float ps[kAttChunk];
  __shared__ float wred[kAttWaves][2];
  __shared__ float opart[kAttWaves][kD];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int qi = blockIdx.y, split = blockIdx.x;
  const int h = qi / a.group;
  const int i0 = split * kAttChunk;
  const int cnt = min(kAttChunk, a.topk - i0);
  const int j = t >> 1, half = t & 1;              // row slot and channel half of this thread
  // the selected row: index load, then both row loads in one round trip
  const bool valid = j < cnt;
  int64_t key = valid ? a.idx[int64_t(qi) * a.topk + i0 + j] : 0;
  const bool in_range = valid && key >= 0 && key < a.n;
  if (!in_range) key = 0;                          // (row 0 is read and ignored)
  const int64_t row = int64_t(h) * a.stride_head + key * a.stride_token + half * kHalf;
  const uint4* kr = reinterpret_cast<const uint4*>(a.krows + row);
  const uint4* vr = reinterpret_cast<const uint4*>(a.vrows + row);
  uint4 kw[8], vw[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) kw[r] = kr[r];
#pragma unroll
  for (int r = 0; r < 8; ++r) vw[r] = vr[r];
  if (t < kD) qs[t] = a.q[int64_t(qi) * kD + t] * a.scale;
  __syncthreads();
  float dot = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float* qp = &qs[half * kHalf + 8 * r];
    const uint32_t w[4] = {kw[r].x, kw[r].y, kw[r].z, kw[r].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dot = fmaf(bf16_lo(w[e]), qp[2 * e], dot);
      dot = fmaf(bf16_hi(w[e]), qp[2 * e + 1], dot);
    }
    uint32_t* vd = &vs[j][half * (kHalf / 2) + 4 * r];
    vd[0] = vw[r].x;
    vd[1] = vw[r].y;
    vd[2] = vw[r].z;
    vd[3] = vw[r].w;
  }
  dot += __uint_as_float(dpp_u32<kDppXor1>(0u, __float_as_uint(dot)));   // the other half's channels
  const float s = in_range ? dot : -INFINITY;
  // chunk maximum and the weights
  float m = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) wred[wave][0] = m;
  __syncthreads();
  m = wred[0][0];
#pragma unroll
  for (int w = 1; w < kAttWaves; ++w) m = fmaxf(m, wred[w][0]);
  // (a chunk always holds a valid row unless every index is out of range)
  const float p = (in_range && half == 0) ? expf(s - m) : 0.0f;
  if (half == 0) ps[j] = p;
  float l = p;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off, 64);
  if (lane == 0) wred[wave][1] = l;
  __syncthreads();
  // weighted sum of the staged V rows: wavefront w takes rows w, w + 4, ...;
  // lane c2 the channels 2 c2, 2 c2 + 1
  float o0 = 0.0f, o1 = 0.0f;
  for (int r = wave; r < cnt; r += kAttWaves) {
    const float pr = ps[r];
    const uint32_t vv = vs[r][lane];
    o0 = fmaf(pr, bf16_lo(vv), o0);
    o1 = fmaf(pr, bf16_hi(vv), o1);
  }
  opart[wave][2 * lane] = o0;
  opart[wave][2 * lane + 1] = o1;
  __syncthreads();
  float* dst = a.part + (int64_t(qi) * a.nsplit + split) * (kD + 2);
  if (t < kD) {
    float o = opart[0][t];
#pragma unroll
    for (int w = 1; w < kAttWaves; ++w) o += opart[w][t];
    dst[t] = o;
  }
  if (t == 0) {
    float lsum = wred[0][1];
#pragma unroll
    for (int w = 1; w < kAttWaves; ++w) lsum += wred[w][1];
    dst[kD] = m;
    dst[kD + 1] = lsum;
  }
}

__global__ __launch_bounds__(kD) void attend_combine_kernel(AttendArgs a) {
  const int qi = blockIdx.x, c = threadIdx.x;
  const float* src = a.part + int64_t(qi) * a.nsplit * (kD + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, src[s * (kD + 2) + kD]);
  float o = 0.0f, L = 0.0f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = src[s * (kD + 2) + kD];
    const float w = ms == -INFINITY ? 0.0f : expf(ms - M);
    o = fmaf(w, src[s * (kD + 2) + c], o);
    L = fmaf(w, src[s * (kD + 2) + kD + 1], L);
  }
  a.out[int64_t(qi) * kD + c] = L > 0.0f ? o / L : 0.0f;
}

}  // namespace

int attend_splits(int k) { return (k + kAttChunk - 1) / kAttChunk; }

hipError_t launch_attend(const uint16_t* k_rows, const uint16_t* v_rows, int64_t stride_head,
                         int64_t stride_token, int64_t n, const float* q, const int32_t* idx, int num_q,
                         int group, int k, float scale, float* part, float* out, hipStream_t stream) {
  AttendArgs a{};
  a.krows = k_rows;
  a.vrows = v_rows;
  a.stride_head = stride_head;
  a.stride_token = stride_token;
  a.n = n;
  a.q = q;
  a.idx = idx;
  a.group = group;
  a.topk = k;
  a.nsplit = attend_splits(k);
  a.scale = scale;
  a.part = part;
  a.out = out;
  hipLaunchKernelGGL(attend_partial_kernel, dim3(a.nsplit, num_q), dim3(kAttThreads), 0, stream, a);
  hipLaunchKernelGGL(attend_combine_kernel, dim3(num_q), dim3(kD), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fathom
