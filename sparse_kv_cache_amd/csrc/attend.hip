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
// (K for the scores, V staged in LDS for the weighted sum), 16 lanes per row
// so that each load instruction reads whole 128-byte lines, and writes the
// chunk's partial (max m_s, sum l_s, o_s); a second kernel combines the
// chunks of each query: M = max_s m_s, o = sum_s e^(m_s - M) o_s /
// sum_s e^(m_s - M) l_s.  All arithmetic is fp32.
#include "fathom_internal.h"
#include "wave_ops.h"

#include <cmath>

namespace fathom {
namespace {

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kAttChunk = 128;                     // selected rows per workgroup
constexpr int kRowLanes = 16;                      // lanes per row: 16 bytes (8 channels) each
constexpr int kRowsPerPass = 64 / kRowLanes;       // rows a wavefront loads per instruction
constexpr int kPasses = kAttChunk / (kAttWaves * kRowsPerPass);

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sum over the 16 lanes of a DPP row, returned to all of them.
__device__ __forceinline__ float row_sum16(float v) {
  v += __uint_as_float(dpp_u32<kDppXor1>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppXor2>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppRowHalfMirror>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppRowMirror>(0u, __float_as_uint(v)));
  return v;
}

struct AttendArgs {
  const uint16_t* krows;   // bf16 rows: head h, key i at krows[h * stride_head + i * stride_token]
  const uint16_t* vrows;
  int64_t stride_head, stride_token;
  int64_t n;
  const int32_t* lengths;  // null, or keys per head
  const float* q;          // [Q][kD]
  const int32_t* idx;      // [Q][k]
  int group, topk, nsplit;
  float scale;
  float* part;             // [Q][nsplit][kD + 2]: o_s, m_s, l_s
  float* out;              // [Q][kD]
};

// Workgroup = (chunk of kAttChunk selected rows, query).  Wavefront w loads
// rows w * kRowsPerPass * kPasses + ...: per instruction, 4 rows of 16 lanes
// each, a lane taking 16 bytes (8 channels) of a row, so every instruction
// covers whole 128-byte lines.
__global__ __launch_bounds__(kAttThreads) void attend_partial_kernel(AttendArgs a) {
  __shared__ uint4 vs[kAttChunk][kRowLanes + 1];   // staged V rows; +16 bytes against bank conflicts
  __shared__ float ps[kAttChunk];
  __shared__ float wred[kAttWaves][2];
  __shared__ float opart[kAttWaves][kD];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int qi = blockIdx.y, split = blockIdx.x;
  const int h = qi / a.group;
  const int64_t nh = head_length(a.lengths, h, a.n);
  const int i0 = split * kAttChunk;
  const int cnt = min(kAttChunk, a.topk - i0);
  const int piece = lane & (kRowLanes - 1), sub = lane / kRowLanes;
  // this lane's 8 query channels, scaled
  float qv[8];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.q + int64_t(qi) * kD + 8 * piece);
    const float4 q0 = qp[0], q1 = qp[1];
    qv[0] = q0.x * a.scale; qv[1] = q0.y * a.scale; qv[2] = q0.z * a.scale; qv[3] = q0.w * a.scale;
    qv[4] = q1.x * a.scale; qv[5] = q1.y * a.scale; qv[6] = q1.z * a.scale; qv[7] = q1.w * a.scale;
  }
  // the rows of this lane in each pass: indexes first, then all row loads
  int slot[kPasses];
  bool ok[kPasses];
  uint4 kw[kPasses], vw[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    slot[p] = (wave * kPasses + p) * kRowsPerPass + sub;
    const int jj = min(slot[p], cnt - 1);
    const int64_t key = a.idx[int64_t(qi) * a.topk + i0 + jj];
    ok[p] = slot[p] < cnt && key >= 0 && key < nh;
    const int64_t row = int64_t(h) * a.stride_head + (ok[p] ? key : 0) * a.stride_token + 8 * piece;
    kw[p] = *reinterpret_cast<const uint4*>(a.krows + row);
    vw[p] = *reinterpret_cast<const uint4*>(a.vrows + row);
  }
  float sv[kPasses];
  float m = -INFINITY;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const uint32_t w[4] = {kw[p].x, kw[p].y, kw[p].z, kw[p].w};
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dot = fmaf(bf16_lo(w[e]), qv[2 * e], dot);
      dot = fmaf(bf16_hi(w[e]), qv[2 * e + 1], dot);
    }
    dot = row_sum16(dot);
    sv[p] = ok[p] ? dot : -INFINITY;
    m = fmaxf(m, sv[p]);
    vs[slot[p]][piece] = vw[p];
  }
  // chunk maximum and the weights
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) wred[wave][0] = m;
  __syncthreads();
  m = wred[0][0];
#pragma unroll
  for (int w = 1; w < kAttWaves; ++w) m = fmaxf(m, wred[w][0]);
  float l = 0.0f;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const float pr = ok[p] ? expf(sv[p] - m) : 0.0f;
    if (piece == 0) {
      ps[slot[p]] = pr;
      l += pr;
    }
  }
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) l += __shfl_xor(l, off, 64);
  if (lane == 0) wred[wave][1] = l;
  __syncthreads();
  // weighted sum of the staged V rows: wavefront w takes rows w, w + 4, ...;
  // lane c2 the channels 2 c2, 2 c2 + 1
  float o0 = 0.0f, o1 = 0.0f;
  for (int r = wave; r < cnt; r += kAttWaves) {
    const float pr = ps[r];
    const uint32_t vv = reinterpret_cast<const uint32_t*>(&vs[r][0])[lane];
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

// (every partial of the query loads at once: the loop over chunks is
// unrolled to its bound, kMaxK / kAttChunk)
constexpr int kMaxSplits = kMaxK / kAttChunk;

__global__ __launch_bounds__(kD) void attend_combine_kernel(AttendArgs a) {
  const int qi = blockIdx.x, c = threadIdx.x;
  const float* src = a.part + int64_t(qi) * a.nsplit * (kD + 2);
  float ov[kMaxSplits], mv[kMaxSplits], lv[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const int ss = min(s, a.nsplit - 1);   // (re-reads the last chunk; weighted 0 below)
    ov[s] = src[ss * (kD + 2) + c];
    mv[s] = src[ss * (kD + 2) + kD];
    lv[s] = src[ss * (kD + 2) + kD + 1];
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) M = s < a.nsplit ? fmaxf(M, mv[s]) : M;
  float o = 0.0f, L = 0.0f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const float w = (s < a.nsplit && mv[s] != -INFINITY) ? expf(mv[s] - M) : 0.0f;
    o = fmaf(w, ov[s], o);
    L = fmaf(w, lv[s], L);
  }
  a.out[int64_t(qi) * kD + c] = L > 0.0f ? o / L : 0.0f;
}

}  // namespace

int attend_splits(int k) { return (k + kAttChunk - 1) / kAttChunk; }

hipError_t launch_attend(const uint16_t* k_rows, const uint16_t* v_rows, int64_t stride_head,
                         int64_t stride_token, int64_t n, const int32_t* lengths, const float* q, const int32_t* idx, int num_q,
                         int group, int k, float scale, float* part, float* out, hipStream_t stream) {
  AttendArgs a{};
  a.krows = k_rows;
  a.vrows = v_rows;
  a.stride_head = stride_head;
  a.stride_token = stride_token;
  a.n = n;
  a.lengths = lengths;
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
