// Quantize-and-transpose packer: fp32 keys -> channel-major MSB-first bit planes.
//
// Follows "Fathom Makes KV-Cache Scans Query-Adaptive for Long-Context
// Decoding" (para 2: the 4-bit K cache is stored as channel-major bit planes,
// a t-plane prefix being the channel's t-bit quantized value) and "Fathom:
// Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches"
// (abstract s3, s6).  Per (head, channel) asymmetric 16-bin floor quantizer;
// the per-channel variance the allocator weights channels by is computed here
// from exact integer moments of the codes.
//
// All float steps use explicit round-to-nearest intrinsics (no contraction),
// so planes, lo, step and var are bit-exact and independent of launch order.

#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kRangeThreads = 256;
constexpr int kRangeRows = 4096;        // key rows per range workgroup
constexpr int kQuantThreads = 512;      // 8 waves, one wave per 64 keys
constexpr int kTileKeys = 512;          // keys per quantize tile (16 plane words)
constexpr int kTileWords = kTileKeys / 32;
constexpr int kCodeStride = kD / 4 + 1; // u32 words per key row of codes in LDS (+1: bank spread)
constexpr int kTilesPerBlock = 4;

__global__ void pack_init_kernel(PackWorkspace ws, int count) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) {
    ws.kmin[i] = 0xffffffffu;
    ws.kmax[i] = 0u;
    ws.s1[i] = 0ull;
    ws.s2[i] = 0ull;
  }
}

// Per-channel min / max over the head's keys.  Thread = (4-channel group, row
// phase); each workgroup covers kRangeRows rows and folds into the workspace
// with ordered-integer atomics (exact, order independent).
__global__ __launch_bounds__(kRangeThreads) void pack_range_kernel(
    const float* __restrict__ keys, int64_t stride_head, int64_t stride_token, int64_t n,
    PackWorkspace ws) {
  const int h = blockIdx.y;
  const int cg = threadIdx.x & 31;          // channels 4cg .. 4cg+3
  const int r0 = threadIdx.x >> 5;          // 0..7
  const int64_t row_begin = int64_t(blockIdx.x) * kRangeRows;
  const int64_t row_end = row_begin + kRangeRows < n ? row_begin + kRangeRows : n;
  const float* base = keys + int64_t(h) * stride_head + 4 * cg;

  float mn[4], mx[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) { mn[t] = INFINITY; mx[t] = -INFINITY; }
  for (int64_t i = row_begin + r0; i < row_end; i += 8) {
    float4 v = *reinterpret_cast<const float4*>(base + i * stride_token);
    mn[0] = fminf(mn[0], v.x); mx[0] = fmaxf(mx[0], v.x);
    mn[1] = fminf(mn[1], v.y); mx[1] = fmaxf(mx[1], v.y);
    mn[2] = fminf(mn[2], v.z); mx[2] = fmaxf(mx[2], v.z);
    mn[3] = fminf(mn[3], v.w); mx[3] = fmaxf(mx[3], v.w);
  }
  __shared__ uint32_t smin[8][kD], smax[8][kD];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    smin[r0][4 * cg + t] = float_to_ordered(mn[t]);
    smax[r0][4 * cg + t] = float_to_ordered(mx[t]);
  }
  __syncthreads();
  if (threadIdx.x < kD) {
    const int c = threadIdx.x;
    uint32_t a = smin[0][c], b = smax[0][c];
    for (int r = 1; r < 8; ++r) {
      a = min(a, smin[r][c]);
      b = max(b, smax[r][c]);
    }
    atomicMin(&ws.kmin[h * kD + c], a);
    atomicMax(&ws.kmax[h * kD + c], b);
  }
}

// Quantize a tile of 512 keys, transpose the codes into bit-plane words with
// wavefront ballots (lane = key), and accumulate the integer moments.
__global__ __launch_bounds__(kQuantThreads) void pack_quant_kernel(
    const float* __restrict__ keys, int64_t stride_head, int64_t stride_token, int64_t n,
    int64_t ldw, int num_tiles, uint32_t* __restrict__ planes, PackWorkspace ws) {
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  __shared__ float s_lo[kD], s_inv[kD];
  __shared__ uint32_t s_code[kTileKeys * kCodeStride];          // 4 codes per word
  __shared__ uint32_t s_words[kD * kPlanes * kTileWords];        // [c][j][word]
  __shared__ uint32_t s_m1[16][kD], s_m2[16][kD];

  if (tid < kD) {
    const float lo = ordered_to_float(ws.kmin[h * kD + tid]);
    const float hi = ordered_to_float(ws.kmax[h * kD + tid]);
    const float r = __fsub_rn(hi, lo);
    s_lo[tid] = lo;
    s_inv[tid] = r > 0.0f ? __fdiv_rn(16.0f, r) : 0.0f;
  }
  __syncthreads();

  const int cg = tid & 31;      // channel group for the load phase
  const int rg = tid >> 5;      // row group 0..15
  float lo4[4], inv4[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) { lo4[t] = s_lo[4 * cg + t]; inv4[t] = s_inv[4 * cg + t]; }
  uint32_t m1[4] = {0, 0, 0, 0}, m2[4] = {0, 0, 0, 0};
  const float* head_keys = keys + int64_t(h) * stride_head + 4 * cg;

  for (int tile = blockIdx.x * kTilesPerBlock;
       tile < num_tiles && tile < (blockIdx.x + 1) * kTilesPerBlock; ++tile) {
    const int64_t key0 = int64_t(tile) * kTileKeys;
    // 1) load + quantize: 16 row groups x 32 rows each
    for (int r = rg; r < kTileKeys; r += 16) {
      const int64_t i = key0 + r;
      uint32_t packed = 0;
      if (i < n) {
        float4 v = *reinterpret_cast<const float4*>(head_keys + i * stride_token);
        float kv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float u = __fmul_rn(__fsub_rn(kv[t], lo4[t]), inv4[t]);
          const uint32_t code = u >= 15.0f ? 15u : static_cast<uint32_t>(u);  // u >= 0: trunc = floor
          m1[t] += code;
          m2[t] += code * code;
          packed |= code << (8 * t);
        }
      }
      s_code[r * kCodeStride + cg] = packed;
    }
    __syncthreads();
    // 2) transpose: wave w owns keys 64w .. 64w+63 of the tile, lane = key
    {
      const int key = wave * 64 + lane;
      for (int cw = 0; cw < kD / 4; ++cw) {
        const uint32_t four = s_code[key * kCodeStride + cw];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = cw * 4 + t;
          const uint32_t code = (four >> (8 * t)) & 0xffu;
#pragma unroll
          for (int j = 0; j < kPlanes; ++j) {
            const uint64_t m = __ballot((code >> (3 - j)) & 1u);
            // lanes 0 and 1 store the low / high 32-key words
            if (lane < 2) {
              const uint32_t word = lane == 0 ? static_cast<uint32_t>(m) : static_cast<uint32_t>(m >> 32);
              s_words[(c * kPlanes + j) * kTileWords + wave * 2 + lane] = word;
            }
          }
        }
      }
    }
    __syncthreads();
    // 3) store: one plane row segment (16 words = 64 B) per thread
    {
      const int row = tid;                          // c * 4 + j, 512 rows
      const int64_t w0 = int64_t(tile) * kTileWords;
      uint32_t* dst = planes + (int64_t(h) * kD * kPlanes + row) * ldw + w0;
      const uint32_t* src = s_words + row * kTileWords;
      if (w0 + kTileWords <= ldw) {
#pragma unroll
        for (int v = 0; v < kTileWords / 4; ++v) {
          reinterpret_cast<uint4*>(dst)[v] =
              make_uint4(src[4 * v], src[4 * v + 1], src[4 * v + 2], src[4 * v + 3]);
        }
      } else {
        for (int v = 0; w0 + v < ldw; ++v) dst[v] = src[v];
      }
    }
    __syncthreads();
  }
  // moments: fold the 16 row groups, then one 64-bit atomic per channel
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s_m1[rg][4 * cg + t] = m1[t];
    s_m2[rg][4 * cg + t] = m2[t];
  }
  __syncthreads();
  if (tid < kD) {
    unsigned long long a = 0, b = 0;
    for (int r = 0; r < 16; ++r) {
      a += s_m1[r][tid];
      b += s_m2[r][tid];
    }
    atomicAdd(&ws.s1[h * kD + tid], a);
    atomicAdd(&ws.s2[h * kD + tid], b);
  }
}

__global__ void pack_final_kernel(int count, int64_t n, PackWorkspace ws, float* __restrict__ lo,
                                  float* __restrict__ step, float* __restrict__ var) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float l = ordered_to_float(ws.kmin[i]);
  const float hi = ordered_to_float(ws.kmax[i]);
  const float r = __fsub_rn(hi, l);
  const float st = __fmul_rn(r, 0.0625f);   // exact power-of-two scaling
  lo[i] = l;
  step[i] = st;
  if (var) {
    const long long s1 = static_cast<long long>(ws.s1[i]);
    const long long s2 = static_cast<long long>(ws.s2[i]);
    const long long num = s2 * n - s1 * s1;   // exact: |num| < 2^53 for n <= 2^26
    const double den = __dmul_rn(static_cast<double>(n), static_cast<double>(n));
    const double st64 = static_cast<double>(st);
    const double v = __dmul_rn(__ddiv_rn(static_cast<double>(num), den), __dmul_rn(st64, st64));
    var[i] = __double2float_rn(v);
  }
}

}  // namespace

hipError_t launch_pack(const float* keys, int64_t stride_head, int64_t stride_token, int H, int64_t n,
                       int64_t ldw, uint32_t* planes, float* lo, float* step, float* var,
                       const PackWorkspace& ws, hipStream_t stream) {
  const int count = H * kD;
  hipLaunchKernelGGL(pack_init_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, ws, count);
  const int range_blocks = static_cast<int>((n + kRangeRows - 1) / kRangeRows);
  hipLaunchKernelGGL(pack_range_kernel, dim3(range_blocks, H), dim3(kRangeThreads), 0, stream, keys,
                     stride_head, stride_token, n, ws);
  // tiles cover every word of the padded rows, so padding words are written as zero
  const int num_tiles = static_cast<int>((ldw + kTileWords - 1) / kTileWords);
  const int quant_blocks = (num_tiles + kTilesPerBlock - 1) / kTilesPerBlock;
  hipLaunchKernelGGL(pack_quant_kernel, dim3(quant_blocks, H), dim3(kQuantThreads), 0, stream, keys,
                     stride_head, stride_token, n, ldw, num_tiles, planes, ws);
  hipLaunchKernelGGL(pack_final_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, count, n, ws,
                     lo, step, var);
  return hipGetLastError();
}

}  // namespace fathom
