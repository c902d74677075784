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

#include <algorithm>

#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kRangeThreads = 256;
constexpr int kRangeRows = 4096;        // key rows per range workgroup

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
    const int32_t* __restrict__ lengths, PackWorkspace ws) {
  const int h = blockIdx.y;
  const int cg = threadIdx.x & 31;          // channels 4cg .. 4cg+3
  const int r0 = threadIdx.x >> 5;          // 0..7
  const int64_t nh = head_length(lengths, h, n);
  const int64_t row_begin = int64_t(blockIdx.x) * kRangeRows;
  const int64_t row_end = row_begin + kRangeRows < nh ? row_begin + kRangeRows : nh;
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

// Quantize-and-transpose.  A workgroup (4 wavefronts) packs tiles of 32
// plane words (1024 keys) of one head.  Each half-wavefront owns one plane
// word at a time: its 32 lanes cover the 128 channels (lane = 4-channel
// group) and walk the word's 32 consecutive keys, so lane `cg` ends up with
// the 4-bit codes of channels 4cg..4cg+3 for keys 32w..32w+31.  Packing the
// four codes of key b as a 16-bit value x[b] and transposing the 32 x 16 bit
// matrix in registers yields the 16 plane words of those channels directly
// (bit b = key 32w+b).  The words are staged in LDS so each plane row is
// stored as one 128-byte segment.
constexpr int kQuantThreads = 256;
constexpr int kQuantWords = 32;                       // plane words per tile
constexpr int kHalfWaves = kQuantThreads / 32;        // 8 word slots in flight
constexpr int kKeyBatch = 16;                         // loads in flight per lane

// In-register transpose of the 16-bit values x[0..31] (bit p of x[b]) into
// 16 words (bit b of word p).  The first swap round of the 32 x 32 network
// only packs key b+16 into the upper half of x[b], because the upper halves
// are zero; four rounds on 16 words remain.
__device__ __forceinline__ void transpose32x16(uint32_t (&x)[32], uint32_t (&y)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) y[k] = x[k] | (x[k + 16] << 16);
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) {
    const uint32_t m = sh == 8 ? 0x00ff00ffu : sh == 4 ? 0x0f0f0f0fu : sh == 2 ? 0x33333333u : 0x55555555u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k & sh) continue;
      const uint32_t t = ((y[k] >> sh) ^ y[k + sh]) & m;
      y[k + sh] ^= t;
      y[k] ^= t << sh;
    }
  }
}

__global__ __launch_bounds__(kQuantThreads) void pack_quant_kernel(
    const float* __restrict__ keys, int64_t stride_head, int64_t stride_token, int64_t n,
    const int32_t* __restrict__ lengths, int64_t ldw, int num_tiles, int tiles_per_wg,
    uint32_t* __restrict__ planes, PackWorkspace ws) {
  const int h = blockIdx.y;
  const int64_t nh = head_length(lengths, h, n);
  const int64_t last_key = nh > 0 ? nh - 1 : 0;   // (key 0 exists: n >= 1)
  const int tid = threadIdx.x;
  const int cg = tid & 31;          // channels 4cg .. 4cg+3
  const int hw = tid >> 5;          // word slot 0..7

  __shared__ uint32_t s_words[kQuantWords][kD * kPlanes];   // [word][row = c*4 + j]
  __shared__ uint32_t s_m1[kHalfWaves][kD], s_m2[kHalfWaves][kD];

  float lo4[4], inv4[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = h * kD + 4 * cg + t;
    const float lo = ordered_to_float(ws.kmin[c]);
    const float r = __fsub_rn(ordered_to_float(ws.kmax[c]), lo);
    lo4[t] = lo;
    inv4[t] = r > 0.0f ? __fdiv_rn(16.0f, r) : 0.0f;
  }
  uint32_t m1[4] = {0u, 0u, 0u, 0u}, m2[4] = {0u, 0u, 0u, 0u};
  const float* head_keys = keys + int64_t(h) * stride_head + 4 * cg;

  const int tile_begin = blockIdx.x * tiles_per_wg;
  const int tile_end = min(num_tiles, tile_begin + tiles_per_wg);
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int64_t word_base = int64_t(tile) * kQuantWords;
    for (int wl = hw; wl < kQuantWords; wl += kHalfWaves) {
      const int64_t key0 = (word_base + wl) * 32;
      uint32_t x[32];
#pragma unroll
      for (int half = 0; half < 32; half += kKeyBatch) {
        float4 v[kKeyBatch];
        // unconditional loads: keys past the head's length read its last
        // key and are masked below
#pragma unroll
        for (int b = 0; b < kKeyBatch; ++b) {
          const int64_t i = min<int64_t>(key0 + half + b, last_key);
          v[b] = *reinterpret_cast<const float4*>(head_keys + i * stride_token);
        }
#pragma unroll
        for (int b = 0; b < kKeyBatch; ++b) {
          const bool valid = key0 + half + b < nh;
          const float kv[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
          uint32_t packed = 0u;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float u = __fmul_rn(__fsub_rn(kv[t], lo4[t]), inv4[t]);
            uint32_t code = u >= 15.0f ? 15u : static_cast<uint32_t>(u);   // u >= 0: trunc = floor
            code = valid ? code : 0u;
            m1[t] += code;
            m2[t] += code * code;
            packed |= code << (4 * t);
          }
          x[half + b] = packed;
        }
      }
      uint32_t y[16];
      transpose32x16(x, y);
      // word p = 4t + i holds bit i of channel t's code = plane 3 - i
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_words[wl][(4 * cg + t) * kPlanes + (3 - i)] = y[4 * t + i];
    }
    __syncthreads();
    // store: thread = two plane rows, 32 words (128 bytes) each
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = tid + rr * kQuantThreads;           // c * 4 + j
      uint32_t* dst = planes + (int64_t(h) * kD * kPlanes + row) * ldw + word_base;
      if (word_base + kQuantWords <= ldw) {
#pragma unroll
        for (int v = 0; v < kQuantWords / 4; ++v)
          reinterpret_cast<uint4*>(dst)[v] = make_uint4(s_words[4 * v][row], s_words[4 * v + 1][row],
                                                        s_words[4 * v + 2][row], s_words[4 * v + 3][row]);
      } else {
        for (int v = 0; word_base + v < ldw; ++v) dst[v] = s_words[v][row];
      }
    }
    __syncthreads();
  }
  // moments: fold the 8 word slots, then one 64-bit atomic per channel
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s_m1[hw][4 * cg + t] = m1[t];
    s_m2[hw][4 * cg + t] = m2[t];
  }
  __syncthreads();
  if (tid < kD) {
    unsigned long long a = 0, b = 0;
    for (int r = 0; r < kHalfWaves; ++r) {
      a += s_m1[r][tid];
      b += s_m2[r][tid];
    }
    atomicAdd(&ws.s1[h * kD + tid], a);
    atomicAdd(&ws.s2[h * kD + tid], b);
  }
}

__global__ void pack_final_kernel(int count, int64_t n_bound, const int32_t* __restrict__ lengths, PackWorkspace ws,
                                  float* __restrict__ lo, float* __restrict__ step, float* __restrict__ var) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const int64_t n = head_length(lengths, i / kD, n_bound);
  if (n == 0) {   // an empty head: no range, zero step and variance
    lo[i] = 0.0f;
    step[i] = 0.0f;
    if (var) var[i] = 0.0f;
    return;
  }
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

// Decode-time append: keys n_h .. n_h + m - 1 of every head h (n_h = n, or
// the head's own length) are quantized with the head's packed quantizer (lo,
// step fixed; inv = fl32(16 / fl32(16 step)), the packer's own inverse) and
// their codes, clamped to [0, 15], written into the planes.  One thread per
// (head, channel, word slot) builds a touched word's new bits for all four
// planes and replaces them (read-modify-write; no other thread touches that
// word).  Slot wi is word n_h / 32 + wi; slots past the last touched word
// return at once.
__global__ __launch_bounds__(256) void append_kernel(const float* __restrict__ keys, int64_t stride_head,
                                                     int64_t stride_token, int m, int64_t n,
                                                     const int32_t* __restrict__ lengths, int64_t ldw, int nw,
                                                     int H, uint32_t* __restrict__ planes,
                                                     const float* __restrict__ lo, const float* __restrict__ step) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= int64_t(H) * kD * nw) return;
  const int wi = static_cast<int>(gid % nw);
  const int c = static_cast<int>((gid / nw) % kD);
  const int h = static_cast<int>(gid / (int64_t(nw) * kD));
  const int64_t nh = head_length(lengths, h, n);
  const int64_t w = nh / 32 + wi;
  if (w * 32 >= nh + m) return;            // (nh + m <= n + m <= 32 ldw, so w < ldw below)
  const float l = lo[h * kD + c];
  const float r = __fmul_rn(step[h * kD + c], 16.0f);   // exact power-of-two scaling
  const float inv = r > 0.0f ? __fdiv_rn(16.0f, r) : 0.0f;
  uint32_t mask = 0u, bits[kPlanes] = {0u, 0u, 0u, 0u};
  const int64_t first = max(nh, w * 32), last = min(nh + m, w * 32 + 32);
  for (int64_t i = first; i < last; ++i) {
    const float x = keys[int64_t(h) * stride_head + (i - nh) * stride_token + c];
    const float u = __fmul_rn(__fsub_rn(x, l), inv);
    const int code = static_cast<int>(fminf(fmaxf(floorf(u), 0.0f), 15.0f));
    const uint32_t b = 1u << static_cast<int>(i & 31);
    mask |= b;
#pragma unroll
    for (int j = 0; j < kPlanes; ++j) bits[j] |= ((code >> (kPlanes - 1 - j)) & 1) ? b : 0u;
  }
  uint32_t* row = planes + (int64_t(h) * kD + c) * kPlanes * ldw + w;
#pragma unroll
  for (int j = 0; j < kPlanes; ++j) row[j * ldw] = (row[j * ldw] & ~mask) | bits[j];
}

// After an append with per-head lengths: lengths[h] = n_h + m (a launch of
// its own, so that every thread of the append has read the old length).
__global__ void append_lengths_kernel(int32_t* __restrict__ lengths, int64_t n, int m, int H) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h < H) lengths[h] = static_cast<int32_t>(head_length(lengths, h, n) + m);
}

}  // namespace

hipError_t launch_append(const float* keys, int64_t stride_head, int64_t stride_token, int m, int H, int64_t n,
                         int32_t* lengths, int64_t ldw, uint32_t* planes, const float* lo, const float* step,
                         hipStream_t stream) {
  // word slots per (head, channel): exactly the touched words for one
  // start n, enough for any start with per-head lengths
  const int nw = lengths ? (m + 31) / 32 + 1 : static_cast<int>((n + m - 1) / 32 - n / 32 + 1);
  const int64_t threads = int64_t(H) * kD * nw;
  const int blocks = static_cast<int>((threads + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(256), 0, stream, keys, stride_head, stride_token, m, n,
                     lengths, ldw, nw, H, planes, lo, step);
  if (lengths)
    hipLaunchKernelGGL(append_lengths_kernel, dim3((H + 255) / 256), dim3(256), 0, stream, lengths, n, m, H);
  return hipGetLastError();
}

hipError_t launch_pack(const float* keys, int64_t stride_head, int64_t stride_token, int H, int64_t n,
                       const int32_t* lengths, int64_t ldw, uint32_t* planes, float* lo, float* step, float* var,
                       const PackWorkspace& ws, hipStream_t stream) {
  const int count = H * kD;
  hipLaunchKernelGGL(pack_init_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, ws, count);
  const int range_blocks = static_cast<int>((n + kRangeRows - 1) / kRangeRows);
  hipLaunchKernelGGL(pack_range_kernel, dim3(range_blocks, H), dim3(kRangeThreads), 0, stream, keys,
                     stride_head, stride_token, n, lengths, ws);
  // tiles cover every word of the padded rows, so padding words are written
  // as zero; about 1024 workgroups in total, whatever H
  const int num_tiles = static_cast<int>((ldw + kQuantWords - 1) / kQuantWords);
  const int64_t want = (1024 + H - 1) / H;
  const int tiles_per_wg = static_cast<int>(std::max<int64_t>(1, (num_tiles + want - 1) / want));
  const int quant_blocks = (num_tiles + tiles_per_wg - 1) / tiles_per_wg;
  hipLaunchKernelGGL(pack_quant_kernel, dim3(quant_blocks, H), dim3(kQuantThreads), 0, stream, keys,
                     stride_head, stride_token, n, lengths, ldw, num_tiles, tiles_per_wg, planes, ws);
  hipLaunchKernelGGL(pack_final_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, count, n, lengths, ws,
                     lo, step, var);
  return hipGetLastError();
}

}  // namespace fathom
