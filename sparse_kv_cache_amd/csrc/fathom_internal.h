// Internal declarations shared by the libfathom translation units (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fathom {

constexpr int kD = 128;            // channels per key (the only d supported)
constexpr int kPlanes = 4;         // 4-bit K cache -> 4 bit planes
constexpr int kMaxK = 4096;        // largest top-k
constexpr size_t kChunkTableBytes = 12288;   // one (KV head, query chunk) scan table
constexpr int kCandCap = 16384;    // candidate slots per query (merge sorts them in LDS)
constexpr int kSampleBlockKeys = 1024;  // keys per sampled block (32 plane words)
constexpr int kSampleMaxBlocks = 8;     // sampled blocks per KV head
constexpr int kSampleMaxKeys = kSampleBlockKeys * kSampleMaxBlocks;
constexpr int kQueryChunk = 4;     // query heads scored together per workgroup
// Rescue of queries whose candidate list missed (too short or overflowed):
// up to kRescueSlots such queries per call are rescored by workgroups of the
// merge launch, each taking a slice of at most kRescueSlice keys of the head
// (at most kRescueMaxWgs slices, so heads up to 4M keys).
constexpr int kRescueSlots = 2;
constexpr int kRescueSlice = 16384;
constexpr int kRescueMaxWgs = 256;
constexpr int kRescueHistBins = 2048;
constexpr int64_t kMaxKeys = int64_t(1) << 26;
// One head's plane block (d * 4 rows of ldw words) is addressed with 32-bit
// byte offsets; the largest block is therefore 2^32 - 1 bytes (ldw <=
// 2^21 - 4, i.e. at most 67,108,736 keys per head).
constexpr int64_t kMaxHeadBytes = (int64_t(1) << 32) - 1;
constexpr int64_t kMaxStoreBytes = int64_t(1) << 42;   // 4 TiB of planes per call

// Monotone map float -> uint32 (larger float <-> larger integer).
__host__ __device__ inline uint32_t float_to_ordered(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__host__ __device__ inline float ordered_to_float(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __builtin_bit_cast(float, u);
}

// Keys held by head h: n, or with a per-head length array (ragged
// sessions) lengths[h] clamped to [0, n].
__device__ inline int64_t head_length(const int32_t* lengths, int h, int64_t n) {
  if (!lengths) return n;
  const int64_t v = lengths[h];
  return v < 0 ? 0 : (v > n ? n : v);
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the first HIP error met while enqueuing.

struct PackWorkspace {
  uint32_t* kmin;   // [H][D] ordered-float minimum
  uint32_t* kmax;   // [H][D] ordered-float maximum
  unsigned long long* s1;  // [H][D] sum of codes
  unsigned long long* s2;  // [H][D] sum of squared codes
};

hipError_t launch_pack(const float* keys, int64_t stride_head, int64_t stride_token, int H, int64_t n,
                       const int32_t* lengths, int64_t ldw, uint32_t* planes, float* lo, float* step, float* var,
                       const PackWorkspace& ws, hipStream_t stream);

hipError_t launch_append(const float* keys, int64_t stride_head, int64_t stride_token, int m, int H, int64_t n,
                         int32_t* lengths, int64_t ldw, uint32_t* planes, const float* lo, const float* step,
                         hipStream_t stream);

hipError_t launch_allocate(const float* q, int num_q, int group, const float* var, int budget,
                           uint8_t* alloc, hipStream_t stream);

hipError_t launch_control_allocate(const float* q, int num_q, int mode, int budget, uint8_t* alloc,
                                   hipStream_t stream);

// Attention over selected rows: chunks per query, and the two launches
// (partials into part [num_q][attend_splits(k)][kD + 2], then the combine).
int attend_splits(int k);
hipError_t launch_attend(const uint16_t* k_rows, const uint16_t* v_rows, int64_t stride_head,
                         int64_t stride_token, int64_t n, const int32_t* lengths, const float* q, const int32_t* idx, int num_q,
                         int group, int k, float scale, float* part, float* out, hipStream_t stream);

// Copies the union rows of one KV head (query group's allocation at alloc,
// [group][kD]) from src_head (device view of pinned host memory) into
// dst_head (HBM), same layout; other rows are left as they are.
hipError_t launch_stage_union(const uint32_t* src_head, uint32_t* dst_head, const uint8_t* alloc, int group,
                              int64_t ldw, hipStream_t stream);

// Measurement aid: a streaming read of `bytes` (a multiple of 16) from src;
// sink holds stream_read_blocks() words (written only on an improbable value).
int stream_read_blocks();
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

struct ScanWorkspace {
  float* theta;      // [Q] candidate threshold per query
  uint32_t* count;   // [Q] candidates seen per query
  float* sample;     // [Q][kSampleMaxKeys] scores of the sampled keys
  uint2* cand;       // [Q][kCandCap] (score bits, key index)
  void* tables;      // [Q][kChunkTableBytes] per (KV head, query chunk) scan tables (at most Q chunks)
  uint2* rescue;     // [kRescueSlots][rescue_wgs][k] per-slice top-k lists (ordered score, index)
  uint2* rescue_cnt;       // [kRescueSlots][rescue_wgs] entries in each list, and its lowest (ordered) score
  uint32_t* rescue_hist;   // [kRescueSlots][kRescueHistBins] digits of all list entries
  uint32_t* rescue_done;   // [kRescueSlots] slices finished
  int rescue_wgs;          // slices (workgroups) per rescued query; 0: no rescue
};

// Rescue slices for heads of up to n keys (0 when a slice would exceed
// kRescueSlice keys).
inline int rescue_wgs_for(int64_t n) {
  const int64_t r = (n + kRescueSlice - 1) / kRescueSlice;
  return r <= kRescueMaxWgs ? static_cast<int>(r < 1 ? 1 : r) : 0;
}

struct ScanTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_scan_topk(const uint32_t* planes, const float* lo, const float* step, int H,
                            int64_t n, const int32_t* lengths, int64_t ldw, const float* q, const uint8_t* alloc,
                            int num_q,
                            int group, int k, int32_t* out_idx, float* out_score,
                            float* all_scores, const ScanWorkspace& ws, const ScanTiming* timing,
                            hipStream_t stream, const float* var = nullptr, int budget = 0,
                            uint8_t* alloc_out = nullptr);

}  // namespace fathom
