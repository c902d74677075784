// Plane-prefix key scan with fused top-k (gfx950).
//
// "Fathom Makes KV-Cache Scans Query-Adaptive for Long-Context Decoding",
// paras 1-2, and "Fathom: Per-Query Read Depth for Sparse Decoding over
// Offloaded KV Caches", abstract s1-s3: every decode step ranks all n keys
// for a top-k, and each query reads only the first b_qc bit planes of each
// channel c.  With the planes MSB-first, the b-plane prefix of a channel is
// its b-bit quantized value, so the partially dequantized dot product is
//
//   s_q(i) = C_q + sum_c sum_{j < b_qc} W_qcj bit_{c,j}(i),
//   W_qcj  = q_c step_c 2^(3-j),
//   C_q    = sum_c q_c (lo_c + step_c 2^(3-b_qc))      (bin-centre offsets).
//
// Launch sequence per call (all on the caller's stream):
//   1. scan_sample_kernel    one workgroup per (sampled 1024-key block, KV
//                            head, query chunk).  With the fused allocation
//                            its wavefront g first allocates query g's bits
//                            (allocate_wave.h).  It builds the chunk's union
//                            and scan table (workgroup 0 stores the table),
//                            then scores its block the way the main kernel
//                            does.  When the sample rank of the threshold is
//                            <= 32 it keeps only per-group maxima of the
//                            block's scores, otherwise every sampled score;
//   2. scan_threshold_kernel only when that rank is > 32 or the heads have
//                            lengths of their own: per query, a digit select
//                            over the sampled scores gives theta;
//   3. scan_main_kernel      every key of every head, see below.  With the
//                            group maxima, each workgroup selects theta
//                            itself from them while its first plane loads
//                            are in flight.  Keys whose score can reach
//                            theta go to a per-query candidate list;
//   4. scan_merge_kernel     per query, one digit pass orders the candidates
//                            into buckets and places the k best by counting.
//                            If the list holds fewer than k keys scoring >=
//                            theta, or overflowed, workgroup 0 recomputes the
//                            query's scores and selects the exact top-k
//                            (ties by index).
//
// Main kernel.  A workgroup owns one KV head and a chunk of <= 4 of its GQA
// query heads, and reads, once, the union U of the chunk's plane prefixes
// (padded with zero-weight rows to whole 64-plane blocks).  The score is a
// dense contraction over the union planes, S[q][key] = sum_p W[q][p] bit[p][key],
// done on the matrix cores as v_mfma_i32_16x16x64_i8:
//   A (16 x 64): each query's weights of the block in fixed point,
//       V = round(W 2^30 / sum|W|), split into four balanced base-256 int8
//       digits ("limbs"); row 4g+l holds limb l of query g;
//   B (64 x 16): the bits.  The plane words of a block stream into LDS by DMA;
//       the LDS transpose read (ds_read_b64_tr_b8) gives each lane, per byte,
//       one plane of eight consecutive keys, and one AND per dword with
//       0x01010101 << e keeps key e's bit of every plane, as bit * 2^e;
// so one MFMA gives all 4 queries' 4 limb sums of 16 keys over 64 planes (a
// union's last block of at most 32 planes takes v_mfma_i32_16x16x32_i8 on
// half the rows instead); the epilogue unscales the limbs by shifts and
// recombines them into the exact
// integer t = sum_p V bit, and the score is fma(float(t), sum|W| 2^-30, C_q).
// The tables (limbs, scale, offset C_q, union rows) are built once per chunk
// by the sample kernel.  Keys whose t can reach theta are kept in LDS lists
// per (wavefront, query), in the LDS the union's table leaves free, and
// flushed to the global candidate list at the end.

#include <hip/hip_ext.h>

#include <algorithm>
#include <climits>
#include <cstddef>
#include <type_traits>

#include "allocate_wave.h"
#include "fathom_internal.h"
#include "wave_ops.h"

#ifndef WAVE_X
#define WAVE_X 2
#endif
#ifndef MAIN_STAGES
#define MAIN_STAGES 3
#endif

namespace fathom {
namespace {

constexpr int kMaxUnion = kD * kPlanes;
constexpr int kBlockPlanes = 64;               // union planes per MFMA (its K)
constexpr int kMaxBlocks = kMaxUnion / kBlockPlanes;
// the union is padded with readable zero-weight rows to whole K blocks
constexpr int kPadPlanes = kBlockPlanes;
// A tile is 32 plane words (1024 keys).  Each wavefront takes kWaveX
// groups of 4 words: 16 MFMA columns of 8 keys, in two 64-key segments.
// kWaveX = 2 (4 wavefronts of 110 VGPRs, 4 workgroups per CU) measured
// faster on the 1M-key step than kWaveX = 1 (8 wavefronts of 64-66 VGPRs,
// 3 or 4 workgroups per CU): 45.5 against 48-50 us.
constexpr int kTileWords = 32;
constexpr int kWaveX = WAVE_X;
constexpr int kWaveWords = 4 * kWaveX;
constexpr int kWaveKeys = 8 * kWaveX;                 // keys per lane and tile (one accumulator each)
constexpr int kMainWaves = kTileWords / kWaveWords;
constexpr int kMainThreads = 64 * kMainWaves;
constexpr int kDmaPerWave = 8 / kMainWaves;          // a stage is 8 DMA loads
#ifdef MAIN_WG_PER_CU
constexpr int kMainWgPerCu = MAIN_WG_PER_CU;
#else
constexpr int kMainWgPerCu = kWaveX == 2 ? 4 : 3;    // 16 or 24 wavefronts per CU
#endif
// Workgroup LDS ring of plane words: a stage holds one K block of the
// workgroup's tile (64 planes x 32 words), written by eight LDS DMA loads of
// 8 planes x 128 bytes (two per wave; whole 128-byte lines).  Loads run
// kMainStages - 2 stages ahead of the stage being read, plus the one issued
// while it is read.
constexpr int kMainStages = MAIN_STAGES;
constexpr int kDmaDwords = 8 * kTileWords + 8;           // one DMA load (8 planes x 32 words) + bank padding
constexpr int kStageDwords = 8 * kDmaDwords;
#ifndef WAVE_CAND
#define WAVE_CAND 32
#endif
constexpr int kWaveCand = WAVE_CAND;           // candidates per (wave, query) buffered in LDS, at least
// Largest sample rank served by per-block group maxima: up to half the
// lanes, so that the rank-th largest lane maximum usually leaves at most 64
// candidates for the sort (nearer 64 the selection falls back to a search).
constexpr int kTopR = 32;
constexpr int kListEntries = 512;              // group maxima kept per query (all sampled blocks)
constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / 64;

struct ScanArgs {
  const uint32_t* planes;
  const float* lo;
  const float* step;
  const float* q;
  const uint8_t* alloc;
  const float* var;     // non-null: the sample kernel computes the allocations itself
  int budget;           //   (budget bits) and writes them to alloc_out, which alloc then names
  uint8_t* alloc_out;
  int64_t n;
  const int32_t* lengths;   // null, or keys per head (head_length clamps them to [0, n])
  int64_t ldw;
  int nwords;         // ceil(n / 32)
  int group;          // query heads per KV head
  int cph;            // query chunks of this launch per KV head
  int qoff;           // first query of chunk 0 within its head
  int tiles;          // kTileWords-word tiles per head
  int tiles_per_wg;   // tiles handled by one main workgroup
  int main_wgs;       // main workgroups per (head, query chunk)
  int interleave;     // main-kernel launch order: chunks interleaved (1) or one after another (0)
  int ramp_step;      // scan issue priority: tiles per level of its fall (see TileScanner::run)
  float* theta;
  uint32_t* count;
  float* sample;
  uint2* cand;
  float* all_scores;
  int sample_stride;  // distance between sampled blocks, in 1024-key blocks
  int rsel;           // sample rank of the threshold
  int top_lists;      // rsel <= kTopR: sampled blocks store their group maxima only,
                      //   and the main kernel selects theta from them
  int nsb;            // sampled blocks per head
  int chunks_per_head;
  void* tables;       // [H * chunks_per_head] ChunkTable, written by the sample kernel
  int k;              // top-k
  int num_q;          // query heads of the call
  uint2* rescue;      // rescue lists, counts, histograms and finished-slice counters (see the merge)
  uint2* rescue_cnt;
  uint32_t* rescue_hist;
  uint32_t* rescue_done;
  int rescue_wgs;
};

// Sampled blocks of a head of nh keys when every head has its own length:
// nsb blocks, block i at 1024-key block i * stride (stride from the head's
// own length, so the sample spreads over it).  Returns the stride; svalid
// gets the number of sampled keys below nh.
__device__ inline int ragged_sample(int64_t nh, int nsb, int& svalid) {
  const int64_t nbl = (nh + kSampleBlockKeys - 1) / kSampleBlockKeys;
  const int64_t stride = max<int64_t>(1, nbl / nsb);
  int64_t sv = 0;
  for (int i = 0; i < nsb; ++i) {
    const int64_t left = nh - int64_t(i) * stride * kSampleBlockKeys;
    sv += left <= 0 ? 0 : (left < kSampleBlockKeys ? left : kSampleBlockKeys);
  }
  svalid = static_cast<int>(sv);
  return static_cast<int>(stride);
}

template <int GQ>
struct UnionLds {
  float w[kMaxUnion + kPadPlanes][4];        // W_qcj per union plane; 0 where the query skips it
  uint32_t rowoff[kMaxUnion + kPadPlanes];   // byte offset of the plane row (c*4 + j) in the head
  int off[kPlanes][kD];
  int u[kD];
  double cpart[2][GQ];
  float C[GQ];
  int U;
};

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));

// What the main kernel needs of a (KV head, query chunk): the union rows, the
// MFMA A operands (int8 limbs of the fixed-point plane weights), the scales
// and the score offsets.  Built once per call by the sample kernel.
// Per K block: its A operand and the offsets of its 64 union rows.  Blocks
// sit one after another behind a small header, so the blocks a union uses
// are a prefix of the table (the main kernel keeps its candidates in the
// space of the unused ones).
struct TableBlock {
  uint4 A[4][16];                            // [K slice][row 4g + limb]: 16 int8 limbs
  uint32_t rowoff[kBlockPlanes];             // byte offset of each union row in the head (0: padding)
};
struct ChunkTable {
  float sigma[4];                            // fixed-point scale of each query's weights
  float C[4];                                // score offsets C_q
  int U;                                     // union planes
  int pad_[3];
  TableBlock blk[kMaxBlocks];
};
constexpr int kTableHeadBytes = static_cast<int>(offsetof(ChunkTable, blk));
static_assert(kTableHeadBytes % 16 == 0 && sizeof(TableBlock) % 16 == 0, "A operands stay 16-byte aligned");
static_assert(sizeof(ChunkTable) <= kChunkTableBytes, "chunk table fits its workspace slot");
static_assert(sizeof(ChunkTable) % 16 == 0, "chunk tables are copied as uint4");

// K blocks of a union of U planes; at least one, so an empty union is one
// block of zero weights
__host__ __device__ inline int nblocks_of(int U) { return U > 0 ? (U + kBlockPlanes - 1) / kBlockPlanes : 1; }

// A union of more than one K block whose last block holds at most 32 planes
// scans that block with K = 32 MFMAs: half the B-operand masks and half the
// MFMA work.  Its planes then sit in the first 8 rows of each 16-row slice
// (union plane 64b + pl at slice pl / 8, byte pl % 8), where one transpose
// read per key segment gathers them in the K = 32 operand order; the other
// rows are padding.
__host__ __device__ inline bool half_last_block(int U) {
  return U > kBlockPlanes && U - kBlockPlanes * (nblocks_of(U) - 1) <= 32;
}
// The union plane at table position tp (block tp / 64, slice (tp % 64) / 16,
// byte tp % 16), or -1 for padding.
__host__ __device__ inline int union_plane_at(int tp, int U) {
  const int b = tp / kBlockPlanes, bp = tp % kBlockPlanes;
  int p = tp;
  if (half_last_block(U) && b == nblocks_of(U) - 1) {
    if ((bp & 15) >= 8) return -1;
    p = b * kBlockPlanes + 8 * (bp >> 4) + (bp & 15);
  }
  return p < U ? p : -1;
}
// The table position of union plane p < U (inverse of union_plane_at).
__host__ __device__ inline int table_pos_of(int p, int U) {
  const int b = p / kBlockPlanes, pl = p % kBlockPlanes;
  if (half_last_block(U) && b == nblocks_of(U) - 1) return b * kBlockPlanes + 16 * (pl >> 3) + (pl & 7);
  return p;
}

__device__ inline int chunk_index(const ScanArgs& a, int cy) {
  const int h = cy / a.cph;
  return h * a.chunks_per_head + a.qoff / kQueryChunk + cy % a.cph;
}
__device__ inline int chunk_index(const ScanArgs& a) { return chunk_index(a, static_cast<int>(blockIdx.y)); }

__device__ inline int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  return __popcll(mask & below);
}

// ------------------------------------------------ wavefront primitives
template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ double dpp_f64(double old, double v) {
  const uint64_t o = __builtin_bit_cast(uint64_t, old), x = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = dpp_u32<Ctrl, RowMask>(static_cast<uint32_t>(o), static_cast<uint32_t>(x));
  const uint32_t hi = dpp_u32<Ctrl, RowMask>(static_cast<uint32_t>(o >> 32), static_cast<uint32_t>(x >> 32));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Inclusive prefix sum over the wavefront's 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += dpp_u32<kDppRowShr + 1>(0u, v);
  v += dpp_u32<kDppRowShr + 2>(0u, v);
  v += dpp_u32<kDppRowShr + 4>(0u, v);
  v += dpp_u32<kDppRowShr + 8>(0u, v);
  v += dpp_u32<kDppRowBcast15, 0xa>(0u, v);
  v += dpp_u32<kDppRowBcast31, 0xc>(0u, v);
  return v;
}

__device__ __forceinline__ uint32_t read_lane(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Max and min over the wavefront, returned to every lane.
__device__ __forceinline__ uint2 wave_max_min(uint32_t mx, uint32_t mn) {
  mx = max(mx, dpp_u32<kDppXor1>(mx, mx));
  mn = min(mn, dpp_u32<kDppXor1>(mn, mn));
  mx = max(mx, dpp_u32<kDppXor2>(mx, mx));
  mn = min(mn, dpp_u32<kDppXor2>(mn, mn));
  mx = max(mx, dpp_u32<kDppRowHalfMirror>(mx, mx));
  mn = min(mn, dpp_u32<kDppRowHalfMirror>(mn, mn));
  mx = max(mx, dpp_u32<kDppRowMirror>(mx, mx));
  mn = min(mn, dpp_u32<kDppRowMirror>(mn, mn));
  mx = max(mx, dpp_u32<kDppRowBcast15, 0xa>(mx, mx));
  mn = min(mn, dpp_u32<kDppRowBcast15, 0xa>(mn, mn));
  mx = max(mx, dpp_u32<kDppRowBcast31, 0xc>(mx, mx));
  mn = min(mn, dpp_u32<kDppRowBcast31, 0xc>(mn, mn));
  return make_uint2(read_lane(mx, 63), read_lane(mn, 63));
}

// Sum over the wavefront (lane 63 ends with the total; returned to all).
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kDppXor1>(0.0, v);
  v += dpp_f64<kDppXor2>(0.0, v);
  v += dpp_f64<kDppRowHalfMirror>(0.0, v);
  v += dpp_f64<kDppRowMirror>(0.0, v);
  v += dpp_f64<kDppRowBcast15, 0xa>(0.0, v);
  v += dpp_f64<kDppRowBcast31, 0xc>(0.0, v);
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = read_lane(static_cast<uint32_t>(b), 63), hi = read_lane(static_cast<uint32_t>(b >> 32), 63);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ inline double pow2_3_minus(int b) {
  // 2^(3 - b) for b in 0..4
  return b == 0 ? 8.0 : b == 1 ? 4.0 : b == 2 ? 2.0 : b == 3 ? 1.0 : 0.5;
}


// Per-channel inputs of build_union (thread t < kD holds channel t), loaded
// ahead so their latency overlaps other work.
struct UnionInputs {
  float lo, st, q[4];
  uint32_t b4;   // the channel's plane count for query g in byte g (set before build_union)
};

// Every thread loads (threads past kD re-read channel kD - 1 and ignore it):
// loads under a branch would be waited for inside it.
template <int GQ>
__device__ inline UnionInputs load_union_inputs(const ScanArgs& a, int h, int q0) {
  UnionInputs in{0.0f, 0.0f, {0.0f, 0.0f, 0.0f, 0.0f}, 0u};
  const int t = min(static_cast<int>(threadIdx.x), kD - 1);
  in.lo = a.lo[h * kD + t];
  in.st = a.step[h * kD + t];
#pragma unroll
  for (int g = 0; g < GQ; ++g) in.q[g] = a.q[int64_t(q0 + g) * kD + t];
  if (!a.var) {   // uniform: a given allocation (with a.var the sample kernel computes it)
#pragma unroll
    for (int g = 0; g < GQ; ++g) in.b4 |= static_cast<uint32_t>(a.alloc[int64_t(q0 + g) * kD + t]) << (8 * g);
  }
  return in;
}

// Builds the union plane list of a query chunk (queries q0 .. q0+GQ-1 on one
// KV head, channel inputs and planes per query in `in`), the per-plane
// weights and the score offsets C_q.  Needs blockDim.x >= kD; ends with
// __syncthreads().
template <int GQ>
__device__ void build_union(const ScanArgs& a, const UnionInputs& in, UnionLds<GQ>& s) {
  const int t = threadIdx.x;
  int u = 0, bq[4] = {0, 0, 0, 0};
  float qv[4] = {0.0f, 0.0f, 0.0f, 0.0f}, st = 0.0f;
  if (t < kD) {
    const float lo = in.lo;
    st = in.st;
    double cp[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      bq[g] = min(static_cast<int>((in.b4 >> (8 * g)) & 255u), kPlanes);
      qv[g] = in.q[g];
      u = max(u, bq[g]);
      cp[g] = static_cast<double>(qv[g]) *
              (static_cast<double>(lo) + static_cast<double>(st) * pow2_3_minus(bq[g]));
    }
    s.u[t] = u;
    // C_q: per-wave double sums over 64 channels, then the two halves
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const double v = wave_sum(cp[g]);
      if ((t & 63) == 0) s.cpart[t >> 6][g] = v;
    }
  }
  __syncthreads();
  // Union plane list in (plane j asc, channel c asc) order: plane j of
  // channel c is present when j < u_c (any order would do: the score is a
  // plain sum).
  // cnt[j] = #channels with u > j; exclusive prefix over channels per level.
  if (t < 64) {
    int base = 0;
    for (int j = 0; j < kPlanes; ++j) {
      const int v0 = s.u[2 * t] > j, v1 = s.u[2 * t + 1] > j;
      const int incl = static_cast<int>(wave_incl_sum(static_cast<uint32_t>(v0 + v1)));
      const int excl = base + incl - v0 - v1;
      s.off[j][2 * t] = excl;
      s.off[j][2 * t + 1] = excl + v0;
      base += static_cast<int>(read_lane(static_cast<uint32_t>(incl), 63));
    }
    if (t == 0) s.U = base;
  }
  if (t < GQ) s.C[t] = static_cast<float>(s.cpart[0][t] + s.cpart[1][t]);
  __syncthreads();
  if (t < kD) {
    for (int j = 0; j < u; ++j) {
      const int o = s.off[j][t];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bool on = g < GQ && j < bq[g];
        s.w[o][g] = on ? __fmul_rn(qv[g], st) * static_cast<float>(8 >> j) : 0.0f;
      }
      s.rowoff[o] = static_cast<uint32_t>((t * kPlanes + j) * a.ldw * 4);
    }
  }
  // padding up to whole 64-plane blocks: row 0, weight 0
  const int U = s.U;
  const int pad = (kPadPlanes - U % kPadPlanes) % kPadPlanes;
  if (t < pad) {
    s.w[U + t][0] = s.w[U + t][1] = s.w[U + t][2] = s.w[U + t][3] = 0.0f;
    s.rowoff[U + t] = 0u;
  }
  __syncthreads();
}

// Builds the main kernel's table of this (KV head, query chunk) in T and,
// if store is set, stores it in the workspace.  Needs blockDim.x >= 64; contains barriers.
template <int GQ>
__device__ void build_limbs(const UnionLds<GQ>& s, ChunkTable& T, double (&wsum)[4], int nblk);

// Workgroup barrier for LDS data only: unlike __syncthreads() it does not
// wait for outstanding global loads, so LDS DMA loads issued before it stay
// in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

// First part: rows, offsets and union size (a barrier must follow).
template <int GQ>
__device__ void table_rows(const UnionLds<GQ>& s, ChunkTable& T) {
  const int U = s.U;
  for (int i = threadIdx.x; i < kMaxUnion; i += blockDim.x) {
    const int p = union_plane_at(i, U);
    T.blk[i / kBlockPlanes].rowoff[i % kBlockPlanes] = p >= 0 ? s.rowoff[p] : 0u;
  }
  if (threadIdx.x < 4) T.C[threadIdx.x] = static_cast<int>(threadIdx.x) < GQ ? s.C[threadIdx.x] : 0.0f;
  if (threadIdx.x == 0) T.U = U;
}

// Second part: the A operands and scales, then the store.
template <int GQ>
__device__ void table_limbs(const UnionLds<GQ>& s, ChunkTable& T, double (&wsum)[4]) {
  build_limbs<GQ>(s, T, wsum, nblocks_of(s.U));   // ends with a barrier
}

// Stores the finished table T for the main kernel.  (Issued at the end of
// the sample kernel: a barrier or stage wait after a store waits for its
// write to complete.)
// Every sampled-block workgroup of a chunk builds the same table; workgroup
// `part` of `parts` stores every parts-th piece of it.
__device__ void store_table(const ScanArgs& a, const ChunkTable& T, int part, int parts) {
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(a.tables) + size_t(chunk_index(a)) * kChunkTableBytes);
  const uint4* src = reinterpret_cast<const uint4*>(&T);
  for (int i = part * blockDim.x + threadIdx.x; i < static_cast<int>(sizeof(ChunkTable) / 16); i += parts * blockDim.x)
    dst[i] = src[i];
}

// ----------------------------------------------------------- block select

struct SelectLds {
  uint32_t hist[kSelectWaves][256];
  uint32_t total[256];
  uint32_t wmm[3][kSelectWaves];   // per-wave max, min, count (block_max_min)
  uint32_t sel;
  uint32_t rem;
};

// One radix pass of a block-wide select: given the per-wave histograms of
// the current digit, finds the bin holding the r-th largest value.  Returns
// (bin, r minus the count in the bins above it).
__device__ uint2 select_bin(SelectLds& L, uint32_t r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int b = tid; b < 256; b += blockDim.x) {
    uint32_t sum = 0;
    for (int w = 0; w < kSelectWaves; ++w) sum += L.hist[w][b];
    L.total[b] = sum;
  }
  __syncthreads();
  if (wave == 0) {
    // lane l owns bins 255-4l .. 252-4l (descending order across lanes)
    uint32_t c[4], own = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { c[j] = L.total[255 - 4 * lane - j]; own += c[j]; }
    const uint32_t incl = wave_incl_sum(own);
    uint32_t before = incl - own;   // count in the bins above this lane's bins
    if (before < r && incl >= r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before + c[j] >= r) {
          L.sel = static_cast<uint32_t>(255 - 4 * lane - j);
          L.rem = r - before;
          break;
        }
        before += c[j];
      }
    }
  }
  __syncthreads();
  const uint2 out = make_uint2(L.sel, L.rem);
  __syncthreads();
  return out;
}

__device__ inline void clear_hist(SelectLds& L) {
  for (int i = threadIdx.x; i < kSelectWaves * 256; i += blockDim.x) (&L.hist[0][0])[i] = 0;
  __syncthreads();
}

// Adds one to bin `bin` of this wave's histogram for every lane with `on`.
// When all such lanes share one bin (common in the leading digits, where the
// values agree) a single atomic adds the whole count.
__device__ inline void hist_add(uint32_t* wave_hist, bool on, uint32_t bin) {
  if (!on) return;
  // exec now holds exactly the lanes with `on`
  const uint32_t lead = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bin)));
  const uint64_t act = __ballot(1);
  if (__ballot(bin == lead) == act) {
    if ((threadIdx.x & 63) == __ffsll(static_cast<long long>(act)) - 1)
      atomicAdd(&wave_hist[lead], static_cast<uint32_t>(__popcll(act)));
  } else {
    atomicAdd(&wave_hist[bin], 1u);
  }
}

// Presence mask of a thread's register values: bit j set when value j
// (element tid + j * blockDim.x) is one of the first `count` elements.
template <int PT>
__device__ inline uint32_t present_below(uint32_t count) {
  uint32_t pm = 0;
#pragma unroll
  for (int j = 0; j < PT; ++j) pm |= (threadIdx.x + j * blockDim.x < count) ? (1u << j) : 0u;
  return pm;
}

// Block-wide max, min and number of the present values (ordered keys;
// value j of a thread is present when bit j of pm is set).
// Slots j >= nj (uniform per wavefront) hold nothing and are skipped.
template <int PT>
__device__ uint3 block_max_min(const uint32_t (&v)[PT], uint32_t pm, SelectLds& L, int nj = PT) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    if (j < nj && ((pm >> j) & 1u)) {
      mx = max(mx, v[j]);
      mn = min(mn, v[j]);
    }
  }
  const uint2 w = wave_max_min(mx, mn);
  const uint32_t c = read_lane(wave_incl_sum(static_cast<uint32_t>(__popc(pm))), 63);
  if (lane == 0) {
    L.wmm[0][wave] = w.x;
    L.wmm[1][wave] = w.y;
    L.wmm[2][wave] = c;
  }
  __syncthreads();
  // every wave combines the per-wave results, one per lane
  const bool ok = lane < static_cast<int>(blockDim.x >> 6);
  const uint2 b = wave_max_min(ok ? L.wmm[0][lane] : 0u, ok ? L.wmm[1][lane] : 0xffffffffu);
  const uint32_t cnt = read_lane(wave_incl_sum(ok ? L.wmm[2][lane] : 0u), 63);
  __syncthreads();
  return make_uint3(b.x, b.y, cnt);
}

// r-th largest (1-based, r <= number present) of the present ordered keys
// v[j] held by the block's threads.  Returns (key, r minus the number of
// values strictly above the key).  Radix select, 8 bits per pass, starting
// at the highest byte in which the present values differ.
template <int PT>
__device__ uint2 block_select_regs(const uint32_t (&v)[PT], uint32_t pm, uint32_t r, SelectLds& L) {
  const int wave = threadIdx.x >> 6;
  const uint3 mm = block_max_min<PT>(v, pm, L);
  const uint32_t diff = mm.x ^ mm.y;
  if (diff == 0) return make_uint2(mm.x, r);          // all present values equal
  const int top = (31 - __clz(diff)) & ~7;             // shift of the highest differing byte
  uint32_t pmask = top == 24 ? 0u : (0xffffffffu << (top + 8));
  uint32_t prefix = mm.x & pmask;
  for (int shift = top; shift >= 0; shift -= 8) {
    clear_hist(L);
#pragma unroll
    for (int j = 0; j < PT; ++j)
      hist_add(L.hist[wave], ((pm >> j) & 1u) && (v[j] & pmask) == prefix, (v[j] >> shift) & 255u);
    __syncthreads();
    const uint2 b = select_bin(L, r);
    prefix |= b.x << shift;
    pmask |= 255u << shift;
    r = b.y;
  }
  return make_uint2(prefix, r);
}

// ------------------------------------------------- one-pass digit select
// An 11-bit digit taken just below the highest bit in which the present
// values differ splits them into 2048 ordered buckets; one histogram and one
// descending scan give every bucket's first rank and the bucket holding a
// given rank.  Used for the threshold estimate (two passes) and for the
// candidate merge, which then orders each small bucket by counting.

constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
static_assert(kBins == kRescueHistBins, "the rescue histograms use the digit's bins");
constexpr int kBucketMax = 64;          // largest bucket the merge orders by counting
static_assert(kBins == 2 * kSelectThreads, "the scan gives each thread two bins");

struct DigitLds {
  uint32_t hist[kBins];     // elements per bucket
  uint32_t start[kBins];    // elements in the buckets above
  uint32_t cursor[kBins];   // scatter cursors
  uint32_t wave_total[kSelectWaves];
  uint32_t bstar;           // bucket holding the searched rank
  uint32_t bstart;          // its first rank
  uint32_t bcount;          // its size
  uint32_t big;             // a bucket at or above it exceeds kBucketMax
};

// Zeroes the histogram and cursors (a barrier must follow before use).
__device__ inline void digit_clear(DigitLds& D) {
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) {
    D.hist[i] = 0u;
    D.cursor[i] = 0u;
  }
  if (threadIdx.x == 0) D.big = 0u;
}

// Descending exclusive scan of the histogram and the bucket holding the
// element of 0-based rank r (r < total).  Needs blockDim.x == kBins / 2;
// begins after the histogram's barrier and ends with a barrier.
__device__ void digit_scan(DigitLds& D, uint32_t r) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int bh = kBins - 1 - 2 * t, bl = bh - 1;     // descending across threads
  const uint32_t ch = D.hist[bh], cl = D.hist[bl], own = ch + cl;
  const uint32_t incl = wave_incl_sum(own);
  if (lane == 63) D.wave_total[wave] = incl;
  __syncthreads();
  // totals of the waves before this one: one per lane, prefix-summed
  const uint32_t wt = wave_incl_sum(lane < kSelectWaves ? D.wave_total[lane] : 0u);
  const uint32_t base = wave == 0 ? 0u : read_lane(wt, wave - 1);
  const uint32_t excl = base + incl - own;
  D.start[bh] = excl;
  D.start[bl] = excl + ch;
  if (excl <= r && r < excl + ch) {
    D.bstar = static_cast<uint32_t>(bh);
    D.bstart = excl;
    D.bcount = ch;
  } else if (excl + ch <= r && r < excl + own) {
    D.bstar = static_cast<uint32_t>(bl);
    D.bstart = excl + ch;
    D.bcount = cl;
  }
  if ((excl <= r && ch > static_cast<uint32_t>(kBucketMax)) ||
      (excl + ch <= r && cl > static_cast<uint32_t>(kBucketMax)))
    D.big = 1u;
  __syncthreads();
}

// Same, over values produced on demand by get(i) for i < count.
template <class Get>
__device__ uint2 block_select_fn(int64_t count, uint32_t r, SelectLds& L, Get get) {
  const int tid = threadIdx.x, wave = tid >> 6;
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    clear_hist(L);
    for (int64_t i = tid; i < count; i += blockDim.x) {
      const uint32_t v = get(i);
      if ((v & pmask) == prefix) atomicAdd(&L.hist[wave][(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint2 b = select_bin(L, r);
    prefix |= b.x << shift;
    pmask |= 255u << shift;
    r = b.y;
  }
  return make_uint2(prefix, r);
}

// --------------------------------------------------------------- threshold

// Per query: a score with about rsel sampled scores at or above it.  Two
// digit passes (22 bits below the highest differing bit) locate the bucket
// of the rsel-th largest sample; theta is that bucket's lowest value, so at
// least rsel sampled keys score >= theta.
__global__ __launch_bounds__(kSelectThreads) void scan_threshold_kernel(
    const float* __restrict__ sample, int stot, uint32_t rsel, float* __restrict__ theta,
    uint32_t* __restrict__ count, const int32_t* __restrict__ lengths, int64_t n, int k, int group, int nsb) {
  __shared__ SelectLds L;
  __shared__ DigitLds D;
  constexpr int PT = kSampleMaxKeys / kSelectThreads;
  static_assert(PT * kSelectThreads == kSampleMaxKeys, "one register per sample slot");
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  if (lengths) {   // uniform: the rank from the query's own head length
    const int64_t nh = head_length(lengths, q / group, n);
    int svalid = 0;
    ragged_sample(nh, nsb, svalid);
    if (svalid == 0) {   // an empty head: no key passes
      if (tid == 0) {
        theta[q] = INFINITY;
        count[q] = 0u;
      }
      return;
    }
    int64_t r = (2 * int64_t(k) * svalid + nh - 1) / nh;
    r = max<int64_t>(r, min(svalid, 16));
    rsel = static_cast<uint32_t>(min<int64_t>(r, svalid));
  }
  uint32_t v[PT];
  // unconditional loads (the sample rows are allocated in full); slots past
  // the sample are masked afterwards
#pragma unroll
  for (int j = 0; j < PT; ++j) v[j] = __float_as_uint(sample[int64_t(q) * kSampleMaxKeys + tid + j * kSelectThreads]);
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int i = tid + j * kSelectThreads;
    v[j] = i < stot ? float_to_ordered(__uint_as_float(v[j])) : 0u;
  }
  digit_clear(D);
  const uint32_t pm = present_below<PT>(static_cast<uint32_t>(stot));
  const uint3 mm = block_max_min<PT>(v, pm, L);
  uint32_t th = mm.x;
  if (mm.x != mm.y) {
    uint32_t r = rsel - 1u;
    int hi = 32 - __clz(mm.x ^ mm.y);                // bits >= hi are common
    uint32_t pmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
    uint32_t prefix = mm.x & pmask;
    for (int pass = 0; pass < 2 && hi > 0; ++pass) {
      const int width = min(kDigitBits, hi), shift = hi - width;
      const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
      for (int j = 0; j < PT; ++j) hist_add(D.hist, ((pm >> j) & 1u) && (v[j] & pmask) == prefix, (v[j] >> shift) & dmask);
      __syncthreads();
      digit_scan(D, r);
      prefix |= D.bstar << shift;
      pmask |= dmask << shift;
      r -= D.bstart;
      hi = shift;
      // each thread clears the two bins it scanned; nobody reads them again
      D.hist[kBins - 1 - 2 * tid] = 0u;
      D.hist[kBins - 2 - 2 * tid] = 0u;
      __syncthreads();
    }
    th = prefix;   // lowest value of the bucket: the low bits are zero
  }
  if (tid == 0) {
    theta[q] = ordered_to_float(th);
    count[q] = 0u;
  }
}

// ------------------------------------------------ per-block group maxima
// For rsel <= kTopR the sample kernel stores, per sampled block and query,
// only the maxima of groups of gs keys scored by one lane (gs = 16 with 5 to
// 8 sampled blocks, 8 with 3 or 4, 4 with 2, 2 with 1, so that the blocks
// together keep at most kListEntries maxima), as ordered keys at the front
// of the query's sample row, block b at b * (1024 / gs).  The rsel-th
// largest of these maxima never exceeds the rsel-th largest sampled score
// and, while the best rsel scores fall in distinct groups, equals it; the
// threshold then selects from at most kListEntries values instead of the
// whole sample.
__host__ __device__ inline int group_keys(int nsb) { return nsb > 4 ? 16 : nsb > 2 ? 8 : nsb > 1 ? 4 : 2; }
static_assert(kSampleMaxBlocks * (kSampleBlockKeys / 16) <= kListEntries, "the group maxima fit the list");


// r-th largest (1 <= r <= number of values) of the ordered keys v[m] of the
// wavefront's lanes: bisection on the key with three probes per round, whose
// counts (each < 2^10, so 64 M < 1024) share one packed wavefront sum.
template <int M>
__device__ uint32_t wave_rth_search(const uint32_t (&v)[M], uint32_t r) {
  static_assert(64 * M < 1024, "counts fit 10-bit fields");
  auto cnt = [&](uint32_t t) {
    uint32_t c = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) c += v[m] >= t ? 1u : 0u;
    return c;
  };
  // invariant: count(>= lo) >= r > count(>= hi); no ordered score is 2^32 - 1
  uint32_t lo = 0u, hi = 0xffffffffu;
  while (hi - lo > 1u) {
    const uint32_t step = max(1u, (hi - lo) / 4u);
    const uint32_t t1 = min(lo + step, hi - 1u);
    const uint32_t t2 = min(t1 + step, hi - 1u);
    const uint32_t t3 = min(t2 + step, hi - 1u);
    uint32_t packed = cnt(t1) | (cnt(t2) << 10) | (cnt(t3) << 20);
    packed = read_lane(wave_incl_sum(packed), 63);
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

// The r-th largest (1 <= r <= 64) of the wavefront's ordered keys v[m]
// (m < M; 0 marks an absent key).  The r-th largest per-lane maximum L has
// at least r keys at or above it; when at most 64 do, they are compacted one
// per lane through `scratch` (64 words of LDS private to the wavefront) and
// sorted, otherwise a search finds the rank directly.
template <int M>
__device__ uint32_t wave_rth_largest(const uint32_t (&v)[M], uint32_t r, uint32_t* scratch) {
  const int lane = threadIdx.x & 63;
  uint32_t mx = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m) mx = max(mx, v[m]);
  const uint32_t L = read_lane(wave_sort_desc(mx), static_cast<int>(r) - 1);
  uint32_t c = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) c += static_cast<uint32_t>(__popcll(__ballot(v[m] >= L)));
  if (c > 64u) return wave_rth_search<M>(v, r);   // uniform
  uint32_t base = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bool in = v[m] >= L;
    const uint64_t bal = __ballot(in);
    if (in) scratch[base + lanes_below(bal)] = v[m];
    base += static_cast<uint32_t>(__popcll(bal));
  }
  __builtin_amdgcn_wave_barrier();
  return read_lane(wave_sort_desc(static_cast<uint32_t>(lane) < c ? scratch[lane] : 0u), static_cast<int>(r) - 1);
}

// -------------------------------------------------------------------- main

// Per query: fixed-point weights V = round(W / sigma) with sigma = sum|W| /
// 2^30, split into four balanced base-256 digits (int8 limbs), so the int8
// MFMA accumulates each limb exactly and the score is
// C + sigma * (l0 + 2^8 l1 + 2^16 l2 + 2^24 l3).  Rows of the A operand are
// (query g, limb) = 4g + limb; K slice G of block b covers union planes
// 64b + 16G .. 64b + 16G + 15, slice plane pl at byte pl.
// Fills T.A and T.sigma; wsum is LDS scratch.
template <int GQ>
__device__ void build_limbs(const UnionLds<GQ>& s, ChunkTable& T, double (&wsum)[4], int nblk) {
  const int t = threadIdx.x;
  const int P = nblk * kBlockPlanes;
  const int U = s.U;
  if (t < 64) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int p = t; p < U; p += 64)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] += fabs(static_cast<double>(s.w[p][g]));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const double v = wave_sum(acc[g]);
      if (t == 0) {
        wsum[g] = v;
        T.sigma[g] = static_cast<float>(v * 0x1p-30);
      }
    }
  }
  lds_barrier();
  for (int i = t; i < P * 4; i += blockDim.x) {
    const int tp = i >> 2, g = i & 3;   // table position, query
    const int p = union_plane_at(tp, U);
    const double ws = wsum[g];
    long long v = (ws > 0.0 && p >= 0) ? llrint(static_cast<double>(s.w[p][g]) * (0x1p30 / ws)) : 0ll;
    const int b = tp / kBlockPlanes, G = (tp % kBlockPlanes) / 16, byte = tp % 16;
    uint8_t* row = reinterpret_cast<uint8_t*>(&T.blk[b].A[G][0]);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const long long d = ((v + 128) & 255) - 128;   // balanced digit in [-128, 127]
      row[(4 * g + l) * 16 + byte] = static_cast<uint8_t>(static_cast<int8_t>(d));
      v = (v - d) >> 8;
    }
  }
  lds_barrier();
}

typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// Waits until this wave's loads of a ring stage have landed, then for every
// wave of the workgroup to get there (so the stage is complete and the stage
// read before it is no longer read by anyone).  VMEM operations complete in
// issue order, so with VM loads outstanding issued after the stage's own,
// the stage's loads are complete when at most VM remain.  Inline asm: the
// compiler, not knowing which LDS DMA an LDS read depends on, would wait
// for all of them, and a plain barrier would also wait for all loads.
template <int VM>
__device__ __forceinline__ void sync_stage() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(VM) : "memory");
}

// Reads this lane's B operand bytes of a complete ring stage (inline asm for
// the same reason; the block waits for its own reads).
//
// ds_read_b64_tr_b8 transposes bytes within each group of 16 lanes: lane j
// of the group receives, in byte m, byte j % 8 of the 8-byte row addressed by
// lane j / 8 + 2m of the group.  Lane (G, j) addresses plane 16G + 8k + j / 2
// (k = 0, 1) of the wave's key segment 2X + (j & 1) (X = 0, 1; a segment is
// 64 keys, two words), so it receives octet j % 8 of segment 2X + j / 8 for planes
// 16G + 8k .. + 7, one plane per byte: t[4X + 2k + h] holds planes
// 16G + 8k + 4h .. + 3 in bytes 0..3, bit e of each byte being key 8 (j % 8)
// + e of the segment.  The block also reads the lane's A operand (16 bytes
// at a_addr), which the compiler would otherwise fence the same way.
__device__ __forceinline__ void read_stage(uint32_t addr, uint32_t a_addr, uint32_t (&t)[4 * kWaveX], v4i& A) {
  // plane 16G + 8k + j / 2 sits in row 2G + k of DMA load j / 2 (128 bytes
  // per row), so k adds 128 bytes and X, two segments, 16
  if constexpr (kWaveX == 2) {
    v2u r0, r1, r2, r3;
    asm volatile(
        "ds_read_b128 %4, %6\n\t"
        "ds_read_b64_tr_b8 %0, %5\n\t"
        "ds_read_b64_tr_b8 %1, %5 offset:128\n\t"
        "ds_read_b64_tr_b8 %2, %5 offset:16\n\t"
        "ds_read_b64_tr_b8 %3, %5 offset:144\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(A)
        : "v"(addr), "v"(a_addr)
        : "memory");
    t[0] = r0.x;
    t[1] = r0.y;
    t[2] = r1.x;
    t[3] = r1.y;
    t[4] = r2.x;
    t[5] = r2.y;
    t[6] = r3.x;
    t[7] = r3.y;
  } else {
    v2u r0, r1;
    asm volatile(
        "ds_read_b128 %2, %4\n\t"
        "ds_read_b64_tr_b8 %0, %3\n\t"
        "ds_read_b64_tr_b8 %1, %3 offset:128\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(A)
        : "v"(addr), "v"(a_addr)
        : "memory");
    t[0] = r0.x;
    t[1] = r0.y;
    t[2] = r1.x;
    t[3] = r1.y;
  }
}

// One K block: two sets X of 16 columns, 8 MFMAs each.  For key e of a
// column's octet, masking t[4X + d] with bit e of every byte leaves, in byte
// e' of dword d, slice plane (4d + e')'s bit of the key times 2^e: the B
// operand column is the key's bits scaled by 2^e (as int8, -128 for e = 7),
// so acc[8X + e] holds the key's limb sums times that scale.  The first
// block of a tile starts from a zero accumulator.
template <bool FIRST>
__device__ __forceinline__ void mfma_block(const uint32_t (&t)[4 * kWaveX], v4i A, v4i (&acc)[kWaveKeys]) {
  const v4i zero = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kWaveKeys; ++i) {
    const uint32_t m = 0x01010101u << (i & 7);
    const int X = i >> 3;
    v4i bv;
    bv.x = static_cast<int>(t[4 * X + 0] & m);
    bv.y = static_cast<int>(t[4 * X + 1] & m);
    bv.z = static_cast<int>(t[4 * X + 2] & m);
    bv.w = static_cast<int>(t[4 * X + 3] & m);
    acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, bv, FIRST ? zero : acc[i], 0, 0, 0);
  }
}

// A half block (see half_last_block): the first transpose read of each key
// segment (rows 16G .. 16G + 7, union planes 8G .. 8G + 7) and the first 8
// bytes of the slice's A operand.
__device__ __forceinline__ void read_stage_half(uint32_t addr, uint32_t a_addr, uint32_t (&t)[2 * kWaveX],
                                                long& A) {
  if constexpr (kWaveX == 2) {
    v2u r0, r2;
    asm volatile(
        "ds_read_b64 %2, %4\n\t"
        "ds_read_b64_tr_b8 %0, %3\n\t"
        "ds_read_b64_tr_b8 %1, %3 offset:16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r2), "=&v"(A)
        : "v"(addr), "v"(a_addr)
        : "memory");
    t[0] = r0.x;
    t[1] = r0.y;
    t[2] = r2.x;
    t[3] = r2.y;
  } else {
    v2u r0;
    asm volatile(
        "ds_read_b64 %1, %3\n\t"
        "ds_read_b64_tr_b8 %0, %2\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(A)
        : "v"(addr), "v"(a_addr)
        : "memory");
    t[0] = r0.x;
    t[1] = r0.y;
  }
}

// A half block: K = 32 MFMAs, two masked dwords per key.
template <bool FIRST>
__device__ __forceinline__ void mfma_half(const uint32_t (&t)[2 * kWaveX], long A, v4i (&acc)[kWaveKeys]) {
  const v4i zero = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kWaveKeys; ++i) {
    const uint32_t m = 0x01010101u << (i & 7);
    const int X = i >> 3;
    const long bv = static_cast<long>((static_cast<uint64_t>(t[2 * X + 1] & m) << 32) | (t[2 * X] & m));
    acc[i] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, bv, FIRST ? zero : acc[i], 0, 0, 0);
  }
}

// Inclusive prefix sum over the 16 lanes of a DPP row.
__device__ __forceinline__ uint32_t row_incl_sum(uint32_t v) {
  v += dpp_u32<kDppRowShr + 1>(0u, v);
  v += dpp_u32<kDppRowShr + 2>(0u, v);
  v += dpp_u32<kDppRowShr + 4>(0u, v);
  v += dpp_u32<kDppRowShr + 8>(0u, v);
  return v;
}

// Scores tiles first_tile + i * tile_stride (i < ntiles) of KV head h with
// the chunk table T: run(epi) calls epi(tile, acc) for each, where acc[8X + e]
// holds, for lane (G, col), query G's limb sums of key 8X + e of the lane's
// column (see the epilogues).  Plane words stream through the LDS ring by
// DMA, kMainStages - 1 (tile, block) steps ahead; prologue() issues the first
// of those loads and needs only T.U and T.rowoff, so the caller may still be
// building the rest of T.  All waves of the workgroup make the same calls
// (run contains barriers).
struct TileScanner {
  const ScanArgs& a;
  const ChunkTable& T;
  uint32_t (*ring)[kStageDwords];
  int first_tile, tile_stride, ntiles;
  int nblk, wave, lane, col, G, nsteps;
  bool half;   // the last block is a half block (uniform)
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t dma_lane_off, ring_lane, a_lane;
  int it_tile, it_b = 0, it_slot = 0, issued = 0;   // next step to load (uniform)

  __device__ TileScanner(const ScanArgs& a_, const ChunkTable& T_, uint32_t (&ring_)[kMainStages][kStageDwords], int h,
                         int first_tile_, int tile_stride_, int ntiles_)
      : a(a_), T(T_), ring(ring_), first_tile(first_tile_), tile_stride(tile_stride_), ntiles(ntiles_) {
    nblk = nblocks_of(T.U);
    half = half_last_block(T.U);
    wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    lane = threadIdx.x & 63;
    col = lane & 15;
    G = lane >> 4;
    nsteps = max(0, ntiles) * nblk;   // (tile, block) steps
    it_tile = first_tile;
    // Loads.  DMA load q = kDmaPerWave wave + j of a stage, lane l: row
    // l >> 3 holds plane q + 8 (l >> 3) of the block, bytes 16 (l & 7) .. + 15
    // of the tile's 128.  (The eight planes a transpose read gathers then sit
    // in eight different loads, whose padding spreads them over the banks.)
    // The buffer's size bounds the reads: words past the head's last plane
    // row read as zero (past a row's end they read the next row; such keys
    // are masked out).
    const char* head = reinterpret_cast<const char*>(a.planes + int64_t(h) * kD * kPlanes * a.ldw);
    const int64_t head_bytes = int64_t(kD) * kPlanes * a.ldw * 4;
    const uint32_t nrec = head_bytes > int64_t(0xffffffff) ? 0xffffffffu : static_cast<uint32_t>(head_bytes);
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(head), static_cast<short>(0),
                                             static_cast<int>(nrec), 0x00020000);
    dma_lane_off = 16u * static_cast<uint32_t>(lane & 7);
    // transpose-read address of lane (G, col): plane 16G + col / 2 (row 2G
    // of DMA load col / 2) of the wave's segment col & 1
    ring_lane = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[0][0])) +
                static_cast<uint32_t>((col >> 1) * kDmaDwords + 2 * G * kTileWords + wave * kWaveWords) * 4u +
                8u * static_cast<uint32_t>(col & 1);
    a_lane = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&T.blk[0].A[G][col]));
  }

  // Plane words are read once per call: the loads carry the non-temporal
  // cache policy (streamed through L2 and the Infinity Cache instead of
  // displacing other lines), measured 42.7 -> 40.5 us for the main kernel.
  static constexpr int kCpolNt = 2;

  __device__ void issue() {
    if (issued < nsteps) {
      const uint32_t woff = static_cast<uint32_t>(it_tile * kTileWords) * 4u;
#pragma unroll
      for (int j = 0; j < kDmaPerWave; ++j) {
        const int q = kDmaPerWave * wave + j;
        const uint32_t vo = T.blk[it_b].rowoff[q + 8 * (lane >> 3)] + dma_lane_off + woff;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, &ring[it_slot][q * kDmaDwords], 16, vo, 0, 0, kCpolNt);
      }
      ++issued;
      if (++it_b == nblk) {
        it_b = 0;
        it_tile += tile_stride;
      }
      it_slot = it_slot + 1 == kMainStages ? 0 : it_slot + 1;
    }
  }

  __device__ void prologue() {
#pragma unroll
    for (int i = 0; i < kMainStages - 1; ++i) issue();
  }

  template <class Epi>
  __device__ void run(Epi&& epi) {
    int step_i = 0, slot = 0;
    for (int ti = 0, tile = first_tile; ti < ntiles; ++ti, tile += tile_stride) {
      // Issue priority falls over the last tiles of the run, one level per
      // a.ramp_step tiles, from 3 down to 0 for the last ones.  The
      // workgroups sharing a CU start together; with equal priority the
      // oldest wins arbitration and the youngest ends up scanning alone at
      // the end, at a fraction of the CU's throughput.  Falling priority
      // lets the ones behind catch up, so they finish close together.
      // Steps of 2 tiles from 3: many sessions (two generations of 8-tile
      // runs) 71.4-73.6 against 74.2-75.1 us with steps of 1 from 2; the
      // 1M-key step 39.8-40.4 against 40.0-40.9 us with steps of 2 from 2
      // and about 0.5 us more with steps of 1 from 2.
      {
        const int left = ntiles - 1 - ti;   // uniform
        if (left >= 3 * a.ramp_step) {
          __builtin_amdgcn_s_setprio(3);
        } else if (left >= 2 * a.ramp_step) {
          __builtin_amdgcn_s_setprio(2);
        } else if (left >= a.ramp_step) {
          __builtin_amdgcn_s_setprio(1);
        } else {
          __builtin_amdgcn_s_setprio(0);
        }
      }
      v4i acc[kWaveKeys];
      // the stage of step b is ready to read at (LDS byte address) addr and
      // its A operand at a_addr; the last steps have fewer loads behind them
      // and wait for all
      auto next_stage = [&](int b, uint32_t& addr, uint32_t& a_addr) {
        if (step_i + kMainStages - 2 < nsteps) {
          sync_stage<kDmaPerWave * (kMainStages - 2)>();
        } else {
          sync_stage<0>();
        }
        issue();   // into the slot every wave has finished reading
        addr = ring_lane + static_cast<uint32_t>(slot * kStageDwords) * 4u;
        a_addr = a_lane + static_cast<uint32_t>(b * sizeof(TableBlock));
        ++step_i;
        slot = slot + 1 == kMainStages ? 0 : slot + 1;
      };
      auto step = [&](auto first, int b) {
        uint32_t addr, a_addr;
        next_stage(b, addr, a_addr);
        uint32_t x[4 * kWaveX];
        v4i A;
        read_stage(addr, a_addr, x, A);
        mfma_block<decltype(first)::value>(x, A, acc);
      };
      const int nfull = half ? nblk - 1 : nblk;   // uniform
      step(std::true_type{}, 0);   // nblk >= 1: an empty union is one block of zero weights
      for (int b = 1; b < nfull; ++b) step(std::false_type{}, b);
      if (half) {   // uniform: the last block, never the first
        uint32_t addr, a_addr;
        next_stage(nblk - 1, addr, a_addr);
        uint32_t x[2 * kWaveX];
        long A;
        read_stage_half(addr, a_addr, x, A);
        mfma_half<false>(x, A, acc);
      }
      epi(tile, acc);
    }
  }
};

// Exact limb sums t of the 16 keys of a lane's column (see TileScanner): key
// 8X + e comes out scaled by 2^e (-128 for e = 7).  Unscaling limb j is a
// shift by 8j - e, exact (the sums are multiples of 2^e), and t = l0 + 2^8 l1
// + 2^16 l2 + 2^24 l3 is exact in wrapping int32 arithmetic because
// |t| < 2^31.  Keys with e = 7 give -t, which t_of undoes.
__device__ __forceinline__ void limb_sums(const v4i (&acc)[kWaveKeys], int (&tv)[kWaveKeys]) {
#pragma unroll
  for (int i = 0; i < kWaveKeys; ++i) {
    const int e = i & 7;
    // (empty asm: keeps the Horner form, which needs one op per limb)
    uint32_t z = (static_cast<uint32_t>(acc[i].w) << 8) + static_cast<uint32_t>(acc[i].z);
    asm("" : "+v"(z));
    uint32_t y = (z << 8) + static_cast<uint32_t>(acc[i].y);   // 2^e (l1 + 2^8 l2 + 2^16 l3)
    asm("" : "+v"(y));
    tv[i] = static_cast<int>((y << (8 - e)) + static_cast<uint32_t>(acc[i].x >> e));
  }
}

// b where the lane's bit of mask is set, else a (v_cndmask with a lane mask).
__device__ __forceinline__ int lane_select(int a, int b, uint64_t mask) {
  int r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
  return r;
}

// First key of the 8 keys 8X .. 8X + 7 of lane (G, col)'s column in a tile
// (the wave's segments are 64 keys; X picks the second pair of segments).
__device__ __forceinline__ int64_t column_key(int tile, int wave, int col, int X) {
  return (int64_t(tile) * kTileWords + wave * kWaveWords) * 32 + (col >> 3) * 64 + 8 * (col & 7) + 128 * X;
}

// kMainWgPerCu workgroups share a CU's 160 KB of LDS.  Beside its ring a
// main workgroup holds the chunk table and its candidate buffers in one
// arena (the small arrays fit in the 512 bytes left over): the buffers take
// what the table's blocks past the union leave, so a small union leaves
// room for more candidates per wave and query before they spill to the
// global list (2.7 times kWaveCand with three blocks).
constexpr int kMainArenaBytes =
    (160 * 1024 / kMainWgPerCu - static_cast<int>(sizeof(uint32_t)) * kMainStages * kStageDwords - 512) / 16 * 16;
static_assert(static_cast<int>(sizeof(ChunkTable) + sizeof(uint2) * kMainWaves * 4 * kWaveCand) <= kMainArenaBytes,
              "main-kernel LDS fits kMainWgPerCu workgroups per CU");

// (the second launch bound is the minimum number of wavefronts per SIMD)
template <int GQ>
__global__ __launch_bounds__(kMainThreads, kMainWgPerCu * kMainWaves / 4) void scan_main_kernel(ScanArgs a) {
  __shared__ __align__(16) uint32_t arena[kMainArenaBytes / 4];   // chunk table, then candidate buffers
  __shared__ uint32_t ring[kMainStages][kStageDwords];
  __shared__ uint32_t wkept[kMainWaves][4];
  __shared__ uint32_t wbase_s[kMainWaves][4];
  __shared__ float theta_s[4];
  __shared__ uint32_t full_s[4];   // the query's global list has overflowed (seen by this workgroup)
  // 1-D grid over the C (head, query chunk) pairs of the launch and their
  // a.main_wgs workgroups each: chunk cy, its workgroup cx.  Interleaved
  // (workgroup i scans chunk i % C) with one generation of resident
  // workgroups: each chunk's workgroups then sit in every stretch of the
  // launch order, and the CUs' workgroup slots, filled in that order, each
  // hold one chunk (measured on the 1M-key step: main kernel 41.2 -> 40.0
  // us).  One chunk after another with several generations: interleaved,
  // the 128-head shape ran 3.5 us slower (each generation then reads the
  // same narrow band of every head's plane rows).
  const int nchunk = static_cast<int>(gridDim.x) / a.main_wgs;
  const int bi = static_cast<int>(blockIdx.x);
  const int cy = a.interleave ? bi % nchunk : bi / a.main_wgs;
  const int cx = a.interleave ? bi / nchunk : bi % a.main_wgs;
  ChunkTable& T = *reinterpret_cast<ChunkTable*>(arena);
  const int h = cy / a.cph;
  const int q0 = h * a.group + a.qoff + (cy % a.cph) * kQueryChunk;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  // With per-block lists, wavefront g selects theta of query q0 + g itself
  // (every workgroup of the chunk gets the same value): its lanes load entry
  // `lane` of each sampled block's list together with the table.
  constexpr int kLv = kListEntries / 64;
  uint32_t lv[kLv];
  if (a.top_lists && wave < GQ) {   // uniform
    const uint32_t* row = reinterpret_cast<const uint32_t*>(a.sample) + int64_t(q0 + wave) * kSampleMaxKeys;
    const int entries = a.nsb * (kSampleBlockKeys / group_keys(a.nsb));
#pragma unroll
    for (int m = 0; m < kLv; ++m) lv[m] = m * 64 + lane < entries ? row[m * 64 + lane] : 0u;
  }
  {
    // (read unconditionally, with the table, and used only without lists)
    const float theta_in = a.theta[q0 + min(static_cast<int>(threadIdx.x) & 3, GQ - 1)];
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.tables) +
                                                      size_t(chunk_index(a, cy)) * kChunkTableBytes);
    uint4* dst = reinterpret_cast<uint4*>(&T);
    // all of a thread's loads issue before any store (a loop would wait for
    // each load in turn); indexes past the table copy its last piece again
    constexpr int kPieces = static_cast<int>(sizeof(ChunkTable) / 16);
    constexpr int kPer = (kPieces + kMainThreads - 1) / kMainThreads;
    uint4 piece[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) piece[r] = src[min(static_cast<int>(threadIdx.x) + r * kMainThreads, kPieces - 1)];
#pragma unroll
    for (int r = 0; r < kPer; ++r) dst[min(static_cast<int>(threadIdx.x) + r * kMainThreads, kPieces - 1)] = piece[r];
    // (every thread stores, the same value per slot: a store under a branch
    // would pull the load into it)
    theta_s[threadIdx.x & 3] = (a.top_lists || static_cast<int>(threadIdx.x & 3) >= GQ) ? 0.0f : theta_in;
    full_s[threadIdx.x & 3] = 0u;
  }
  __syncthreads();
  // candidate buffers: cap entries per (wave, query) behind the union's blocks
  const int cand_pairs = (kTableHeadBytes + nblocks_of(T.U) * static_cast<int>(sizeof(TableBlock))) / 8;   // uniform
  const uint32_t cap = static_cast<uint32_t>((kMainArenaBytes / 8 - cand_pairs) / (kMainWaves * 4));
  uint2* cbuf = reinterpret_cast<uint2*>(arena) + cand_pairs;   // [wave][query][cap]
  const int64_t nh = head_length(a.lengths, h, a.n);
  const int head_tiles = static_cast<int>(((nh + 31) / 32 + kTileWords - 1) / kTileWords);
  const int tile_begin = cx * a.tiles_per_wg;
  const int tile_end = min(min(a.tiles, head_tiles), tile_begin + a.tiles_per_wg);
  TileScanner scanner(a, T, ring, h, tile_begin, 1, tile_end - tile_begin);
  scanner.prologue();   // the first plane loads are in flight during the selection
  // The selection runs at the top issue priority: a workgroup that starts
  // it after its CU's other workgroups have begun scanning would otherwise
  // wait behind their VALU work (which drops below it after their first
  // tiles).
  __builtin_amdgcn_s_setprio(3);
  if (a.top_lists) {   // uniform
    if (wave < GQ) {
      const float th = ordered_to_float(
          wave_rth_largest<kLv>(lv, static_cast<uint32_t>(a.rsel), reinterpret_cast<uint32_t*>(cbuf + wave * 4 * cap)));
      if (lane == 0) theta_s[wave] = th;   // (workgroup 0 stores it at the end)
    }
    lds_barrier();
  }

  const int col = lane & 15;            // MFMA column: octet col & 7 of key segments 2X + (col >> 3)
  const int G = lane >> 4;              // K slice; in the result, the query of the lane
  const bool qvalid = G < GQ;
  // The filter runs on the exact integer limb sum t (|t| <= 2^30 (1 + eps);
  // score = fma(float(t), sigma, C)): t >= theta_i is a necessary condition
  // for score >= theta.  The margins cover the roundings of float(t) (at most
  // 64), of the fma and of this set-up (done in fp64), so every key scoring
  // >= theta is a candidate, plus possibly a few just below it; the merge
  // checks that the k-th candidate scores >= theta.
  int theta_i;
  {
    const float sigma = T.sigma[G], Cq = T.C[G], theta = theta_s[G];
    double tt;
    if (sigma > 0.0f) {
      const double slack = (fabs(static_cast<double>(theta)) + fabs(static_cast<double>(Cq))) * 0x1p-20;
      tt = (static_cast<double>(theta) - static_cast<double>(Cq) - slack) / static_cast<double>(sigma) - 65.0;
    } else {
      tt = Cq >= theta ? -INFINITY : INFINITY;   // every score equals C
    }
    theta_i = tt <= -0x1p31 ? INT_MIN : tt >= 0x1p31 ? INT_MAX : static_cast<int>(ceil(tt));
  }

  uint32_t wc0 = 0, wc1 = 0, wc2 = 0, wc3 = 0;   // this wave's candidates per query so far (uniform)
  scanner.run([&](int tile, const v4i (&acc)[kWaveKeys]) {
    const int64_t key0 = column_key(tile, wave, col, 0);
    const int64_t key1 = kWaveX == 2 ? column_key(tile, wave, col, 1) : key0;
    auto key_of = [&](int i) { return (i < 8 ? key0 : key1) + (i & 7); };
    // keys of the lane that count: only the head's last tile holds keys past
    // its end, so the others skip the range clamps
    uint32_t vmask = qvalid ? (1u << kWaveKeys) - 1u : 0u;
    if ((int64_t(tile) + 1) * kTileWords * 32 > nh) {   // uniform
      const int nv0 = static_cast<int>(max<int64_t>(0, min<int64_t>(8, nh - key0)));
      const int nv1 = kWaveX == 2 ? static_cast<int>(max<int64_t>(0, min<int64_t>(8, nh - key1))) : 0;
      vmask &= ((1u << nv0) - 1u) | (((1u << nv1) - 1u) << 8);
    }
    int tv[kWaveKeys];
    limb_sums(acc, tv);
    auto t_of = [&](int i) { return (i & 7) == 7 ? -tv[i] : tv[i]; };
    // (scale and offset re-read from LDS: only candidates need them)
    auto score_of = [&](int i) { return fmaf(static_cast<float>(t_of(i)), T.sigma[G], T.C[G]); };
    if (a.all_scores) {
#pragma unroll
      for (int i = 0; i < kWaveKeys; ++i)
        if ((vmask >> i) & 1u) a.all_scores[int64_t(q0 + G) * a.n + key_of(i)] = score_of(i);
    }
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < kWaveKeys; ++i) bits |= t_of(i) >= theta_i ? (1u << i) : 0u;
    bits &= vmask;
    if (__ballot(bits != 0) == 0) return;   // uniform
    // Candidates go to this wave's LDS buffer of their query: a DPP row holds
    // one query (lanes 16G..16G+15) and a row prefix sum orders its lanes.
    // Slots past the buffer spill to the global list, reserved with one
    // global atomic per (wave, query).
    const uint32_t mine = __popc(bits);
    const uint32_t incl = row_incl_sum(mine);
    const uint32_t t0 = read_lane(incl, 15), t1 = read_lane(incl, 31);
    const uint32_t t2 = read_lane(incl, 47), t3 = read_lane(incl, 63);
    const uint32_t wave_off = G == 0 ? wc0 : G == 1 ? wc1 : G == 2 ? wc2 : wc3;
    wc0 += t0;
    wc1 += t1;
    wc2 += t2;
    wc3 += t3;
    const uint32_t slot0 = wave_off + incl - mine;
    const uint32_t spill = slot0 + mine > cap ? slot0 + mine - max(slot0, cap) : 0u;
    uint32_t gpos = 0;
    if (__ballot(spill != 0) != 0) {   // uniform
      // the last lane of each query's row reserves the row's spilled slots:
      // one atomic per query, all in flight together
      // Once a query's list has overflowed (count > kCandCap: the merge
      // rescues it) further slots are useless: no more atomics on its count,
      // and its candidates are not walked.
      const uint32_t sincl = row_incl_sum(spill);
      uint32_t gb = 0;
      if (col == 15 && qvalid && sincl != 0) {
        if (full_s[G]) {
          gb = 0x40000000u;
        } else {
          gb = atomicAdd(&a.count[q0 + G], sincl);
          if (gb + sincl > static_cast<uint32_t>(kCandCap)) full_s[G] = 1u;
        }
      }
      uint32_t rb = 0;
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const uint32_t b = read_lane(gb, 16 * g + 15);
        rb = G == g ? b : rb;
      }
      gpos = rb + sincl - spill;
    }
    if (bits != 0 && gpos < 0x40000000u) {
      // Lanes pass few keys: walk the set bits only.  The key's t is picked
      // from the registers by a select tree on the bits of its index (a
      // computed index into tv would move it to scratch).
      const float sig = T.sigma[G], cq = T.C[G];
      int tn[kWaveKeys];
#pragma unroll
      for (int i = 0; i < kWaveKeys; ++i) tn[i] = t_of(i);
      uint32_t slot_c = slot0;
      uint32_t rem = bits;
      while (rem != 0u) {
        const int i = __ffs(static_cast<int>(rem)) - 1;
        rem &= rem - 1u;
        // (lane-mask selects written out: as plain selects the compiler
        // would turn them back into an indexed array)
        const uint64_t m0 = __ballot((i & 1) != 0), m1 = __ballot((i & 2) != 0);
        const uint64_t m2 = __ballot((i & 4) != 0);
        int t8[8], t4[4], t2[2];
        if constexpr (kWaveKeys == 16) {
          const uint64_t m3 = __ballot((i & 8) != 0);
#pragma unroll
          for (int m = 0; m < 8; ++m) t8[m] = lane_select(tn[m], tn[m + 8], m3);
        } else {
#pragma unroll
          for (int m = 0; m < 8; ++m) t8[m] = tn[m];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) t4[m] = lane_select(t8[2 * m], t8[2 * m + 1], m0);
#pragma unroll
        for (int m = 0; m < 2; ++m) t2[m] = lane_select(t4[2 * m], t4[2 * m + 1], m1);
        const int t = lane_select(t2[0], t2[1], m2);
        const float sc = fmaf(static_cast<float>(t), sig, cq);
        const uint32_t key = static_cast<uint32_t>(((i & 8) ? key1 : key0) + (i & 7));
        const uint2 e = make_uint2(__float_as_uint(sc), key);
        if (slot_c < cap) {
          cbuf[(wave * 4 + G) * cap + slot_c] = e;
        } else {
          if (gpos < static_cast<uint32_t>(kCandCap)) a.cand[int64_t(q0 + G) * kCandCap + gpos] = e;
          ++gpos;
        }
        ++slot_c;
      }
    }
  });
  // flush: one global atomic per query reserves the buffered candidates'
  // slots, in wave order
  if (lane == 0) {
    wkept[wave][0] = min(wc0, cap);
    wkept[wave][1] = min(wc1, cap);
    wkept[wave][2] = min(wc2, cap);
    wkept[wave][3] = min(wc3, cap);
  }
  __syncthreads();
  if (threadIdx.x < GQ) {
    const int g = threadIdx.x;
    uint32_t total = 0;
#pragma unroll
    for (int v = 0; v < kMainWaves; ++v) total += wkept[v][g];
    uint32_t base = total ? atomicAdd(&a.count[q0 + g], total) : 0u;
#pragma unroll
    for (int v = 0; v < kMainWaves; ++v) {
      wbase_s[v][g] = base;
      base += wkept[v][g];
    }
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const uint32_t kept = wkept[wave][g], b0 = wbase_s[wave][g];
    for (uint32_t i = lane; i < kept; i += 64)
      if (b0 + i < static_cast<uint32_t>(kCandCap)) a.cand[int64_t(q0 + g) * kCandCap + b0 + i] = cbuf[(wave * 4 + g) * cap + i];
  }
  // the threshold of each query, for the merge
  if (a.top_lists && cx == 0 && static_cast<int>(threadIdx.x) < GQ) a.theta[q0 + threadIdx.x] = theta_s[threadIdx.x];
}

// ------------------------------------------------------------------ sample

// Workgroup = (sampled 1024-key block, KV head, query chunk): builds the
// chunk's table in LDS (workgroup 0 also stores it for the main kernel) and
// scores the block's keys exactly as the main kernel does.  With a.var set,
// wavefront g first computes the allocation of query q0 + g (workgroup 0
// also stores it in a.alloc_out).
template <int GQ>
__global__ __launch_bounds__(kMainThreads) void scan_sample_kernel(ScanArgs a) {
  __shared__ UnionLds<GQ> s;
  __shared__ ChunkTable T;
  __shared__ double wsum[4];
  __shared__ uint32_t ring[kMainStages][kStageDwords];
  __shared__ uint16_t s_alloc[4][kD / 2];
  const int h = blockIdx.y / a.cph;
  const int q0 = h * a.group + a.qoff + (blockIdx.y % a.cph) * kQueryChunk;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  UnionInputs in = load_union_inputs<GQ>(a, h, q0);   // in flight during the allocation
  // the main kernel's candidate counts start at 0 (on the path without
  // per-block lists the threshold kernel resets them), and so do the merge's
  // rescue counters
  if (a.top_lists && blockIdx.x == 0 && static_cast<int>(threadIdx.x) < GQ) a.count[q0 + threadIdx.x] = 0u;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    if (static_cast<int>(threadIdx.x) < kRescueSlots) a.rescue_done[threadIdx.x] = 0u;
    for (int i = threadIdx.x; i < kRescueSlots * kRescueHistBins; i += blockDim.x) a.rescue_hist[i] = 0u;
  }
  if (a.var) {   // uniform
    if (wave < GQ) {
      // (the ring is free until the plane loads start: 64 words per wavefront)
      const uint2 b = allocate_query_wave(a.q + int64_t(q0 + wave) * kD, a.var + int64_t(h) * kD, a.budget,
                                          &ring[0][64 * wave]);
      const uint16_t pair = static_cast<uint16_t>(b.x | (b.y << 8));
      s_alloc[wave][lane] = pair;
    }
    __syncthreads();
    // (read here, from the LDS array itself: through a pointer that may also
    // name global memory they would be flat loads, each waited for alone)
    if (threadIdx.x < kD) {
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const uint16_t pair = s_alloc[g][threadIdx.x >> 1];
        in.b4 |= static_cast<uint32_t>((pair >> (8 * (threadIdx.x & 1))) & 255u) << (8 * g);
      }
    }
  }
  build_union<GQ>(a, in, s);
  table_rows<GQ>(s, T);
  __syncthreads();
  const int col = lane & 15;
  const int G = lane >> 4;
  const int sbi = blockIdx.x;
  const int64_t nh = head_length(a.lengths, h, a.n);
  int stride = a.sample_stride;
  if (a.lengths) {   // uniform
    int svalid_unused = 0;
    stride = ragged_sample(nh, a.nsb, svalid_unused);
  }
  const int tile = sbi * stride;   // a sampled block is one tile
  TileScanner sc(a, T, ring, h, tile, 0, 1);
  sc.prologue();   // the block's plane words load while the limbs are built
  table_limbs<GQ>(s, T, wsum);
  sc.run([&](int tile_, const v4i (&acc)[kWaveKeys]) {
    if (G >= GQ) return;
    int tv[kWaveKeys];
    limb_sums(acc, tv);
    const float sigma = T.sigma[G], Cq = T.C[G];
    uint32_t ok[kWaveKeys];
#pragma unroll
    for (int i = 0; i < kWaveKeys; ++i) {
      const int64_t key = column_key(tile_, wave, col, i >> 3) + (i & 7);
      const int t = (i & 7) == 7 ? -tv[i] : tv[i];
      const float sc = fmaf(static_cast<float>(t), sigma, Cq);
      const int local = static_cast<int>(key - int64_t(tile_) * kTileWords * 32);
      const float score = key < nh ? sc : -INFINITY;
      ok[i] = float_to_ordered(score);
      if (!a.top_lists) a.sample[int64_t(q0 + G) * kSampleMaxKeys + sbi * kSampleBlockKeys + local] = score;
    }
    if (a.top_lists) {
      // maxima of the lane's keys in groups of 2, 4, 8 and 16 (the last
      // across two lanes when a lane scores 8 keys); the group size is
      // uniform
      const int gs = group_keys(a.nsb);
      uint32_t* list = reinterpret_cast<uint32_t*>(a.sample) + int64_t(q0 + G) * kSampleMaxKeys +
                       sbi * (kSampleBlockKeys / gs);
      uint32_t m2[kWaveKeys / 2], m4[kWaveKeys / 4], m8[kWaveKeys / 8];
#pragma unroll
      for (int g = 0; g < kWaveKeys / 2; ++g) m2[g] = max(ok[2 * g], ok[2 * g + 1]);
#pragma unroll
      for (int g = 0; g < kWaveKeys / 4; ++g) m4[g] = max(m2[2 * g], m2[2 * g + 1]);
#pragma unroll
      for (int g = 0; g < kWaveKeys / 8; ++g) m8[g] = max(m4[2 * g], m4[2 * g + 1]);
      const int lane_slot = wave * 16 + col;   // the lane's place among the block's lanes
      if (gs == 2) {
#pragma unroll
        for (int g = 0; g < kWaveKeys / 2; ++g) list[lane_slot * (kWaveKeys / 2) + g] = m2[g];
      } else if (gs == 4) {
#pragma unroll
        for (int g = 0; g < kWaveKeys / 4; ++g) list[lane_slot * (kWaveKeys / 4) + g] = m4[g];
      } else if (gs == 8) {
#pragma unroll
        for (int g = 0; g < kWaveKeys / 8; ++g) list[lane_slot * (kWaveKeys / 8) + g] = m8[g];
      } else if constexpr (kWaveKeys == 16) {
        list[lane_slot] = max(m8[0], m8[1]);
      } else {
        const uint32_t m16 = max(m8[0], dpp_u32<kDppXor1>(m8[0], m8[0]));
        if ((col & 1) == 0) list[wave * 8 + (col >> 1)] = m16;
      }
    }
  });
  // the chunk's workgroups store a share of its table each, and workgroup 0
  // the allocations, last
  store_table(a, T, blockIdx.x, gridDim.x);
  if (blockIdx.x == 0 && a.var && wave < GQ)
    *reinterpret_cast<uint16_t*>(a.alloc_out + int64_t(q0 + wave) * kD + 2 * lane) = s_alloc[wave][lane];
}

// ------------------------------------------------------------------- merge

// The fast merge path keeps at most k - 1 + kBucketMax keys at the front of
// the sort buffer; its digit tables live behind them.
constexpr int kFastKept = 8192;
// Workgroups per query in the merge (up to kMergeSplit, fewer with many
// queries: each repeats the load, histogram and scan): workgroup w places
// only the output ranks [w k / W, (w + 1) k / W); the general and fallback
// paths run in workgroup 0 alone.
constexpr int kMergeSplit = 4;
static_assert(kMaxK - 1 + kBucketMax <= kFastKept, "kept keys stay in front of the digit tables");
static_assert(kFastKept * 8 + sizeof(DigitLds) <= kCandCap * 8, "digit tables fit in the sort buffer");

__device__ inline unsigned long long sort_key(uint32_t ordered, uint32_t idx) {
  return (static_cast<unsigned long long>(ordered) << 32) | static_cast<uint32_t>(~idx);
}

// Descending bitonic sort of N = kSelectThreads * E 64-bit keys, held E per
// thread in blocked order (thread t holds elements tE .. tE+E-1).  A
// compare-exchange at stride s runs in registers when s < E, between the
// lanes of a wavefront (ds_bpermute) when s < 64E, and through LDS (buf, N
// keys) otherwise, where consecutive large strides of one merge share a
// single write-back of the registers.
template <int E>
__device__ void sort_regs_desc(unsigned long long (&x)[E], unsigned long long* buf) {
  constexpr unsigned N = kSelectThreads * E;
  const unsigned t = threadIdx.x;
  for (unsigned size = 2; size <= N; size <<= 1) {
    unsigned stride = size >> 1;
    if (stride >= 64u * E) {
#pragma unroll
      for (int e = 0; e < E; ++e) buf[t * E + e] = x[e];
      __syncthreads();
      for (; stride >= 64u * E; stride >>= 1) {
        for (unsigned r = t; r < N / 2; r += kSelectThreads) {
          const unsigned lo_i = 2 * r - (r & (stride - 1));
          const unsigned hi_i = lo_i + stride;
          const bool desc = (lo_i & size) == 0;
          const unsigned long long a = buf[lo_i], b = buf[hi_i];
          if ((a < b) == desc) {
            buf[lo_i] = b;
            buf[hi_i] = a;
          }
        }
        __syncthreads();
      }
      // each thread reads back only its own elements, which no other thread
      // writes before the next barrier
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = buf[t * E + e];
    }
    for (; stride >= static_cast<unsigned>(E); stride >>= 1) {
      const int m = static_cast<int>(stride / E);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const unsigned i = t * E + e;
        const unsigned long long y = __shfl_xor(x[e], m);
        const bool keep_max = ((i & size) == 0) == ((i & stride) == 0);
        x[e] = keep_max ? (x[e] > y ? x[e] : y) : (x[e] < y ? x[e] : y);
      }
    }
#pragma unroll
    for (int sr = E / 2; sr >= 1; sr >>= 1) {
      if (static_cast<unsigned>(sr) < size) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e & sr) continue;
          const unsigned i = t * E + e;
          const bool desc = (i & size) == 0;
          const unsigned long long a = x[e], b = x[e | sr];
          const unsigned long long hi = a > b ? a : b, lo = a > b ? b : a;
          x[e] = desc ? hi : lo;
          x[e | sr] = desc ? lo : hi;
        }
      }
    }
  }
}

// Sorts the first `kept` keys of buf (descending) and writes the first k;
// ranks at or past `kept` (a head holding fewer than k keys) get index -1
// and score -inf.  Needs kSelectThreads * E >= max(kept, k).
template <int E>
__device__ void sort_and_write(unsigned long long* buf, unsigned kept, int k, int q,
                               int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  unsigned long long x[E];
  const unsigned t = threadIdx.x;
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = t * E + e < kept ? buf[t * E + e] : 0ull;
  __syncthreads();
  sort_regs_desc<E>(x, buf);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const unsigned i = t * E + e;
    if (i < static_cast<unsigned>(k)) {
      const bool real = i < kept;
      out_idx[int64_t(q) * k + i] = real ? static_cast<int32_t>(~static_cast<uint32_t>(x[e])) : -1;
      out_score[int64_t(q) * k + i] = real ? ordered_to_float(static_cast<uint32_t>(x[e] >> 32)) : -INFINITY;
    }
  }
}

// What the merge needs to score keys of one query exactly as the main kernel
// does: the query's nonzero fixed-point plane weights V (recombined from the
// chunk table's int8 limbs), their rows, and the scale and offset.  The score
// of key i is fmaf(float(t), sigma, C) with t = sum V bit_p(i), an exact
// integer (wrapping int32 sums are exact because |t| < 2^31).
struct QueryPlan {
  uint32_t rowoff[kMaxUnion];   // byte offset of the plane row in the head
  int32_t V[kMaxUnion];
  uint32_t np;                  // planes with V != 0
  uint32_t tneg, tpos;          // sums of the negative and of the positive V: t lies in [tneg, tpos]
  float sigma, C;
};
// The plan sits at the end of the merge's sort buffer, behind the kept keys
// and the digit tables.
constexpr int kPlanSlots = static_cast<int>((sizeof(QueryPlan) + 7) / 8);
static_assert(kFastKept + (sizeof(DigitLds) + 7) / 8 + kPlanSlots <= kCandCap, "the plan fits behind the digit tables");
__device__ inline QueryPlan& plan_in(unsigned long long* keys) {
  return *reinterpret_cast<QueryPlan*>(keys + kCandCap - kPlanSlots);
}

// An 11-bit digit of the ordered scores of one query, placed below the bits
// that every possible score shares (all scores lie between the scores of
// t = tneg and t = tpos): digit(o) = (o >> shift) & mask, and bucket b holds
// the scores from common | (b << shift) up.
struct PlanDigit {
  uint32_t shift, mask, common;
};
__device__ inline PlanDigit plan_digit(const QueryPlan& P) {
  const uint32_t o_lo = float_to_ordered(fmaf(static_cast<float>(static_cast<int32_t>(P.tneg)), P.sigma, P.C));
  const uint32_t o_hi = float_to_ordered(fmaf(static_cast<float>(static_cast<int32_t>(P.tpos)), P.sigma, P.C));
  const uint32_t diff = o_lo ^ o_hi;
  const int hi = diff ? 32 - __clz(diff) : 0;   // bits >= hi are common
  const int width = min(kDigitBits, hi), shift = hi - width;
  PlanDigit d;
  d.shift = static_cast<uint32_t>(shift);
  d.mask = (1u << width) - 1u;
  d.common = hi >= 32 ? 0u : (o_lo & ~((1u << hi) - 1u));
  return d;
}

// Whole workgroup (blockDim.x >= kMaxUnion); ends with a barrier.
__device__ void load_plan(const ScanArgs& a, int q, QueryPlan& P) {
  const int h = q / a.group, r = q % a.group, g = r % kQueryChunk;
  const ChunkTable& T = *reinterpret_cast<const ChunkTable*>(
      static_cast<const char*>(a.tables) + (size_t(h) * a.chunks_per_head + r / kQueryChunk) * kChunkTableBytes);
  const int t = threadIdx.x;
  if (t == 0) {
    P.np = 0u;
    P.tneg = 0u;
    P.tpos = 0u;
  }
  __syncthreads();
  const int U = T.U;
  if (t < U) {
    const int tp = table_pos_of(t, U);
    const int b = tp / kBlockPlanes, G = (tp % kBlockPlanes) / 16, byte = tp % 16;
    const int8_t* row = reinterpret_cast<const int8_t*>(&T.blk[b].A[G][0]);
    uint32_t v = 0;
#pragma unroll
    for (int l = 3; l >= 0; --l) v = (v << 8) + static_cast<uint32_t>(static_cast<int32_t>(row[(4 * g + l) * 16 + byte]));
    if (v != 0u) {
      const uint32_t slot = atomicAdd(&P.np, 1u);
      P.rowoff[slot] = T.blk[b].rowoff[tp % kBlockPlanes];
      P.V[slot] = static_cast<int32_t>(v);
      // (wrapping sums of one sign, exact: they stay below 2^31 in magnitude)
      atomicAdd(static_cast<int32_t>(v) < 0 ? &P.tneg : &P.tpos, v);
    }
  }
  if (t == 0) {
    P.sigma = T.sigma[g];
    P.C = T.C[g];
  }
  __syncthreads();
}

// Ordered score of key i of the head whose planes start at head_planes.
__device__ inline uint32_t plan_score(const uint32_t* head_planes, const QueryPlan& P, int64_t i) {
  const uint32_t* base = head_planes + (i >> 5);
  const uint32_t sh = static_cast<uint32_t>(i & 31);
  uint32_t t = 0;
  const uint32_t np = P.np;
#pragma unroll 8
  for (uint32_t p = 0; p < np; ++p) {
    const uint32_t w = base[P.rowoff[p] >> 2];
    t += ((w >> sh) & 1u) ? static_cast<uint32_t>(P.V[p]) : 0u;
  }
  return float_to_ordered(fmaf(static_cast<float>(static_cast<int32_t>(t)), P.sigma, P.C));
}

// Ordered scores of keys i0 + j * kSelectThreads (j < PT, those below i_end;
// slots past it get 0 and no load), all PT words of a plane loaded together.
template <int PT>
__device__ inline void plan_scores(const uint32_t* head_planes, const QueryPlan& P, int64_t i0, int64_t i_end,
                                   uint32_t (&v)[PT]) {
  static_assert(kSelectThreads % 32 == 0, "slots of a thread share the bit position");
  const uint32_t sh = static_cast<uint32_t>(i0 & 31);
  const int64_t last_word = (i_end - 1) >> 5;   // i_end > i0 >= 0 for any valid slot
  uint32_t wo[PT], t[PT];
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    wo[j] = static_cast<uint32_t>(min<int64_t>((i0 + int64_t(j) * kSelectThreads) >> 5, max<int64_t>(last_word, 0)));
    t[j] = 0u;
  }
  const uint32_t np = P.np;
  for (uint32_t p = 0; p < np; ++p) {
    const uint32_t* row = head_planes + (P.rowoff[p] >> 2);
    const uint32_t V = static_cast<uint32_t>(P.V[p]);
    uint32_t x[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) x[j] = row[wo[j]];
#pragma unroll
    for (int j = 0; j < PT; ++j) t[j] += ((x[j] >> sh) & 1u) ? V : 0u;
  }
#pragma unroll
  for (int j = 0; j < PT; ++j)
    v[j] = i0 + int64_t(j) * kSelectThreads < i_end
               ? float_to_ordered(fmaf(static_cast<float>(static_cast<int32_t>(t[j])), P.sigma, P.C))
               : 0u;
}

// Sum over the workgroup's kSelectThreads threads, returned to all.
__device__ inline uint32_t block_sum(uint32_t v, uint32_t* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = read_lane(wave_incl_sum(v), 63);
  if (lane == 0) s_wave[wave] = v;
  __syncthreads();
  uint32_t tot = 0;
  for (int wv = 0; wv < kSelectWaves; ++wv) tot += s_wave[wv];
  __syncthreads();
  return tot;
}

// Of `count` entries (ordered score, key index) read by get(i), keeps in
// keys[] every entry above kth (n_gt of them) and the first need_eq entries
// equal to kth in position order (the callers' positions follow key order, so
// ties go to the lower key index).  Positions are read CH per thread at a
// time, so their loads are in flight together.  Whole workgroup of
// kSelectThreads; s_count and s_wave are LDS scratch.
template <int CH, class Get>
__device__ void collect_given(int64_t count, uint32_t kth, uint32_t need_eq, uint32_t n_gt, Get get,
                              unsigned long long* keys, uint32_t* s_count, uint32_t* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_count[0] = 0;
  __syncthreads();
  uint32_t eq_taken = 0;
  for (int64_t base = 0; base < count; base += int64_t(CH) * kSelectThreads) {
    uint2 e[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t i = base + int64_t(c) * kSelectThreads + tid;
      e[c] = i < count ? get(i) : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t i = base + int64_t(c) * kSelectThreads + tid;
      const bool valid = i < count;
      const bool gt = valid && e[c].x > kth;
      const bool eq = valid && e[c].x == kth;
      if (gt) {
        const uint32_t slot = atomicAdd(&s_count[0], 1u);
        keys[slot] = sort_key(e[c].x, e[c].y);
      }
      const uint64_t bal = __ballot(eq);
      if (lane == 0) s_wave[wave] = static_cast<uint32_t>(__popcll(bal));
      __syncthreads();
      uint32_t before = 0, total = 0;
      for (int wv = 0; wv < kSelectWaves; ++wv) {
        const uint32_t cw = s_wave[wv];
        before += wv < wave ? cw : 0u;
        total += cw;
      }
      if (eq) {
        const uint32_t rank = eq_taken + before + static_cast<uint32_t>(lanes_below(bal));
        if (rank < need_eq) keys[n_gt + rank] = sort_key(e[c].x, e[c].y);
      }
      eq_taken += total;
      __syncthreads();
    }
    if (s_count[0] == n_gt && eq_taken >= need_eq) break;   // uniform: everything kept is found
  }
  __syncthreads();
}

// Exact top-keff of `count` entries read by get(i) (in increasing i within
// each of its select passes), ties to the lower position: the keff entries
// go to keys[0, keff).
template <class Get>
__device__ void exact_collect(int64_t count, int keff, Get get, unsigned long long* keys, SelectLds& L,
                              uint32_t* s_count, uint32_t* s_wave) {
  if (keff <= 0) return;   // uniform
  const uint2 sel = block_select_fn(count, static_cast<uint32_t>(keff), L, [&](int64_t i) { return get(i).x; });
  collect_given<1>(count, sel.x, sel.y, static_cast<uint32_t>(keff) - sel.y, get, keys, s_count, s_wave);
}

// Sorts keys[0, kept) and writes the first k outputs of query q.
__device__ void sort_write_any(unsigned long long* keys, unsigned kept, int k, int q, int32_t* __restrict__ out_idx,
                               float* __restrict__ out_score) {
  const unsigned span = max(kept, static_cast<unsigned>(k));
  if (span <= kSelectThreads) {
    sort_and_write<1>(keys, kept, k, q, out_idx, out_score);
  } else if (span <= 2 * kSelectThreads) {
    sort_and_write<2>(keys, kept, k, q, out_idx, out_score);
  } else if (span <= 4 * kSelectThreads) {
    sort_and_write<4>(keys, kept, k, q, out_idx, out_score);
  } else if (span <= 8 * kSelectThreads) {
    sort_and_write<8>(keys, kept, k, q, out_idx, out_score);
  } else {
    sort_and_write<16>(keys, kept, k, q, out_idx, out_score);
  }
}

// A query's candidate list missed when it holds fewer than k keys or
// overflowed.  Such a query is rescued by the rescue workgroups when its head
// fits their slices and it is among the first kRescueSlots such queries (in
// query order); otherwise workgroup 0 of its merge recomputes it alone.
__device__ inline bool list_missed(uint32_t cnt, int k) {
  return cnt < static_cast<uint32_t>(k) || cnt > static_cast<uint32_t>(kCandCap);
}
__device__ inline bool rescuable(const ScanArgs& a, int q) {
  return a.rescue_wgs > 0 &&
         head_length(a.lengths, q / a.group, a.n) <= int64_t(a.rescue_wgs) * kRescueSlice;
}

// Rescue slot of query q (-1: not rescued): counts the missed, rescuable
// queries before it.  Whole workgroup; uniform result.
__device__ int rescue_slot(const ScanArgs& a, int q, int k, uint32_t* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (!list_missed(a.count[q], k) || !rescuable(a, q)) return -1;
  uint32_t before = 0;
  for (int base = 0; base < q; base += kSelectThreads) {   // uniform
    const int i = base + tid;
    const bool m = i < q && list_missed(a.count[i], k) && rescuable(a, i);
    const uint64_t bal = __ballot(m);
    if (lane == 0) s_wave[wave] = static_cast<uint32_t>(__popcll(bal));
    __syncthreads();
    for (int wv = 0; wv < kSelectWaves; ++wv) before += s_wave[wv];
    __syncthreads();
  }
  return before < static_cast<uint32_t>(kRescueSlots) ? static_cast<int>(before) : -1;
}

// Scores of the slice keys s0 + tid + j * kSelectThreads (j < PT, those
// below s1; 0 for the rest) for a plan, with the slice's plane words staged
// in LDS (stage: `cap` words): a chunk of J slots at a time, all of the
// chunk's loads issued before any is used, so the slice costs a few memory
// round trips rather than one per plane.  Whole workgroup.
template <int PT>
__device__ void staged_scores(const uint32_t* head_planes, const QueryPlan& P, int64_t s0, int64_t s1,
                              uint32_t* stage, int cap, uint32_t (&v)[PT]) {
  const int tid = threadIdx.x;
  const int np = static_cast<int>(P.np);
  // J slots of 1024 keys span at most 32 J + 1 words per plane
  const int J = max(1, min(PT, (cap / max(np, 1) - 1) / 32));
  const int cw = 32 * J + 1;   // staged words per plane
#pragma unroll
  for (int j = 0; j < PT; ++j) v[j] = 0u;
  for (int j0 = 0; j0 < PT; j0 += J) {   // uniform
    const int64_t kb = s0 + int64_t(j0) * kSelectThreads;
    if (kb >= s1) break;
    const int64_t ke = min(s1, s0 + int64_t(j0 + J) * kSelectThreads);
    const int64_t wb = kb >> 5;
    const int nwc = static_cast<int>(((ke - 1) >> 5) - wb + 1);   // <= cw
    const int total = np * nwc;
    // stage: eight loads in flight per thread, then their stores
    for (int e0 = 0; e0 < total; e0 += 8 * kSelectThreads) {
      uint32_t x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kSelectThreads + tid;
        const int pp = e / nwc, w = e - pp * nwc;
        x[u] = e < total ? head_planes[(P.rowoff[pp] >> 2) + wb + w] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kSelectThreads + tid;
        const int pp = e / nwc, w = e - pp * nwc;
        if (e < total) stage[pp * cw + w] = x[u];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      if (j < j0 || j >= j0 + J) continue;   // uniform
      const int64_t i = s0 + tid + int64_t(j) * kSelectThreads;
      if (i < s1) {
        const int wl = static_cast<int>((i >> 5) - wb);
        const uint32_t sh = static_cast<uint32_t>(i & 31);
        uint32_t t = 0;
        for (int pp = 0; pp < np; ++pp)
          t += ((stage[pp * cw + wl] >> sh) & 1u) ? static_cast<uint32_t>(P.V[pp]) : 0u;
        v[j] = float_to_ordered(fmaf(static_cast<float>(static_cast<int32_t>(t)), P.sigma, P.C));
      }
    }
    __syncthreads();
  }
}

// One rescue workgroup: slice r of every rescued query.  Each slice's exact
// top-keff (keys in key order) goes to the query's rescue list, and its
// entries' digits (plan_digit) to the query's shared histogram; the workgroup
// that finishes the last slice of a query merges the lists and writes the
// query's output.  Memory order: each list, count and histogram update is
// released by an agent-scope fence before the slice counter's increment, and
// the last workgroup acquires them with a fence after it.
__device__ void rescue_role(const ScanArgs& a, int k, int r, int32_t* __restrict__ out_idx,
                            float* __restrict__ out_score, unsigned long long* keys, SelectLds& L,
                            uint32_t* s_count, uint32_t* s_wave, uint32_t* s_pref, int* s_list) {
  constexpr int PT = kRescueSlice / kSelectThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.rescue_wgs;
  // the rescued queries: the first kRescueSlots missed, rescuable ones
  int found = 0;
  for (int base = 0; base < a.num_q && found < kRescueSlots; base += kSelectThreads) {   // uniform
    const int i = base + tid;
    const bool m = i < a.num_q && list_missed(a.count[i], k) && rescuable(a, i);
    const uint64_t bal = __ballot(m);
    if (lane == 0) s_wave[wave] = static_cast<uint32_t>(__popcll(bal));
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int wv = 0; wv < kSelectWaves; ++wv) {
      before += wv < wave ? s_wave[wv] : 0u;
      total += s_wave[wv];
    }
    const uint32_t rank = static_cast<uint32_t>(found) + before + static_cast<uint32_t>(lanes_below(bal));
    if (m && rank < static_cast<uint32_t>(kRescueSlots)) s_list[rank] = i;
    found += static_cast<int>(total);
    __syncthreads();
  }
  found = min(found, kRescueSlots);
  QueryPlan& P = plan_in(keys);
  uint32_t* lhist = &L.hist[0][0];   // 2048 bins, while no select runs
  for (int slot = 0; slot < found; ++slot) {
    const int f = s_list[slot];
    load_plan(a, f, P);
    const PlanDigit dg = plan_digit(P);
    const int h = f / a.group;
    const int64_t nh = head_length(a.lengths, h, a.n);
    const int keff = static_cast<int>(min<int64_t>(k, nh));
    const int64_t s0 = int64_t(r) * nh / R, s1 = int64_t(r + 1) * nh / R;   // at most kRescueSlice keys
    const uint32_t* head_planes = a.planes + int64_t(h) * kD * kPlanes * a.ldw;
    uint32_t v[PT];
    staged_scores<PT>(head_planes, P, s0, s1, reinterpret_cast<uint32_t*>(keys), 2 * (kCandCap - kPlanSlots), v);
    uint32_t pm = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) pm |= s0 + tid + j * kSelectThreads < s1 ? (1u << j) : 0u;
    const int kk = static_cast<int>(min<int64_t>(keff, s1 - s0));
    uint32_t kth_slice = 0u;
    uint2* list = a.rescue + (size_t(slot) * R + r) * size_t(k);
    uint32_t* ghist = a.rescue_hist + size_t(slot) * kBins;
    if (kk > 0) {   // uniform
      const uint2 sel = block_select_regs<PT>(v, pm, static_cast<uint32_t>(kk), L);
      const uint32_t kth = sel.x, need_eq = sel.y;
      kth_slice = kth;
      for (int i = tid; i < kBins; i += kSelectThreads) lhist[i] = 0u;
      __syncthreads();
      // the slice's top-kk in key order: every entry above kth, and the
      // first need_eq equal to it
      uint32_t base = 0, eq_taken = 0;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const bool pres = (pm >> j) & 1u;
        const bool gt = pres && v[j] > kth, eq = pres && v[j] == kth;
        const uint64_t beq = __ballot(eq);
        if (lane == 0) s_wave[wave] = static_cast<uint32_t>(__popcll(beq));
        __syncthreads();
        uint32_t eq_before = 0, eq_total = 0;
        for (int wv = 0; wv < kSelectWaves; ++wv) {
          eq_before += wv < wave ? s_wave[wv] : 0u;
          eq_total += s_wave[wv];
        }
        const bool take = gt || (eq && eq_taken + eq_before + static_cast<uint32_t>(lanes_below(beq)) < need_eq);
        __syncthreads();
        const uint64_t btk = __ballot(take);
        if (lane == 0) s_wave[wave] = static_cast<uint32_t>(__popcll(btk));
        __syncthreads();
        uint32_t tk_before = 0, tk_total = 0;
        for (int wv = 0; wv < kSelectWaves; ++wv) {
          tk_before += wv < wave ? s_wave[wv] : 0u;
          tk_total += s_wave[wv];
        }
        if (take)
          list[base + tk_before + static_cast<uint32_t>(lanes_below(btk))] =
              make_uint2(v[j], static_cast<uint32_t>(s0 + tid + j * kSelectThreads));
        hist_add(lhist, take, (v[j] >> dg.shift) & dg.mask);
        base += tk_total;
        eq_taken += eq_total;
        __syncthreads();
      }
      for (int i = tid; i < kBins; i += kSelectThreads)
        if (lhist[i]) atomicAdd(&ghist[i], lhist[i]);
    }
    if (tid == 0) a.rescue_cnt[slot * R + r] = make_uint2(static_cast<uint32_t>(kk), kth_slice);
    __threadfence();
    __syncthreads();
    if (tid == 0) s_count[1] = atomicAdd(&a.rescue_done[slot], 1u);
    __syncthreads();
    const uint32_t done_before = s_count[1];
    __syncthreads();   // (s_count is written again below)
    if (done_before != static_cast<uint32_t>(R - 1)) continue;   // uniform: not the last slice
    __threadfence();
    // The last slice: merge the R lists (in slice order, so positions follow
    // key order).
    if (tid == 0) {
      uint32_t acc = 0, M = 0;
      for (int i = 0; i < R; ++i) {
        const uint2 c = a.rescue_cnt[slot * R + i];
        s_pref[i] = acc;
        acc += c.x;
        if (c.x == static_cast<uint32_t>(keff)) M = max(M, c.y);
      }
      s_pref[R] = acc;
      s_count[1] = M;
    }
    __syncthreads();
    const uint32_t total = s_pref[R], M = s_count[1];
    __syncthreads();
    const uint2* lists = a.rescue + size_t(slot) * R * size_t(k);
    // position -> entry: the slice from a per-thread cursor over the prefix
    // counts (a thread's positions rise within a pass; a lower position
    // starts a new pass)
    int cur = 0;
    int64_t last_i = -1;
    auto entry = [&](int64_t i) -> uint2 {
      if (i < last_i) cur = 0;
      last_i = i;
      while (s_pref[cur + 1] <= static_cast<uint32_t>(i)) ++cur;
      const v2u32 e = __builtin_nontemporal_load(
          reinterpret_cast<const v2u32*>(lists + size_t(cur) * k + (static_cast<uint32_t>(i) - s_pref[cur])));
      return make_uint2(e.x, e.y);
    };
    constexpr int CH = 8;
    if (keff > 0) {   // uniform
      // The histogram of all list entries gives the bucket holding the
      // keff-th largest; every entry from that bucket's lower edge up is
      // collected, when they fit, and sorted.
      DigitLds& D = *reinterpret_cast<DigitLds*>(keys + kFastKept);
      for (int i = tid; i < kBins; i += kSelectThreads) {
        const v2u32 hv = __builtin_nontemporal_load(reinterpret_cast<const v2u32*>(ghist) + i / 2);
        D.hist[i] = (i & 1) ? hv.y : hv.x;
      }
      if (tid == 0) D.big = 0u;
      __syncthreads();
      digit_scan(D, static_cast<uint32_t>(keff) - 1u);
      const uint32_t C = D.bstart + D.bcount;
      const uint32_t low = dg.common | (D.bstar << dg.shift);
      __syncthreads();
      if (C <= static_cast<uint32_t>(kFastKept)) {   // uniform
        if (tid == 0) s_count[0] = 0u;
        __syncthreads();
        for (int64_t b0 = 0; b0 < total; b0 += int64_t(CH) * kSelectThreads) {
          uint2 e[CH];
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            const int64_t i = b0 + int64_t(c) * kSelectThreads + tid;
            e[c] = i < total ? entry(i) : make_uint2(0u, 0u);
          }
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            const int64_t i = b0 + int64_t(c) * kSelectThreads + tid;
            if (i < total && e[c].x >= low) keys[atomicAdd(&s_count[0], 1u)] = sort_key(e[c].x, e[c].y);
          }
        }
        __syncthreads();
        sort_write_any(keys, C, k, f, out_idx, out_score);
        __syncthreads();
        continue;
      }
      if (dg.shift == 0u) {   // uniform
        // each bucket is a single score, so the keff-th largest is `low`
        // itself: every entry above it and the first ties in key order
        collect_given<CH>(total, low, static_cast<uint32_t>(keff) - D.bstart, D.bstart, entry, keys, s_count,
                          s_wave);
        sort_write_any(keys, static_cast<unsigned>(keff), k, f, out_idx, out_score);
        __syncthreads();
        continue;
      }
    }
    // Many entries share the bucket (ties): a slice that kept keff keys has
    // keff keys at or above its own keff-th score, so the keff-th largest is
    // at least the largest such score M.
    uint32_t my_gt = 0, my_eq = 0;
    for (int64_t b0 = 0; b0 < total; b0 += int64_t(CH) * kSelectThreads) {
      uint2 e[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int64_t i = b0 + int64_t(c) * kSelectThreads + tid;
        e[c] = i < total ? entry(i) : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const bool valid = b0 + int64_t(c) * kSelectThreads + tid < total;
        my_gt += (valid && e[c].x > M) ? 1u : 0u;
        my_eq += (valid && e[c].x == M) ? 1u : 0u;
      }
    }
    const uint32_t c_gt = block_sum(my_gt, s_wave), c_eq = block_sum(my_eq, s_wave);
    if (c_gt + c_eq <= static_cast<uint32_t>(kFastKept)) {   // uniform
      collect_given<CH>(total, M, c_eq, c_gt, entry, keys, s_count, s_wave);
      sort_write_any(keys, c_gt + c_eq, k, f, out_idx, out_score);
    } else if (c_gt < static_cast<uint32_t>(keff)) {
      // M is then the keff-th largest: all entries above it and the first
      // ties in key order
      collect_given<CH>(total, M, static_cast<uint32_t>(keff) - c_gt, c_gt, entry, keys, s_count, s_wave);
      sort_write_any(keys, static_cast<unsigned>(keff), k, f, out_idx, out_score);
    } else {
      exact_collect(total, keff, entry, keys, L, s_count, s_wave);
      sort_write_any(keys, static_cast<unsigned>(keff), k, f, out_idx, out_score);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kSelectThreads) void scan_merge_kernel(ScanArgs a, int k, int parts,
                                                                    int32_t* __restrict__ out_idx,
                                                                    float* __restrict__ out_score) {
  constexpr int PT = kCandCap / kSelectThreads;
  __shared__ unsigned long long keys[kCandCap];     // sort buffer (score, ~index)
  __shared__ SelectLds L;
  __shared__ uint32_t s_count[2];
  __shared__ uint32_t s_wave[kSelectWaves];
  __shared__ uint32_t s_span[2];   // positions filled by this workgroup's scatter
  __shared__ uint32_t s_pref[kRescueMaxWgs + 1];
  __shared__ int s_list[kRescueSlots];
  const int bid = blockIdx.x;
  if (bid >= a.num_q * parts) {   // uniform: a rescue workgroup
    rescue_role(a, k, bid - a.num_q * parts, out_idx, out_score, keys, L, s_count, s_wave, s_pref, s_list);
    return;
  }
  const int q = bid % a.num_q;
  const int part = bid / a.num_q;
  const uint32_t p_lo = static_cast<uint32_t>(int64_t(k) * part / parts);
  const uint32_t p_hi = static_cast<uint32_t>(int64_t(k) * (part + 1) / parts);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  static_assert(PT * kSelectThreads == kCandCap, "one register per candidate slot");
  // The first kSpecSlots slots of the list load at once, before the count
  // arrives (the list is allocated to its capacity; slots past the count
  // are masked later), so the two memory round trips overlap.  The rest load
  // only for a longer list, bounded by the count (a lane past it reads 0
  // without a memory access).
  constexpr int kSpecSlots = 6;
  uint32_t v[PT], id[PT];
  {
    const __amdgpu_buffer_rsrc_t cand = __builtin_amdgcn_make_buffer_rsrc(
        a.cand + int64_t(q) * kCandCap, static_cast<short>(0), kSpecSlots * kSelectThreads * 8, 0x00020000);
#pragma unroll
    for (int j = 0; j < kSpecSlots; ++j) {
      const v2u32 e = __builtin_amdgcn_raw_buffer_load_b64(cand, (tid + j * kSelectThreads) * 8, 0, 0);
      v[j] = e.x;
      id[j] = e.y;
    }
  }
  const uint32_t cnt = a.count[q];
  // (loaded with the count and consumed here: left to its use under the
  // branch below, the load would cost a round trip of its own)
  const float theta_q = a.theta[q];
  asm volatile("" : : "v"(theta_q));
  unsigned kept = 0;
  bool fast = false;   // uniform
  if (list_missed(cnt, k) && rescue_slot(a, q, k, s_wave) >= 0) return;   // uniform: the rescue places it

  if (cnt >= static_cast<uint32_t>(k) && cnt <= static_cast<uint32_t>(kCandCap)) {
    if (cnt > static_cast<uint32_t>(kSpecSlots * kSelectThreads)) {   // uniform
      const __amdgpu_buffer_rsrc_t cand = __builtin_amdgcn_make_buffer_rsrc(
          a.cand + int64_t(q) * kCandCap, static_cast<short>(0), static_cast<int>(cnt * 8u), 0x00020000);
#pragma unroll
      for (int j = kSpecSlots; j < PT; ++j) {
        const v2u32 e = __builtin_amdgcn_raw_buffer_load_b64(cand, (tid + j * kSelectThreads) * 8, 0, 0);
        v[j] = float_to_ordered(__uint_as_float(e.x));
        id[j] = e.y;
      }
    }
    // slots j < nj of this wavefront hold candidates; the others are left
    // out (their pm bit stays clear, and every later use tests pm)
    const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63);
    const int nj = min(PT, max(0, (static_cast<int>(cnt) - wbase + kSelectThreads - 1) / kSelectThreads));
    // The scan's filter may also pass keys just below theta; only candidates
    // scoring >= theta count, and the list is complete for the top k exactly
    // when at least k of them do.
    const uint32_t theta_o = float_to_ordered(theta_q);
    uint32_t pm = 0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      if (j < nj) {   // uniform
        const uint32_t i = tid + j * kSelectThreads;
        v[j] = i < cnt ? (j < kSpecSlots ? float_to_ordered(__uint_as_float(v[j])) : v[j]) : 0u;
        pm |= (i < cnt && v[j] >= theta_o) ? (1u << j) : 0u;
      }
    }
    DigitLds& D = *reinterpret_cast<DigitLds*>(keys + kFastKept);
    digit_clear(D);
    const uint3 mm = block_max_min<PT>(v, pm, L, nj);
    if (mm.z >= static_cast<uint32_t>(k)) {
      fast = true;
      // Fast path: one digit pass puts the candidates into ordered buckets;
      // those at or above the bucket holding rank k-1 are scattered in
      // bucket order and each is placed by counting the larger keys of its
      // bucket.
      bool placed = false;
      if (mm.x != mm.y) {
        const int hi = 32 - __clz(mm.x ^ mm.y);
        const int width = min(kDigitBits, hi), shift = hi - width;
        const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
        for (int j = 0; j < PT; ++j)
          if (j < nj) hist_add(D.hist, (pm >> j) & 1u, (v[j] >> shift) & dmask);
        __syncthreads();
        digit_scan(D, static_cast<uint32_t>(k) - 1u);
        if (D.big == 0u) {
          // this workgroup scatters the buckets that overlap its output
          // ranks [p_lo, p_hi); they fill positions [s_span[0], s_span[1])
          const uint32_t bstar = D.bstar;
          if (tid == 0) {
            s_span[0] = 0xffffffffu;
            s_span[1] = 0u;
          }
          __syncthreads();
          uint32_t lo_w = 0xffffffffu, hi_w = 0u;
#pragma unroll
          for (int j = 0; j < PT; ++j) {
            const uint32_t d = (v[j] >> shift) & dmask;
            if (j < nj && ((pm >> j) & 1u) && d >= bstar) {
              const uint32_t b0 = D.start[d], b1 = b0 + D.hist[d];
              if (b0 < p_hi && b1 > p_lo) {
                keys[b0 + atomicAdd(&D.cursor[d], 1u)] = sort_key(v[j], id[j]);
                lo_w = min(lo_w, b0);
                hi_w = max(hi_w, b1);
              }
            }
          }
          const uint2 span = wave_max_min(hi_w, lo_w);
          if (lane == 0 && span.x != 0u) {
            atomicMin(&s_span[0], span.y);
            atomicMax(&s_span[1], span.x);
          }
          __syncthreads();
          const uint32_t sp0 = s_span[0], sp1 = s_span[1];
          for (uint32_t p = sp0 + tid; p < sp1; p += kSelectThreads) {
            const unsigned long long key = keys[p];
            const uint32_t d = (static_cast<uint32_t>(key >> 32) >> shift) & dmask;
            const uint32_t b0 = D.start[d], c = D.hist[d];
            // (four independent reads per round keep several LDS reads in flight)
            uint32_t rank = 0, i = 0;
            for (; i + 4 <= c; i += 4) {
              const unsigned long long k0 = keys[b0 + i], k1 = keys[b0 + i + 1];
              const unsigned long long k2 = keys[b0 + i + 2], k3 = keys[b0 + i + 3];
              rank += (k0 > key ? 1u : 0u) + (k1 > key ? 1u : 0u) + (k2 > key ? 1u : 0u) + (k3 > key ? 1u : 0u);
            }
            for (; i < c; ++i) rank += keys[b0 + i] > key ? 1u : 0u;
            const uint32_t pos = b0 + rank;
            if (pos >= p_lo && pos < p_hi) {
              out_idx[int64_t(q) * k + pos] = static_cast<int32_t>(~static_cast<uint32_t>(key));
              out_score[int64_t(q) * k + pos] = ordered_to_float(static_cast<uint32_t>(key >> 32));
            }
          }
          placed = true;
        }
      }
      if (placed || part != 0) return;   // uniform
      // General path (all scores equal, or a bucket too large to order by
      // counting): the k-th best candidate score by radix select; every
      // candidate at or above it is kept and sorted.
      const uint2 sel = block_select_regs<PT>(v, pm, static_cast<uint32_t>(k), L);
      if (tid == 0) s_count[0] = 0;
      __syncthreads();
      // compaction: one LDS atomic per wave and register slot
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const bool keep = ((pm >> j) & 1u) && v[j] >= sel.x;
        const uint64_t bal = __ballot(keep);
        if (bal == 0) continue;
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&s_count[0], static_cast<uint32_t>(__popcll(bal)));
        base = read_lane(base, 0);
        if (keep) keys[base + lanes_below(bal)] = sort_key(v[j], id[j]);
      }
      __syncthreads();
      kept = s_count[0];
    }
  }
  if (!fast) {
    if (part != 0) return;   // uniform
    // (the early loads are consumed on this path too, so the compiler keeps
    // them ahead of the count test instead of sinking them into the fast path)
#pragma unroll
    for (int j = 0; j < kSpecSlots; ++j) asm volatile("" : : "v"(v[j]), "v"(id[j]));
    // exact fallback, alone: every score recomputed (the main kernel's
    // fixed-point arithmetic) in each select pass; a head holding fewer than
    // k keys returns all of them
    const int h = q / a.group;
    const int64_t nh = head_length(a.lengths, h, a.n);
    const int keff = static_cast<int>(min<int64_t>(k, nh));
    const uint32_t* head_planes = a.planes + int64_t(h) * kD * kPlanes * a.ldw;
    QueryPlan& P = plan_in(keys);
    load_plan(a, q, P);
    exact_collect(nh, keff, [&](int64_t i) { return make_uint2(plan_score(head_planes, P, i), static_cast<uint32_t>(i)); },
                  keys, L, s_count, s_wave);
    kept = static_cast<unsigned>(keff);
  }
  // keys[0, kept) hold the kept keys (kept >= k unless the head holds fewer
  // than k): sort them and write the first k
  sort_write_any(keys, kept, k, q, out_idx, out_score);
}

// Main-kernel launches may carry a start and a stop event: recorded by the
// dispatch itself (hipExtLaunchKernelGGL), they add no packets to the stream.
template <int GQ>
void launch_chunk_class(const ScanArgs& a, int H, int nsb, bool sample_phase, hipEvent_t ev_start,
                        hipEvent_t ev_stop, hipStream_t stream) {
  if (sample_phase) {
    hipLaunchKernelGGL(scan_sample_kernel<GQ>, dim3(nsb, H * a.cph), dim3(kMainThreads), 0, stream, a);
  } else {
    hipExtLaunchKernelGGL(scan_main_kernel<GQ>, dim3(a.main_wgs * H * a.cph), dim3(kMainThreads), 0, stream,
                          ev_start, ev_stop, 0, a);
  }
}

void launch_class(int gq, const ScanArgs& a, int H, int nsb, bool sample_phase, hipEvent_t ev_start,
                  hipEvent_t ev_stop, hipStream_t stream) {
  switch (gq) {
    case 1: launch_chunk_class<1>(a, H, nsb, sample_phase, ev_start, ev_stop, stream); break;
    case 2: launch_chunk_class<2>(a, H, nsb, sample_phase, ev_start, ev_stop, stream); break;
    case 3: launch_chunk_class<3>(a, H, nsb, sample_phase, ev_start, ev_stop, stream); break;
    default: launch_chunk_class<4>(a, H, nsb, sample_phase, ev_start, ev_stop, stream); break;
  }
}

}  // namespace

hipError_t launch_scan_topk(const uint32_t* planes, const float* lo, const float* step, int H,
                            int64_t n, const int32_t* lengths, int64_t ldw, const float* q, const uint8_t* alloc,
                            int num_q, int group, int k, int32_t* out_idx, float* out_score,
                            float* all_scores, const ScanWorkspace& ws, const ScanTiming* timing,
                            hipStream_t stream, const float* var, int budget, uint8_t* alloc_out) {
  ScanArgs a{};
  a.lengths = lengths;
  a.k = k;
  a.planes = planes;
  a.lo = lo;
  a.step = step;
  a.q = q;
  // fused allocation: the sample kernel writes alloc_out, which later
  // kernels read as the allocation
  a.alloc = var ? alloc_out : alloc;
  a.var = var;
  a.budget = budget;
  a.alloc_out = alloc_out;
  a.n = n;
  a.ldw = ldw;
  a.nwords = static_cast<int>((n + 31) / 32);
  a.group = group;
  a.tiles = (a.nwords + kTileWords - 1) / kTileWords;
  a.theta = ws.theta;
  a.count = ws.count;
  a.sample = ws.sample;
  a.cand = ws.cand;
  a.tables = ws.tables;
  a.all_scores = all_scores;
  a.num_q = num_q;
  a.rescue = ws.rescue;
  a.rescue_cnt = ws.rescue_cnt;
  a.rescue_hist = ws.rescue_hist;
  a.rescue_done = ws.rescue_done;
  a.rescue_wgs = ws.rescue_wgs;

  const int full = group / kQueryChunk;
  const int rest = group % kQueryChunk;
  a.chunks_per_head = full + (rest > 0 ? 1 : 0);
  const int64_t chunk_count = int64_t(H) * a.chunks_per_head;

  // sampled blocks: up to 8 blocks of 1024 keys spread evenly over the head;
  // with many (head, chunk) pairs fewer, so that the sample kernel stays
  // near 512 workgroups (one pass over the GPU) -- at least 2
  const int64_t nblocks = (n + kSampleBlockKeys - 1) / kSampleBlockKeys;
  const int64_t blocks_cap = std::max<int64_t>(2, std::min<int64_t>(kSampleMaxBlocks, 512 / chunk_count));
  const int nsb = static_cast<int>(std::min(nblocks, blocks_cap));
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
  a.rsel = static_cast<int>(rsel);
  // With per-head lengths the rank differs per head: the threshold kernel
  // takes each query's rank from its head's length.
  a.top_lists = (rsel <= kTopR && !lengths) ? 1 : 0;
  a.nsb = nsb;

  // main-kernel work split: each workgroup takes a contiguous run of tiles
  // of one (head, query chunk).  With per-block lists every workgroup first
  // selects theta itself, so the tiles go to one generation of resident
  // workgroups (kMainWgPerCu per CU); with theta from the threshold kernel
  // the start is cheap and two generations of shorter runs balance better
  // (workgroups that finish early are replaced by new ones).  Many sessions
  // (128 heads of 128K keys, B = 68): 71.4-73.6 us with two generations
  // against 80.5-82.0 with four, once the candidates of a run fit in LDS
  // (with 32 per wave and query, runs of 8 tiles spilled to the global
  // list about once per four tiles).
  const int64_t total_tiles = chunk_count * a.tiles;
  const int64_t target_wgs = int64_t(a.top_lists ? 1 : 2) * 256 * kMainWgPerCu;
  a.tiles_per_wg = static_cast<int>((total_tiles + target_wgs - 1) / target_wgs);
  if (a.tiles_per_wg < 1) a.tiles_per_wg = 1;
  a.main_wgs = (a.tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  a.interleave = a.top_lists;
  a.ramp_step = 2;

  // timing events: start on the first main launch, stop on the last
  hipEvent_t ev_start = timing ? timing->start : nullptr;
  hipEvent_t ev_stop = timing ? timing->stop : nullptr;
  for (int phase = 0; phase < 2; ++phase) {
    const bool sample_phase = phase == 0;
    if (full > 0) {
      ScanArgs b = a;
      b.cph = full;
      b.qoff = 0;
      launch_class(kQueryChunk, b, H, nsb, sample_phase, ev_start, rest > 0 ? nullptr : ev_stop, stream);
    }
    if (rest > 0) {
      ScanArgs b = a;
      b.cph = 1;
      b.qoff = full * kQueryChunk;
      launch_class(rest, b, H, nsb, sample_phase, full > 0 ? nullptr : ev_start, ev_stop, stream);
    }
    if (sample_phase && !a.top_lists) {
      hipLaunchKernelGGL(scan_threshold_kernel, dim3(num_q), dim3(kSelectThreads), 0, stream, ws.sample,
                         nsb * kSampleBlockKeys, static_cast<uint32_t>(rsel), ws.theta, ws.count, lengths, n, k,
                         group, nsb);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int merge_parts = std::max(1, std::min(kMergeSplit, 256 / std::max(1, num_q)));
  hipLaunchKernelGGL(scan_merge_kernel, dim3(num_q * merge_parts + a.rescue_wgs), dim3(kSelectThreads), 0, stream,
                     a, k, merge_parts, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace fathom
