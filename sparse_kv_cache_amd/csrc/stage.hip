// Host-resident store, staged into HBM head by head: the union rows of a KV
// head's query group (per channel c the contiguous rows j < u_c, u_c the
// deepest prefix any of the group's queries reads) are read from pinned host
// memory over PCIe by the compute units and written into a staging slot,
// while the previous head is scanned from the other slot ("Fathom: Per-Query
// Read Depth for Sparse Decoding over Offloaded KV Caches", abstract s1, s6;
// "Fathom Makes KV-Cache Scans Query-Adaptive for Long-Context Decoding",
// para 1 and the limits paragraph: with the index in host memory, the bytes
// that cross the link are what the method saves).
//
// The union is computed here from the allocation in device memory, so no
// host round trip is needed.  Each workgroup copies a share of one channel's
// contiguous run in 16-byte loads, several in flight per thread.

#include <algorithm>

#include "fathom_internal.h"

namespace fathom {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kStageThreads = 256;
constexpr int kStageUnroll = 8;

__global__ __launch_bounds__(kStageThreads) void stage_union_kernel(const uint32_t* __restrict__ src_head,
                                                                    uint32_t* __restrict__ dst_head,
                                                                    const uint8_t* __restrict__ alloc, int group,
                                                                    int64_t ldw, int splits) {
  const int c = blockIdx.x;
  const int part = blockIdx.y;
  __shared__ int u_s;
  if (threadIdx.x == 0) {
    int u = 0;
    for (int g = 0; g < group; ++g) u = max(u, min(static_cast<int>(alloc[g * kD + c]), kPlanes));
    u_s = u;
  }
  __syncthreads();
  // rows c * 4 .. c * 4 + u - 1 are contiguous: u * ldw words, a multiple of 4
  const int64_t n16 = int64_t(u_s) * ldw / 4;
  const int64_t p0 = n16 * part / splits, p1 = n16 * (part + 1) / splits;
  const v4u* src = reinterpret_cast<const v4u*>(src_head + int64_t(c) * kPlanes * ldw);
  v4u* dst = reinterpret_cast<v4u*>(dst_head + int64_t(c) * kPlanes * ldw);
  for (int64_t i = p0 + threadIdx.x; i < p1; i += kStageUnroll * kStageThreads) {
    v4u x[kStageUnroll];
#pragma unroll
    for (int r = 0; r < kStageUnroll; ++r) {
      const int64_t j = i + r * kStageThreads;
      if (j < p1) x[r] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int r = 0; r < kStageUnroll; ++r) {
      const int64_t j = i + r * kStageThreads;
      if (j < p1) dst[j] = x[r];
    }
  }
}

}  // namespace

hipError_t launch_stage_union(const uint32_t* src_head, uint32_t* dst_head, const uint8_t* alloc, int group,
                              int64_t ldw, hipStream_t stream) {
  // up to 4 rows of ldw words per channel: about 64 KiB per workgroup
  const int64_t max_bytes = int64_t(kPlanes) * ldw * 4;
  const int splits = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(64, (max_bytes + 65535) / 65536)));
  hipLaunchKernelGGL(stage_union_kernel, dim3(kD, splits), dim3(kStageThreads), 0, stream, src_head, dst_head, alloc,
                     group, ldw, splits);
  return hipGetLastError();
}

}  // namespace fathom
