// Wavefront-wide building blocks shared by the kernels: DPP operand routing
// and a bitonic sort across the 64 lanes.
#ifndef FATHOM_WAVE_OPS_H
#define FATHOM_WAVE_OPS_H

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fathom {

// Cross-lane steps use DPP (operand routing inside the VALU instruction) and
// lane swaps rather than ds_bpermute, whose LDS round trip is ~100 cycles per
// step and queues behind the scan's LDS traffic.
// GFX9 DPP controls: quad_perm, row_shr:n, row_mirror, row_half_mirror,
// row_bcast:15 / row_bcast:31 (rows are 16 lanes).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowShl = 0x100;       // + n: row_shl:n (lane reads lane + n of its row)
constexpr int kDppRowShr = 0x110;       // + n: row_shr:n (lane reads lane - n of its row)
constexpr int kDppRowRor = 0x120;       // + n: row_ror:n
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), Ctrl,
                                                           RowMask, 0xf, false));
}

// v of lane (lane ^ J): DPP for J < 16; for 16 and 32 the gfx950 lane swaps
// (v_permlane16_swap / v_permlane32_swap: with v in both operands, the first
// result holds each pair's lower half of v in both halves of the pair, the
// second its upper half), which stay in the VALU.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (J == 1) {
    return dpp_u32<kDppXor1>(v, v);
  } else if constexpr (J == 2) {
    return dpp_u32<kDppXor2>(v, v);
  } else if constexpr (J == 4) {
    const uint32_t up = dpp_u32<kDppRowShl + 4>(v, v);   // lane + 4 (used where bit 2 is clear)
    const uint32_t dn = dpp_u32<kDppRowShr + 4>(v, v);   // lane - 4 (used where it is set)
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return dpp_u32<kDppRowRor + 8>(v, v);               // rotation by half a row
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "xor distances 1 .. 32");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

// One compare-exchange step of a bitonic network: merge size K, distance J.
template <int K, int J>
__device__ __forceinline__ uint32_t bitonic_step(uint32_t v) {
  const uint32_t p = xor_lane<J>(v);
  const int lane = threadIdx.x & 63;
  const bool keep_max = ((lane & J) == 0) == ((lane & K) == 0);
  return keep_max ? max(v, p) : min(v, p);
}

// The wavefront's 64 values (one per lane) in descending order across the lanes.
__device__ inline uint32_t wave_sort_desc(uint32_t v) {
  v = bitonic_step<2, 1>(v);
  v = bitonic_step<4, 2>(v);
  v = bitonic_step<4, 1>(v);
  v = bitonic_step<8, 4>(v);
  v = bitonic_step<8, 2>(v);
  v = bitonic_step<8, 1>(v);
  v = bitonic_step<16, 8>(v);
  v = bitonic_step<16, 4>(v);
  v = bitonic_step<16, 2>(v);
  v = bitonic_step<16, 1>(v);
  v = bitonic_step<32, 16>(v);
  v = bitonic_step<32, 8>(v);
  v = bitonic_step<32, 4>(v);
  v = bitonic_step<32, 2>(v);
  v = bitonic_step<32, 1>(v);
  v = bitonic_step<64, 32>(v);
  v = bitonic_step<64, 16>(v);
  v = bitonic_step<64, 8>(v);
  v = bitonic_step<64, 4>(v);
  v = bitonic_step<64, 2>(v);
  v = bitonic_step<64, 1>(v);
  return v;
}

}  // namespace fathom

#endif  // FATHOM_WAVE_OPS_H
