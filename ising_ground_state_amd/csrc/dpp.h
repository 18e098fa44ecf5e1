// Cross-lane reductions through DPP for the search kernels (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace qubo {

// Cross-lane moves through DPP (data-parallel primitives: the source lane is
// picked by the VALU instruction itself, no LDS round trip).  gfx9 controls:
// quad_perm within 4 lanes, mirrors within 8 and 16 lanes, and the broadcasts of
// lane 15 of each row into the next row and of lane 31 into rows 2 and 3.  Lanes
// of rows outside row_mask keep `old`.
constexpr int kDppSwap1 = 0xB1;      // quad_perm [1, 0, 3, 2]: lane ^ 1
constexpr int kDppSwap2 = 0x4E;      // quad_perm [2, 3, 0, 1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within 8 lanes
constexpr int kDppMirror = 0x140;    // lane i <- 15 - i within 16 lanes
constexpr int kDppBcast15 = 0x142;   // rows 1, 3 <- lane 15 of rows 0, 2
constexpr int kDppBcast31 = 0x143;   // rows 2, 3 <- lane 31

template <int Ctrl, int RowMask>
__device__ __forceinline__ int dpp_i32(int old, int v)
{
    return __builtin_amdgcn_update_dpp(old, v, Ctrl, RowMask, 0xf, false);
}

template <int Ctrl, int RowMask>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t old, uint64_t v)
{
    const uint32_t lo = (uint32_t)dpp_i32<Ctrl, RowMask>((int)(uint32_t)old, (int)(uint32_t)v);
    const uint32_t hi = (uint32_t)dpp_i32<Ctrl, RowMask>((int)(uint32_t)(old >> 32), (int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// One reduction step of `op` over lanes paired by a DPP control; lanes outside
// row_mask combine with the identity `id`.
template <int Ctrl, int RowMask, class T, class Op>
__device__ __forceinline__ void dpp_step(T &v, T id, Op op)
{
    if constexpr (sizeof(T) == 8)
        v = op(v, (T)dpp_u64<Ctrl, RowMask>((uint64_t)id, (uint64_t)v));
    else
        v = op(v, (T)dpp_i32<Ctrl, RowMask>((int)id, (int)v));
}

// Reduction of a commutative, associative `op` over the 64 lanes: pairs, quads,
// half-rows and rows by swaps and mirrors, then rows 0+1 and 2+3 by the lane-15
// broadcast and all four by the lane-31 broadcast.  Lane 63 ends with the
// result, which is returned to every lane (wave-uniform).
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T v, T id, Op op)
{
    static_assert(std::is_integral<T>::value, "lanes move as integer bits");
    dpp_step<kDppSwap1, 0xf>(v, id, op);
    dpp_step<kDppSwap2, 0xf>(v, id, op);
    dpp_step<kDppHalfMirror, 0xf>(v, id, op);
    dpp_step<kDppMirror, 0xf>(v, id, op);
    dpp_step<kDppBcast15, 0xa>(v, id, op);
    dpp_step<kDppBcast31, 0xc>(v, id, op);
    if constexpr (sizeof(T) == 8)
        return (T)readlane_u64((uint64_t)v, 63);
    else
        return (T)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace qubo
