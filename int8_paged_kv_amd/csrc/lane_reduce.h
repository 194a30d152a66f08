// Reductions over aligned groups of 16, 32 or 64 lanes of a wavefront, with
// the result in every lane of the group, bit-identical across them.
//
// The steps pair lanes 1 and 2 apart (DPP quad permutations), the mirrored
// halves of each 8 and each 16 lanes (DPP row mirrors), then, for 32- and
// 64-lane groups, lanes 16 apart (a swizzle inside 32 lanes) and, for 64-lane
// groups, the two 32-lane halves (lanes 0 and 32 read out).  A 16-lane group
// therefore sums in the same order as the first half of a 32-lane one.  Before every step the lanes on each side of a
// pairing already hold one identical value, so a commutative operation leaves
// all lanes agreeing.  DPP and swizzle patterns are immediates: no lane index
// arithmetic as with a general shuffle.  All lanes of the wave must be active.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8kv {
namespace lanes {

constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;       // lane i <- 15 - i within 16
constexpr int kSwzXor16 = (0x10 << 10) | 0x1F;   // bit mode: lane i <- i ^ 16 within 32

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) { return __uint_as_float(dpp<CTRL>(__float_as_uint(v))); }
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
    const uint64_t lo = dpp<CTRL>(static_cast<uint32_t>(u)), hi = dpp<CTRL>(static_cast<uint32_t>(u >> 32));
    return __longlong_as_double(static_cast<long long>(lo | (hi << 32)));
}

__device__ __forceinline__ uint32_t swz16(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), kSwzXor16));
}
__device__ __forceinline__ float swz16(float v) { return __uint_as_float(swz16(__float_as_uint(v))); }
__device__ __forceinline__ double swz16(double v) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
    const uint64_t lo = swz16(static_cast<uint32_t>(u)), hi = swz16(static_cast<uint32_t>(u >> 32));
    return __longlong_as_double(static_cast<long long>(lo | (hi << 32)));
}

__device__ __forceinline__ float read_lane(float v, int l) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(v)), l)));
}
__device__ __forceinline__ double read_lane(double v, int l) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
    const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), l));
    const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), l));
    return __longlong_as_double(static_cast<long long>(lo | (hi << 32)));
}

template <int WIDTH, typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, Op op) {
    static_assert(WIDTH == 16 || WIDTH == 32 || WIDTH == 64, "groups of 16, 32 or 64 lanes");
    v = op(v, dpp<kDppXor1>(v));
    v = op(v, dpp<kDppXor2>(v));
    v = op(v, dpp<kDppHalfMirror>(v));
    v = op(v, dpp<kDppMirror>(v));
    if (WIDTH >= 32) v = op(v, swz16(v));
    if (WIDTH == 64) v = op(read_lane(v, 0), read_lane(v, 32));
    return v;
}

}  // namespace lanes

// max over the group (fmaxf: a NaN operand is ignored)
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
    return lanes::group_reduce<WIDTH>(v, [](float a, float b) { return fmaxf(a, b); });
}

// binary64 sum over the group, as a tree of pairwise sums
template <int WIDTH>
__device__ __forceinline__ double group_sum(double v) {
    return lanes::group_reduce<WIDTH>(v, [](double a, double b) { return a + b; });
}

}  // namespace q8kv
