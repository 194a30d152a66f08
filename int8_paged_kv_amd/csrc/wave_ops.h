// Wavefront-level helpers shared by the decode kernels: DPP row reductions,
// uniform values, an inclusive prefix sum and an in-order LDS hand-off.
#pragma once
#include "q8kv_internal.h"

namespace q8kv {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor1 = 0x121;
constexpr int kRowRor2 = 0x122;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Reductions over the 16 lanes of a DPP row (rotations within the row).
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dpp_mov<kRowRor1>(v));
    v = fmaxf(v, dpp_mov<kRowRor2>(v));
    v = fmaxf(v, dpp_mov<kRowRor4>(v));
    return fmaxf(v, dpp_mov<kRowRor8>(v));
}
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_mov<kRowRor1>(v);
    v += dpp_mov<kRowRor2>(v);
    v += dpp_mov<kRowRor4>(v);
    return v + dpp_mov<kRowRor8>(v);
}

// LDS hand-off between the lanes of one wavefront: LDS operations of a
// wavefront execute in order, so only compiler reordering must be prevented
// (the wavefronts of a workgroup never wait for each other).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, uint32_t lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t t = __shfl_up(v, d, kWave);
        if (lane >= static_cast<uint32_t>(d)) v += t;
    }
    return v;
}

__device__ __forceinline__ uint32_t lane_value(uint32_t v, uint32_t l) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), static_cast<int>(l)));
}

}  // namespace q8kv
