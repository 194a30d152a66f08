// The per-head RMSNorm + partial rotary step on one vector held by a group of
// lanes, shared by the norm + rotary kernels and the decode step that applies
// it to q rows and to the appended K row.  What it computes and its rounding
// points are described in norm_rope.hip (the "attention.rs" page's q/k
// norm-and-rope dispatch).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "lane_reduce.h"

namespace q8kv {
namespace {

__device__ __forceinline__ float4 load4(const float* p, bool vec4) {
    if (vec4) return *reinterpret_cast<const float4*>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
}

// Per-lane operands of the step that do not depend on the vector: its four
// weights and, for lanes holding rotated elements, four cos and four sin
// values from the table row of the vector's position (rot/8 lanes hold the
// first elements a of the pairs, the next rot/8 the second elements b).
struct RopeLane {
    float4 wt, c, s;
};
__device__ __forceinline__ float4 load_weight4(const float* weight, uint32_t w, uint32_t hs4, bool pvec4) {
    return w < hs4 ? load4(weight + 4 * w, pvec4) : make_float4(0.f, 0.f, 0.f, 0.f);
}
__device__ __forceinline__ void load_cs4(const float* cs, uint32_t w, uint32_t rot, bool pvec4, float4& c, float4& s) {
    const uint32_t h8 = rot / 8;
    c = s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (w >= 2 * h8) return;
    const uint32_t i0 = 4 * (w < h8 ? w : w - h8);
    c = load4(cs + i0, pvec4);
    s = load4(cs + rot / 2 + i0, pvec4);
}

// The mean of a sum over head_size elements, as the binary64 quotient.  A
// power-of-two head size divides exactly by multiplying with its reciprocal
// (2^-k, built from its exponent bits), which spares the division sequence.
struct RowMean {
    uint32_t head_size;
    bool pow2;
    double inv;
    __device__ __forceinline__ explicit RowMean(uint32_t hs) : head_size(hs), pow2((hs & (hs - 1)) == 0), inv(0.0) {
        if (pow2) inv = __longlong_as_double(static_cast<long long>(1023 - __builtin_ctz(hs)) << 52);
    }
    __device__ __forceinline__ double operator()(double ss) const {
        return pow2 ? ss * inv : ss / static_cast<double>(head_size);
    }
};

// Lane w of a group of WIDTH lanes holds elements 4w .. 4w+3 of x (zeros for
// w >= head_size/4); returns the same elements of the normalized and rotated
// vector.
template <int WIDTH>
__device__ __forceinline__ float4 norm_rope4(float4 x, uint32_t w, const RowMean& mean, const RopeLane& op,
                                             uint32_t rot, float eps) {
#pragma clang fp contract(off)
    const double ss = group_sum<WIDTH>(static_cast<double>(x.x) * x.x + static_cast<double>(x.y) * x.y +
                                       static_cast<double>(x.z) * x.z + static_cast<double>(x.w) * x.w);
    const float r = static_cast<float>(1.0 / sqrt(mean(ss) + static_cast<double>(eps)));
    float4 n;
    n.x = (x.x * r) * op.wt.x;
    n.y = (x.y * r) * op.wt.y;
    n.z = (x.z * r) * op.wt.z;
    n.w = (x.w * r) * op.wt.w;
    // Rotated lanes: the first rot/8 lanes hold the a's, the next rot/8 the b's.
    const uint32_t h8 = rot / 8;
    const bool first = w < h8, second = !first && w < 2 * h8;
    const uint32_t src = first ? w + h8 : (second ? w - h8 : w);
    // byte address of the partner lane in the wave (the same for every vector of the wave)
    const int addr = static_cast<int>(((__lane_id() & ~static_cast<uint32_t>(WIDTH - 1)) + src) << 2);
    float4 p;
    p.x = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(n.x)));
    p.y = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(n.y)));
    p.z = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(n.z)));
    p.w = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(n.w)));
    if (!first && !second) return n;
    const float c[4] = {op.c.x, op.c.y, op.c.z, op.c.w};
    const float s[4] = {op.s.x, op.s.y, op.s.z, op.s.w};
    const float nn[4] = {n.x, n.y, n.z, n.w}, pp[4] = {p.x, p.y, p.z, p.w};
    float y[4];
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        const float own = nn[l] * c[l];
        const float other = pp[l] * s[l];
        y[l] = first ? own - other : own + other;     // a c - b s  |  b c + a s
    }
    return make_float4(y[0], y[1], y[2], y[3]);
}

__device__ __forceinline__ const float* table_row(const float* table, const uint32_t* positions, uint32_t t,
                                                  uint32_t rot, uint32_t num_positions) {
    if (rot == 0) return table;
    uint32_t p = positions[t];
    p = p < num_positions ? p : num_positions - 1;    // out of contract; clamped rather than read out of bounds
    return table + static_cast<uint64_t>(p) * rot;
}

}  // namespace
}  // namespace q8kv
