// Per-head RMSNorm + partial rotary embedding, on q rows and fused into the
// q8 cache write of K.
//
// The "attention.rs" page normalizes q and k per head (learned weight, rms
// eps) and rotates the first rot = head_dim * partial_rotary_factor elements
// at the row's position (rope theta) before the q8 append; the kernel body is
// not printed.  Computed here (the usual per-head RMSNorm, then a rotate-half
// rotary embedding):
//   r   = 1 / sqrt(mean_d x_d^2 + eps)
//   n_d = x_d * r * w_d
//   for i < rot/2, a = n_i, b = n_{i+rot/2}, phi = pos * theta^(-2i/rot):
//     y_i = a cos(phi) - b sin(phi),  y_{i+rot/2} = b cos(phi) + a sin(phi)
//   y_d = n_d for d >= rot.
// The K result feeds the quantizer, whose codes are decided in binary32, so
// the rounding points are fixed: the sum of squares, mean + eps, square root
// and reciprocal in binary64, r rounded once to binary32; x*r and then *w as
// binary32 products; cos and sin from a per-position table computed in
// binary64 and rounded to binary32 (q8_rope_table); each rotated element as
// two binary32 products and one binary32 sum or difference, never fused.
//
// MI355X mapping: a vector is held by head_size/4 lanes, four elements each,
// as in the cache writer.  The sum of squares is a binary64 xor-shuffle
// reduction over those lanes; the partner of rotated element i (i + rot/2, or
// i - rot/2) sits in lane w +- rot/8 (rot a multiple of 8), fetched with one
// shuffle.  The fused writer runs one wavefront per (token, kv head), or in
// large writes per group of consecutive ones whose loads are all in flight
// together: for head sizes up to 128 lanes 0-31 take K through the norm and
// the rotation and lanes 32-63 pack V beside them, otherwise the wave does K
// and then V.
#include "q8kv_internal.h"
#include "q8_pack.h"

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

// Lane w of a group of WIDTH lanes holds elements 4w .. 4w+3 of x (zeros for
// w >= head_size/4); returns the same elements of the normalized and rotated
// vector.
template <int WIDTH>
__device__ __forceinline__ float4 norm_rope4(float4 x, uint32_t w, uint32_t head_size, const RopeLane& op,
                                             uint32_t rot, float eps) {
#pragma clang fp contract(off)
    double ss = static_cast<double>(x.x) * x.x + static_cast<double>(x.y) * x.y +
                static_cast<double>(x.z) * x.z + static_cast<double>(x.w) * x.w;
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, WIDTH);
    const float r = static_cast<float>(1.0 / sqrt(ss / static_cast<double>(head_size) + static_cast<double>(eps)));
    float4 n;
    n.x = (x.x * r) * op.wt.x;
    n.y = (x.y * r) * op.wt.y;
    n.z = (x.z * r) * op.wt.z;
    n.w = (x.w * r) * op.wt.w;
    // Rotated lanes: the first rot/8 lanes hold the a's, the next rot/8 the b's.
    const uint32_t h8 = rot / 8;
    const bool first = w < h8, second = !first && w < 2 * h8;
    const uint32_t src = first ? w + h8 : (second ? w - h8 : w);
    float4 p;
    p.x = __shfl(n.x, static_cast<int>(src), WIDTH);
    p.y = __shfl(n.y, static_cast<int>(src), WIDTH);
    p.z = __shfl(n.z, static_cast<int>(src), WIDTH);
    p.w = __shfl(n.w, static_cast<int>(src), WIDTH);
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

// table[p*rot + i] = cos(p * theta^(-2i/rot)), table[p*rot + rot/2 + i] = sin(...).
__global__ __launch_bounds__(256) void rope_table_kernel(float* table, uint32_t num_positions, uint32_t rot,
                                                          double theta) {
    const uint32_t half = rot / 2;
    const uint64_t k = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (k >= static_cast<uint64_t>(num_positions) * half) return;
    const uint32_t p = static_cast<uint32_t>(k / half), i = static_cast<uint32_t>(k % half);
    const double phi = static_cast<double>(p) * pow(theta, -(2.0 * i) / static_cast<double>(rot));
    table[static_cast<uint64_t>(p) * rot + i] = static_cast<float>(cos(phi));
    table[static_cast<uint64_t>(p) * rot + half + i] = static_cast<float>(sin(phi));
}

// Rows of f32 heads, WIDTH lanes per (row, head).
template <int WIDTH>
__global__ __launch_bounds__(256) void norm_rope_kernel(NormRopeArgs a, bool vec4) {
    constexpr int PER_WAVE = kWave / WIDTH;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t w = lane % WIDTH;
    const uint64_t unit = (static_cast<uint64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave) * PER_WAVE +
                          lane / WIDTH;
    const uint64_t units = static_cast<uint64_t>(a.num_rows) * a.num_heads;
    // Whole waves return together or not at all (the reductions shuffle across the group).
    if ((unit - lane / WIDTH) >= units) return;
    const bool live = unit < units;
    const uint32_t t = live ? static_cast<uint32_t>(unit / a.num_heads) : 0u;
    const uint32_t h = live ? static_cast<uint32_t>(unit % a.num_heads) : 0u;
    const uint32_t hs4 = a.head_size / 4;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live && w < hs4)
        x = load4(a.x + static_cast<uint64_t>(t) * a.x_stride + static_cast<uint64_t>(h) * a.head_stride + 4 * w, vec4);
    RopeLane op;
    op.wt = load_weight4(a.weight, w, hs4, a.params_vec4);
    const float* cs = live ? table_row(a.table, a.positions, t, a.rot, a.num_positions) : a.table;
    load_cs4(cs, w, a.rot, a.params_vec4, op.c, op.s);
    const float4 y = norm_rope4<WIDTH>(x, w, a.head_size, op, a.rot, a.eps);
    if (live && w < hs4) {
        float* o = a.out + static_cast<uint64_t>(t) * a.out_stride + static_cast<uint64_t>(h) * a.head_size + 4 * w;
        if (vec4) *reinterpret_cast<float4*>(o) = y;
        else { o[0] = y.x; o[1] = y.y; o[2] = y.z; o[3] = y.w; }
    }
}

// Cache write with the norm + rotary step on K: one wave per NP consecutive
// (token, kv head) pairs, every pair's rows and slot loaded before any is
// processed (NP > 1 for large writes, to keep several rows in flight).
template <bool HALF, int NP>
__global__ __launch_bounds__(256) void norm_rope_cache_write_kernel(NormRopeCacheWriteArgs a, bool vec4) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t first = (static_cast<uint64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave) * NP;
    const uint64_t pairs = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads;
    if (first >= pairs) return;
    const uint32_t hs4 = a.head_size / 4, wpt = hs4 + 1;
    float4 xk[NP], xv[NP];
    uint32_t slot[NP], head[NP], posn[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        xk[i] = xv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        slot[i] = kPadSlot;
        head[i] = posn[i] = 0;
        const uint64_t pair = first + i;
        if (pair >= pairs) continue;                     // wave-uniform
        const uint32_t t = static_cast<uint32_t>(pair / a.num_kv_heads);
        const uint32_t h = static_cast<uint32_t>(pair % a.num_kv_heads);
        head[i] = h;
        // A pad token's rows and position may be read (loaded with the slot),
        // but nothing is written for it.
        const float* ksrc = a.key + static_cast<uint64_t>(t) * a.key_stride + static_cast<uint64_t>(h) * a.head_size;
        const float* vsrc = a.value + static_cast<uint64_t>(t) * a.value_stride + static_cast<uint64_t>(h) * a.head_size;
        if (HALF) {
            const uint32_t w = lane & 31;
            if (w < hs4) xk[i] = load4((lane >= 32 ? vsrc : ksrc) + 4 * w, vec4);
        } else if (lane < hs4) {
            xk[i] = load4(ksrc + 4 * lane, vec4);
            xv[i] = load4(vsrc + 4 * lane, vec4);
        }
        slot[i] = a.slot_mapping[t];
        if (a.rot > 0) posn[i] = a.positions[t];
    }
    // The table rows of every pair's position, loaded together (one round
    // trip after the rows), and the norm weight once per wave.
    const uint32_t w = HALF ? (lane & 31) : lane;
    RopeLane op[NP];
    const float4 wt = load_weight4(a.weight, w, hs4, a.params_vec4);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        op[i].wt = wt;
        op[i].c = op[i].s = make_float4(0.f, 0.f, 0.f, 0.f);
        if (slot[i] == kPadSlot || a.rot == 0) continue;
        // positions[t] < num_positions is a caller contract: clamped rather than read out of bounds
        const uint32_t p = posn[i] < a.num_positions ? posn[i] : a.num_positions - 1;
        load_cs4(a.table + static_cast<uint64_t>(p) * a.rot, w, a.rot, a.params_vec4, op[i].c, op[i].s);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        if (slot[i] == kPadSlot) continue;
        const uint64_t block = slot[i] / a.block_size, off = slot[i] % a.block_size;
        if (block >= a.num_blocks) continue;             // out of contract; skipped rather than written out of bounds
        const uint64_t dst = ((block * a.num_kv_heads + head[i]) * a.block_size + off) * wpt;
        if (HALF) {
            const bool is_v = lane >= 32;
            const float4 y = norm_rope4<32>(xk[i], w, a.head_size, op[i], a.rot, a.eps);
            pack_vector<32>(is_v ? xk[i] : y, (is_v ? a.value_cache : a.key_cache) + dst, hs4, w);
        } else {
            const float4 y = norm_rope4<64>(xk[i], lane, a.head_size, op[i], a.rot, a.eps);
            pack_vector<64>(y, a.key_cache + dst, hs4, lane);
            pack_vector<64>(xv[i], a.value_cache + dst, hs4, lane);
        }
    }
}

}  // namespace

hipError_t launch_rope_table(float* table, uint32_t num_positions, uint32_t rot, double theta, hipStream_t stream) {
    const uint64_t n = static_cast<uint64_t>(num_positions) * (rot / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream, table,
                       num_positions, rot, theta);
    return hipGetLastError();
}

hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t stream) {
    const bool vec4 = reinterpret_cast<uintptr_t>(a.x) % 16 == 0 && reinterpret_cast<uintptr_t>(a.out) % 16 == 0 &&
                      a.x_stride % 4 == 0 && a.head_stride % 4 == 0 && a.out_stride % 4 == 0;
    const uint64_t units = static_cast<uint64_t>(a.num_rows) * a.num_heads;
    if (a.head_size / 4 <= 32) {
        const uint64_t waves = (units + 1) / 2;
        hipLaunchKernelGGL(norm_rope_kernel<32>, dim3(static_cast<uint32_t>((waves + 3) / 4)), dim3(256), 0, stream, a,
                           vec4);
    } else {
        hipLaunchKernelGGL(norm_rope_kernel<64>, dim3(static_cast<uint32_t>((units + 3) / 4)), dim3(256), 0, stream, a,
                           vec4);
    }
    return hipGetLastError();
}

hipError_t launch_norm_rope_cache_write(const NormRopeCacheWriteArgs& a, hipStream_t stream) {
    const uint64_t pairs = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads;
    const bool vec4 = reinterpret_cast<uintptr_t>(a.key) % 16 == 0 && reinterpret_cast<uintptr_t>(a.value) % 16 == 0 &&
                      a.key_stride % 4 == 0 && a.value_stride % 4 == 0;
    const bool half = a.head_size / 4 <= 32;
    if (pairs >= kWriteBatchMinPairs) {
        // Two pairs per wave: the step's registers for four would cut occupancy from 8 waves per SIMD to 5.
        constexpr int NP = 2;
        const dim3 grid(static_cast<uint32_t>((pairs + 4 * NP - 1) / (4 * NP)));
        if (half) hipLaunchKernelGGL((norm_rope_cache_write_kernel<true, NP>), grid, dim3(256), 0, stream, a, vec4);
        else hipLaunchKernelGGL((norm_rope_cache_write_kernel<false, NP>), grid, dim3(256), 0, stream, a, vec4);
    } else {
        const dim3 grid(static_cast<uint32_t>((pairs + 3) / 4));
        if (half) hipLaunchKernelGGL((norm_rope_cache_write_kernel<true, 1>), grid, dim3(256), 0, stream, a, vec4);
        else hipLaunchKernelGGL((norm_rope_cache_write_kernel<false, 1>), grid, dim3(256), 0, stream, a, vec4);
    }
    return hipGetLastError();
}

}  // namespace q8kv
