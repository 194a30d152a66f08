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
// as in the cache writer.  The sum of squares is a binary64 tree reduction
// over those lanes (DPP and swizzle steps); the partner of rotated element i
// (i + rot/2, or i - rot/2) sits in lane w +- rot/8 (rot a multiple of 8),
// fetched with one permute.  The fused writer runs one wavefront per (token, kv head), or in
// large writes per group of consecutive ones whose loads are all in flight
// together: for head sizes up to 128 lanes 0-31 take K through the norm and
// the rotation and lanes 32-63 pack V beside them, otherwise the wave does K
// and then V.
#include "q8kv_internal.h"
#include "norm_rope_ops.h"
#include "q8_pack.h"
#include "wave_ops.h"

namespace q8kv {
namespace {

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

// Rows of f32 heads, WIDTH lanes per (row, head); block: the workgroup's
// index among those doing rows.
template <int WIDTH>
__device__ __forceinline__ void norm_rope_rows(const NormRopeArgs& a, bool vec4, uint32_t block) {
    constexpr int PER_WAVE = kWave / WIDTH;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t w = lane % WIDTH;
    const uint64_t unit = (static_cast<uint64_t>(block) * (blockDim.x / kWave) + threadIdx.x / kWave) * PER_WAVE +
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
    const float4 y = norm_rope4<WIDTH>(x, w, RowMean(a.head_size), op, a.rot, a.eps);
    if (live && w < hs4) {
        float* o = a.out + static_cast<uint64_t>(t) * a.out_stride + static_cast<uint64_t>(h) * a.head_size + 4 * w;
        if (vec4) *reinterpret_cast<float4*>(o) = y;
        else { o[0] = y.x; o[1] = y.y; o[2] = y.z; o[3] = y.w; }
    }
}

template <int WIDTH>
__global__ __launch_bounds__(256) void norm_rope_kernel(NormRopeArgs a, bool vec4) {
    norm_rope_rows<WIDTH>(a, vec4, blockIdx.x);
}

// Cache write with the norm + rotary step on K: one wave per NP consecutive
// (token, kv head) pairs, every pair's rows and slot loaded before any is
// processed (NP > 1 for large writes, to keep several rows in flight).  With
// SAME_T the NP pairs are heads of one token (NP divides num_kv_heads): one
// slot, one position and one table row serve them all.
template <bool HALF, int NP, bool SAME_T>
__device__ __forceinline__ void norm_rope_write_pairs(const NormRopeCacheWriteArgs& a, bool vec4, uint32_t block) {
    static_assert(SAME_T || NP <= 2, "without SAME_T a wave's pairs may span two tokens at most");
    constexpr int NT = SAME_T ? 1 : NP;                  // tokens per wave
    // Two heads of one token side by side: lanes 0-31 hold head 2j's K (then
    // V) and lanes 32-63 head 2j+1's, so the norm runs once per two K vectors
    // instead of once per K vector beside an idle V half.
    constexpr bool PAIRED = HALF && SAME_T && NP % 2 == 0;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    // Wave-uniform pair indices: the slot and position of a pair are then
    // scalar loads, counted apart from the rows' vector loads, so the table
    // rows can be requested while the rows are still in flight.
    const uint64_t first = (static_cast<uint64_t>(block) * (blockDim.x / kWave) + uniform(threadIdx.x / kWave)) * NP;
    const uint64_t pairs = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads;
    if (first >= pairs) return;
    // One division per wave; the wave's later pairs step through the heads.
    const uint32_t t0 = static_cast<uint32_t>(first / a.num_kv_heads);
    const uint32_t h0 = static_cast<uint32_t>(first - static_cast<uint64_t>(t0) * a.num_kv_heads);
    const uint32_t hs4 = a.head_size / 4, wpt = hs4 + 1;
    float4 xk[NP], xv[NP];
    uint32_t head[NP], tok[NP], slot[NT], posn[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) slot[i] = kPadSlot, posn[i] = 0;
    // The slots come first (wave-uniform scalar loads); a pad token's rows and
    // position are then not read at all, and nothing is written for it.
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        uint32_t t = t0, h = h0 + i;
        if (!SAME_T && h >= a.num_kv_heads) h -= a.num_kv_heads, ++t;
        head[i] = h;
        tok[i] = t;
        if (first + i < pairs && (!SAME_T || i == 0)) slot[SAME_T ? 0 : i] = a.slot_mapping[t];
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        xk[i] = xv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int ti = SAME_T ? 0 : i;
        if (first + i >= pairs || slot[ti] == kPadSlot) continue;    // wave-uniform
        const uint32_t t = tok[i], h = head[i];
        const float* ksrc = a.key + static_cast<uint64_t>(t) * a.key_stride + static_cast<uint64_t>(h) * a.head_size;
        const float* vsrc = a.value + static_cast<uint64_t>(t) * a.value_stride + static_cast<uint64_t>(h) * a.head_size;
        if (PAIRED) {
            // rows loaded below, two heads per instruction
        } else if (HALF) {
            const uint32_t w = lane & 31;
            if (w < hs4) xk[i] = load4((lane >= 32 ? vsrc : ksrc) + 4 * w, vec4);
        } else if (lane < hs4) {
            xk[i] = load4(ksrc + 4 * lane, vec4);
            xv[i] = load4(vsrc + 4 * lane, vec4);
        }
        if ((!SAME_T || i == 0) && a.rot > 0) posn[ti] = a.positions[t];
    }
    if (PAIRED && slot[0] != kPadSlot && (lane & 31) < hs4) {
        // register set j: head h0+2j in lanes 0-31, h0+2j+1 in lanes 32-63; K in xk, V in xv
#pragma unroll
        for (int j = 0; j < NP / 2; ++j) {
            const uint64_t hj = h0 + 2 * j + (lane >> 5);
            xk[j] = load4(a.key + static_cast<uint64_t>(t0) * a.key_stride + hj * a.head_size + 4 * (lane & 31), vec4);
            xv[j] = load4(a.value + static_cast<uint64_t>(t0) * a.value_stride + hj * a.head_size + 4 * (lane & 31), vec4);
        }
    }
    // The table rows of the positions, requested as soon as the positions are
    // in (before the rows), and the norm weight once per wave.
    const uint32_t w = HALF ? (lane & 31) : lane;
    RopeLane op[NT];
    const float4 wt = load_weight4(a.weight, w, hs4, a.params_vec4);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        op[i].wt = wt;
        op[i].c = op[i].s = make_float4(0.f, 0.f, 0.f, 0.f);
        if (slot[i] == kPadSlot || a.rot == 0) continue;
        // positions[t] < num_positions is a caller contract: clamped rather than read out of bounds
        const uint32_t p = posn[i] < a.num_positions ? posn[i] : a.num_positions - 1;
        load_cs4(a.table + static_cast<uint64_t>(p) * a.rot, w, a.rot, a.params_vec4, op[i].c, op[i].s);
    }
    // Cache row of each token: block and offset in it (slots are 32-bit).
    uint32_t blk[NT], off[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        blk[i] = slot[i] / a.block_size;
        off[i] = slot[i] - blk[i] * a.block_size;
    }
    const RowMean mean(a.head_size);
    if (PAIRED) {
        // every pair of the wave is in range (pairs is a multiple of NP) and shares slot[0]
        if (slot[0] == kPadSlot || blk[0] >= a.num_blocks) return;
        const uint32_t hv = head[0] + (lane >> 5);     // this half's head in pair group 0
#pragma unroll
        for (int j = 0; j < NP / 2; ++j) {
            const uint64_t dst = ((static_cast<uint64_t>(blk[0]) * a.num_kv_heads + hv + 2 * j) * a.block_size + off[0]) * wpt;
            const float4 y = norm_rope4<32>(xk[j], w, mean, op[0], a.rot, a.eps);
            pack_vector<32>(y, a.key_cache + dst, hs4, w);
            pack_vector<32>(xv[j], a.value_cache + dst, hs4, w);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int ti = SAME_T ? 0 : i;
        if (first + i >= pairs || slot[ti] == kPadSlot) continue;
        if (blk[ti] >= a.num_blocks) continue;           // out of contract; skipped rather than written out of bounds
        const uint64_t dst = ((static_cast<uint64_t>(blk[ti]) * a.num_kv_heads + head[i]) * a.block_size + off[ti]) * wpt;
        if (HALF) {
            const bool is_v = lane >= 32;
            const float4 y = norm_rope4<32>(xk[i], w, mean, op[ti], a.rot, a.eps);
            pack_vector<32>(is_v ? xk[i] : y, (is_v ? a.value_cache : a.key_cache) + dst, hs4, w);
        } else {
            const float4 y = norm_rope4<64>(xk[i], lane, mean, op[ti], a.rot, a.eps);
            pack_vector<64>(y, a.key_cache + dst, hs4, lane);
            pack_vector<64>(xv[i], a.value_cache + dst, hs4, lane);
        }
    }
}

template <bool HALF, int NP, bool SAME_T>
__global__ __launch_bounds__(256) void norm_rope_cache_write_kernel(NormRopeCacheWriteArgs a, bool vec4) {
    norm_rope_write_pairs<HALF, NP, SAME_T>(a, vec4, blockIdx.x);
}

// q rows and the new K/V rows of a step in one launch: workgroups below
// q_blocks take q (row, head) units, the others one (token, kv head) pair per
// wave.  SMALL: head size up to 128 (32 lanes per q head, K and V side by
// side in the writer).
template <bool SMALL>
__global__ __launch_bounds__(256) void norm_rope_qk_write_kernel(NormRopeArgs q, NormRopeCacheWriteArgs k,
                                                                 uint32_t q_blocks, bool q_vec4, bool k_vec4) {
    if (blockIdx.x < q_blocks) norm_rope_rows<SMALL ? 32 : 64>(q, q_vec4, blockIdx.x);
    else norm_rope_write_pairs<SMALL, 1, true>(k, k_vec4, blockIdx.x - q_blocks);
}

}  // namespace

hipError_t launch_rope_table(float* table, uint32_t num_positions, uint32_t rot, double theta, hipStream_t stream) {
    const uint64_t n = static_cast<uint64_t>(num_positions) * (rot / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream, table,
                       num_positions, rot, theta);
    return hipGetLastError();
}

namespace {
bool rows_vec4(const NormRopeArgs& a) {
    return reinterpret_cast<uintptr_t>(a.x) % 16 == 0 && reinterpret_cast<uintptr_t>(a.out) % 16 == 0 &&
           a.x_stride % 4 == 0 && a.head_stride % 4 == 0 && a.out_stride % 4 == 0;
}
bool pairs_vec4(const NormRopeCacheWriteArgs& a) {
    return reinterpret_cast<uintptr_t>(a.key) % 16 == 0 && reinterpret_cast<uintptr_t>(a.value) % 16 == 0 &&
           a.key_stride % 4 == 0 && a.value_stride % 4 == 0;
}
// workgroups of 4 waves for the q rows: two (row, head) units per wave at
// head sizes up to 128, one above
uint32_t rows_blocks(const NormRopeArgs& a) {
    const uint64_t units = static_cast<uint64_t>(a.num_rows) * a.num_heads;
    const uint64_t waves = a.head_size / 4 <= 32 ? (units + 1) / 2 : units;
    return static_cast<uint32_t>((waves + 3) / 4);
}
}  // namespace

hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t stream) {
    const bool vec4 = rows_vec4(a);
    if (a.head_size / 4 <= 32)
        hipLaunchKernelGGL(norm_rope_kernel<32>, dim3(rows_blocks(a)), dim3(256), 0, stream, a, vec4);
    else
        hipLaunchKernelGGL(norm_rope_kernel<64>, dim3(rows_blocks(a)), dim3(256), 0, stream, a, vec4);
    return hipGetLastError();
}

hipError_t launch_norm_rope_cache_write(const NormRopeCacheWriteArgs& a, hipStream_t stream) {
    const uint64_t pairs = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads;
    const bool vec4 = pairs_vec4(a);
    const bool half = a.head_size / 4 <= 32;
    const uint32_t grid_1 = static_cast<uint32_t>((pairs + 3) / 4);      // one pair per wave
    if (pairs >= kWriteBatchMinPairs && half && a.num_kv_heads % 4 == 0) {
        // Four heads of one token per wave, sharing the slot, position and table row.
        const dim3 grid(static_cast<uint32_t>((pairs + 15) / 16));
        hipLaunchKernelGGL((norm_rope_cache_write_kernel<true, 4, true>), grid, dim3(256), 0, stream, a, vec4);
    } else if (pairs >= kWriteBatchMinPairs) {
        // Two pairs per wave: for head sizes above 128 the registers for four
        // would cut occupancy below 8 waves per SIMD.
        const dim3 grid(static_cast<uint32_t>((pairs + 7) / 8));
        const bool same_t = a.num_kv_heads % 2 == 0;
        if (half && same_t) hipLaunchKernelGGL((norm_rope_cache_write_kernel<true, 2, true>), grid, dim3(256), 0, stream, a, vec4);
        else if (half) hipLaunchKernelGGL((norm_rope_cache_write_kernel<true, 2, false>), grid, dim3(256), 0, stream, a, vec4);
        else if (same_t) hipLaunchKernelGGL((norm_rope_cache_write_kernel<false, 2, true>), grid, dim3(256), 0, stream, a, vec4);
        else hipLaunchKernelGGL((norm_rope_cache_write_kernel<false, 2, false>), grid, dim3(256), 0, stream, a, vec4);
    } else {
        if (half) hipLaunchKernelGGL((norm_rope_cache_write_kernel<true, 1, true>), dim3(grid_1), dim3(256), 0, stream, a, vec4);
        else hipLaunchKernelGGL((norm_rope_cache_write_kernel<false, 1, true>), dim3(grid_1), dim3(256), 0, stream, a, vec4);
    }
    return hipGetLastError();
}

hipError_t launch_norm_rope_qk_cache_write(const NormRopeArgs& q, const NormRopeCacheWriteArgs& k,
                                           hipStream_t stream) {
    const uint64_t pairs = static_cast<uint64_t>(k.num_tokens) * k.num_kv_heads;
    const bool no_q = q.num_rows == 0 || q.num_heads == 0;
    if (pairs >= kWriteBatchMinPairs || no_q || pairs == 0 ||
        (no_q ? 0u : rows_blocks(q)) + (pairs + 3) / 4 > kMaxGridBlocks) {
        // a bulk write keeps its batched kernel; an empty side needs no combined
        // launch; nor does a combination whose grid would pass the launch limit
        if (!no_q) {
            const hipError_t e = launch_norm_rope(q, stream);
            if (e != hipSuccess) return e;
        }
        return pairs ? launch_norm_rope_cache_write(k, stream) : hipSuccess;
    }
    const uint32_t qb = rows_blocks(q);
    const dim3 grid(qb + static_cast<uint32_t>((pairs + 3) / 4));
    if (q.head_size / 4 <= 32)
        hipLaunchKernelGGL(norm_rope_qk_write_kernel<true>, grid, dim3(256), 0, stream, q, k, qb, rows_vec4(q),
                           pairs_vec4(k));
    else
        hipLaunchKernelGGL(norm_rope_qk_write_kernel<false>, grid, dim3(256), 0, stream, q, k, qb, rows_vec4(q),
                           pairs_vec4(k));
    return hipGetLastError();
}

}  // namespace q8kv
