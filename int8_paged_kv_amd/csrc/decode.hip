// Single-query decode attention over the int8 paged KV cache.
//
// What is computed follows the "paged_attn_q8.comp" page: for each (seq s,
// query head h), out = softmax(scale * q . K^T) . V over the sequence's
// positions, K and V dequantized on read as code * token_scale, kv head
// h / (num_heads / num_kv_heads), token t at block_tables[s][t / block_size],
// offset t % block_size.  As on that page, the per-token K scale multiplies
// the code dot product and the per-token V scale is folded into the softmax
// weight.  The visible-list mode (the "attention.rs" page's selective split
// decode) attends the listed positions instead of 0 .. context_len - 1.
//
// MI355X design (not the page's one-workgroup-per-(seq, head) three-pass
// shader):
//   * Work item = one wavefront for (seq, kv head, group of G <= 8 query heads
//     sharing that kv head, context split).  Each K/V byte is read from HBM
//     once for the whole GQA group.
//   * Positions are processed in chunks of 64, one per lane.  A chunk of
//     consecutive, 64-aligned positions is a run of whole cache tiles (or one
//     64-row slice of a larger tile): it is fetched with coalesced 16-byte
//     loads into registers one chunk ahead of use, then written to LDS.  Other
//     chunks (visible lists with gaps) are gathered row by row.
//   * q.K^T and P.V run on the matrix cores as f32 MFMA
//     (v_mfma_f32_4x4x1_16b_f32): 16 blocks of 4x4 outer products.  For
//     q.K^T the 4 rows are 4 query heads and the 64 columns (16 blocks x 4) are
//     the chunk's 64 tokens; one MFMA per head dimension.  For P.V the rows are
//     again 4 query heads, each lane owns one code word (4 dimensions, one
//     MFMA per byte) of one token phase.  Codes are converted with one
//     sign-extending byte-select v_cvt_f32_i32 each, and products are exact
//     f32 products accumulated in f32, like a scalar FMA loop.
//   * Online softmax in the exp2 domain (scale folded with log2 e); running
//     max, sum and the unnormalized output of each split are written to the
//     workspace, and a merge kernel combines the splits (single-split rows are
//     written out directly).
#include "q8kv_internal.h"

namespace q8kv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float code_f32(uint32_t word, int byte) {
    return static_cast<float>(static_cast<int8_t>(word >> (8 * byte)));
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// Reductions over the 16 lanes that share (lane % 4): two DPP row rotations
// (within each row of 16 lanes) and the gfx950 row-swap permutes across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// v_permlane{16,32}_swap with both operands = v: the two results hold v with
// rows (16 lanes) exchanged pairwise, so combining them reduces across rows.
// The elements are copied out before the bit cast (a bit cast of a vector
// element expression reads element 0 with this compiler).
__device__ __forceinline__ void swap16(float v, float& x, float& y) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const unsigned a0 = s[0], a1 = s[1];
    x = __uint_as_float(a0);
    y = __uint_as_float(a1);
}
__device__ __forceinline__ void swap32(float v, float& x, float& y) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const unsigned a0 = s[0], a1 = s[1];
    x = __uint_as_float(a0);
    y = __uint_as_float(a1);
}
__device__ __forceinline__ float swap16_max(float v) { float x, y; swap16(v, x, y); return fmaxf(x, y); }
__device__ __forceinline__ float swap32_max(float v) { float x, y; swap32(v, x, y); return fmaxf(x, y); }
__device__ __forceinline__ float swap16_sum(float v) { float x, y; swap16(v, x, y); return x + y; }
__device__ __forceinline__ float swap32_sum(float v) { float x, y; swap32(v, x, y); return x + y; }
__device__ __forceinline__ float group_max(float v) {
    v = fmaxf(v, dpp_mov<kRowRor4>(v));
    v = fmaxf(v, dpp_mov<kRowRor8>(v));
    return swap32_max(swap16_max(v));
}
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_mov<kRowRor4>(v);
    v += dpp_mov<kRowRor8>(v);
    return swap32_sum(swap16_sum(v));
}

struct SplitConsts {
    uint32_t split_tokens, num_splits, group, num_groups;
    uint32_t seg_u4;        // 16-byte units per tile segment in a chunk
    uint32_t seg_magic;     // ceil(2^32 / seg_u4): u / seg_u4 == mulhi(u, magic) for u < 2^16
    uint32_t seg_rows;      // rows per segment = min(block_size, 64)
    uint32_t tiled_ok;      // segment copies are legal (alignment, block_size shape)
};

// Number of positions sequence s attends.
template <bool VIS>
__device__ __forceinline__ uint32_t positions_of(const DecodeArgs& a, uint32_t s) {
    uint32_t n;
    if (VIS) {
        n = a.num_visible[s];
        n = n < a.vis_stride ? n : a.vis_stride;
    } else {
        n = a.context_lens[s];
        n = n < a.max_context_len ? n : a.max_context_len;
        const uint64_t cap = static_cast<uint64_t>(a.max_num_blocks_per_seq) * a.block_size;
        if (n > cap) n = static_cast<uint32_t>(cap);   // defensive: never index past a table row
    }
    return n;
}

template <bool VIS>
__device__ __forceinline__ uint32_t position_at(const DecodeArgs& a, uint32_t s, uint32_t idx) {
    return VIS ? a.visible_pos[static_cast<uint64_t>(s) * a.vis_stride + idx] : idx;
}

// Word offset of the (block, kv head) tile row `row` holding logical position pos.
__device__ __forceinline__ uint64_t row_word_offset(const DecodeArgs& a, uint32_t s, uint32_t kvh,
                                                    uint32_t pos, uint32_t num_blocks_m1, uint32_t wpt) {
    uint32_t j = pos / a.block_size;
    j = j < a.max_num_blocks_per_seq ? j : a.max_num_blocks_per_seq - 1;
    uint32_t phys = a.block_tables[static_cast<uint64_t>(s) * a.max_num_blocks_per_seq + j];
    phys = phys < num_blocks_m1 ? phys : num_blocks_m1;
    return ((static_cast<uint64_t>(phys) * a.num_kv_heads + kvh) * a.block_size + pos % a.block_size) * wpt;
}

// HS4P: code words per row rounded up to 16, 32 or 64 (the lane layout);
// EXACT: head_size/4 == HS4P; G: query heads per work item (4 or 8).
template <int HS4P, bool EXACT, int G, bool VIS>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a, SplitConsts c, uint32_t num_blocks_m1) {
    constexpr int NG4 = G / 4;                 // MFMA head groups of 4
    constexpr int NPH = kWave / HS4P;          // token phases in P.V
    constexpr int WPT_MAX = HS4P + 1;
    constexpr int NU = (kChunk * WPT_MAX + 4 * kWave - 1) / (4 * kWave);   // 16-byte slots per lane

    __shared__ __align__(16) uint32_t sK[kChunk * WPT_MAX + HS4P + 4];
    __shared__ __align__(16) uint32_t sV[kChunk * WPT_MAX + HS4P + 4];
    __shared__ __align__(16) float sQ[G * HS4P * 4];
    __shared__ float sP[kChunk * G];

    const uint32_t lane = threadIdx.x;
    // Work item = ((s * num_kv_heads + kvh) * num_groups + grp) * num_splits + split.
    const uint32_t split = blockIdx.x % c.num_splits;
    const uint32_t sg = blockIdx.x / c.num_splits;
    const uint32_t grp = sg % c.num_groups;
    const uint32_t kvh = (sg / c.num_groups) % a.num_kv_heads;
    const uint32_t s = sg / c.num_groups / a.num_kv_heads;
    const uint32_t n_pos = positions_of<VIS>(a, s);
    const uint32_t t0 = split * c.split_tokens;
    if (t0 >= n_pos) return;
    const uint32_t t1 = min(n_pos, t0 + c.split_tokens);
    const uint32_t n_split_s = (n_pos + c.split_tokens - 1) / c.split_tokens;

    const uint32_t hs = a.head_size, hs4 = EXACT ? HS4P : hs / 4, wpt = hs4 + 1;
    const uint32_t n_rep = a.num_heads / a.num_kv_heads;
    const uint32_t h0 = kvh * n_rep + grp * G;
    const uint32_t nh = min(static_cast<uint32_t>(G), n_rep - grp * G);

    // Stage q rows of the group (zero for padded dims and absent heads).
    for (uint32_t i = lane; i < G * HS4P * 4; i += kWave) {
        const uint32_t hi = i / (HS4P * 4), d = i % (HS4P * 4);
        float v = 0.0f;
        if (hi < nh && d < hs) v = a.q[static_cast<uint64_t>(s) * a.q_stride + static_cast<uint64_t>(h0 + hi) * hs + d];
        sQ[i] = v;
    }

    // Per-lane 16-byte slot map of a tiled chunk (chunk independent).
    const uint32_t chunk_u4 = kChunk * wpt / 4;
    uint32_t slot_seg[NU], slot_off[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const uint32_t u = lane + kWave * i;
        const uint32_t k = __umulhi(u, c.seg_magic);
        slot_seg[i] = k;
        slot_off[i] = (u - k * c.seg_u4) * 4;
    }

    const uint64_t kv_stride = static_cast<uint64_t>(a.num_kv_heads) * a.block_size * wpt;  // words per block
    const uint64_t kvh_off = static_cast<uint64_t>(kvh) * a.block_size * wpt;
    const uint64_t seq_bt = static_cast<uint64_t>(s) * a.max_num_blocks_per_seq;

    u32x4 kreg[NU], vreg[NU];

    // Is the chunk starting at list index cs a run of consecutive positions
    // from a 64-aligned first position (so it maps onto whole tile segments)?
    auto chunk_tiled = [&](uint32_t cs, uint32_t nv) __attribute__((always_inline)) -> bool {
        if (!c.tiled_ok) return false;
        if (!VIS) return true;
        const uint32_t p0 = position_at<VIS>(a, s, cs);
        const uint32_t pl = position_at<VIS>(a, s, cs + nv - 1);
        return (p0 % kChunk == 0) && (pl - p0 == nv - 1);
    };
    auto issue_tiled = [&](uint32_t cs, uint32_t nv) __attribute__((always_inline)) {
        const uint32_t p0 = position_at<VIS>(a, s, cs);
        const uint32_t blk0 = p0 / a.block_size;
        const uint32_t row0 = p0 % a.block_size;     // nonzero only when block_size > 64
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const uint32_t u = lane + kWave * i;
            const uint32_t k = slot_seg[i];
            const bool live = (u < chunk_u4) && (k * c.seg_rows < nv);
            if (live) {
                uint32_t j = blk0 + (a.block_size <= kChunk ? k : 0);
                j = j < a.max_num_blocks_per_seq ? j : a.max_num_blocks_per_seq - 1;
                uint32_t phys = a.block_tables[seq_bt + j];
                phys = phys < num_blocks_m1 ? phys : num_blocks_m1;
                const uint64_t w = phys * kv_stride + kvh_off + static_cast<uint64_t>(row0) * wpt + slot_off[i];
                kreg[i] = *reinterpret_cast<const u32x4*>(a.key_cache + w);
                vreg[i] = *reinterpret_cast<const u32x4*>(a.value_cache + w);
            }
        }
    };
    auto store_tiled = [&](uint32_t nv) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const uint32_t u = lane + kWave * i;
            if (u < chunk_u4 && slot_seg[i] * c.seg_rows < nv) {
                *reinterpret_cast<u32x4*>(&sK[4 * u]) = kreg[i];
                *reinterpret_cast<u32x4*>(&sV[4 * u]) = vreg[i];
            }
        }
    };
    auto copy_rows = [&](uint32_t cs, uint32_t nv) __attribute__((always_inline)) {
        uint64_t my_row = 0;
        if (lane < nv) my_row = row_word_offset(a, s, kvh, position_at<VIS>(a, s, cs + lane), num_blocks_m1, wpt);
        for (uint32_t r = 0; r < nv; ++r) {
            const uint32_t lo = __shfl(static_cast<uint32_t>(my_row), r, 64);
            const uint32_t hi = __shfl(static_cast<uint32_t>(my_row >> 32), r, 64);
            const uint64_t base = (static_cast<uint64_t>(hi) << 32) | lo;
            for (uint32_t w = lane; w < wpt; w += kWave) {
                sK[r * wpt + w] = a.key_cache[base + w];
                sV[r * wpt + w] = a.value_cache[base + w];
            }
        }
    };

    // Online-softmax state (log2 units) of head 4g + (lane % 4), one entry per MFMA head group.
    float m_run[NG4], l_run[NG4];
#pragma unroll
    for (int g = 0; g < NG4; ++g) { m_run[g] = -INFINITY; l_run[g] = 0.0f; }
    f32x4 acc[NG4][4];
#pragma unroll
    for (int g = 0; g < NG4; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint32_t m4 = lane & 3;            // MFMA row owned by this lane (head within 4)
    const uint32_t pw = lane % HS4P;          // P.V: code word owned by this lane
    const uint32_t ph = lane / HS4P;          // P.V: token phase

    uint32_t cs = t0;
    uint32_t nv = min(static_cast<uint32_t>(kChunk), t1 - cs);
    bool tiled = chunk_tiled(cs, nv);
    if (tiled) issue_tiled(cs, nv);

    while (true) {
        // ---- land this chunk in LDS, prefetch the next one ----
        if (tiled) store_tiled(nv);
        else copy_rows(cs, nv);
        const uint32_t ncs = cs + kChunk;
        const bool more = ncs < t1;
        uint32_t nnv = 0;
        bool ntiled = false;
        if (more) {
            nnv = min(static_cast<uint32_t>(kChunk), t1 - ncs);
            ntiled = chunk_tiled(ncs, nnv);
            if (ntiled) issue_tiled(ncs, nnv);
        }
        __syncthreads();

        // ---- q . K^T on MFMA: A = codes (lane 4b+i: token 4b+i), B = q (lane
        // 4b+n: head 4g+n).  Lane 4b+n ends with the logits of tokens 4b..4b+3
        // for head 4g+n.  Two accumulators (even / odd words) halve the
        // dependent MFMA chain. ----
        f32x4 dot[NG4], dot1[NG4];
#pragma unroll
        for (int g = 0; g < NG4; ++g) { dot[g] = f32x4{0.f, 0.f, 0.f, 0.f}; dot1[g] = dot[g]; }
        const int qk_pairs = (EXACT ? HS4P : static_cast<int>(hs4)) / 2;
#pragma unroll 2
        for (int w2 = 0; w2 < qk_pairs; ++w2) {
            const int w = 2 * w2;
            const uint32_t kw0 = sK[lane * wpt + w];
            const uint32_t kw1 = sK[lane * wpt + w + 1];
#pragma unroll
            for (int g = 0; g < NG4; ++g) {
                const float4 qa = *reinterpret_cast<const float4*>(&sQ[((4 * g + m4) * HS4P + w) * 4]);
                const float4 qb = *reinterpret_cast<const float4*>(&sQ[((4 * g + m4) * HS4P + w + 1) * 4]);
                dot[g] = mfma4(code_f32(kw0, 0), qa.x, dot[g]);
                dot1[g] = mfma4(code_f32(kw1, 0), qb.x, dot1[g]);
                dot[g] = mfma4(code_f32(kw0, 1), qa.y, dot[g]);
                dot1[g] = mfma4(code_f32(kw1, 1), qb.y, dot1[g]);
                dot[g] = mfma4(code_f32(kw0, 2), qa.z, dot[g]);
                dot1[g] = mfma4(code_f32(kw1, 2), qb.z, dot1[g]);
                dot[g] = mfma4(code_f32(kw0, 3), qa.w, dot[g]);
                dot1[g] = mfma4(code_f32(kw1, 3), qb.w, dot1[g]);
            }
        }
        if (!EXACT && (hs4 & 1)) {
            const uint32_t w = hs4 - 1;
            const uint32_t kw0 = sK[lane * wpt + w];
#pragma unroll
            for (int g = 0; g < NG4; ++g) {
                const float4 qa = *reinterpret_cast<const float4*>(&sQ[((4 * g + m4) * HS4P + w) * 4]);
                dot[g] = mfma4(code_f32(kw0, 0), qa.x, dot[g]);
                dot[g] = mfma4(code_f32(kw0, 1), qa.y, dot[g]);
                dot[g] = mfma4(code_f32(kw0, 2), qa.z, dot[g]);
                dot[g] = mfma4(code_f32(kw0, 3), qa.w, dot[g]);
            }
        }

        // ---- online softmax: this lane's head is 4g+m4, its tokens 4*blk+i ----
        const uint32_t blk = lane >> 2;
        float zk[4], vsc[4];
        bool val[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t t = 4 * blk + i;
            val[i] = t < nv;
            zk[i] = __uint_as_float(sK[t * wpt + hs4]) * a.scale_log2;
            vsc[i] = __uint_as_float(sV[t * wpt + hs4]);
        }
#pragma unroll
        for (int g = 0; g < NG4; ++g) {
            const f32x4 d = dot[g] + dot1[g];
            float z[4];
            float cmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[i] = val[i] ? d[i] * zk[i] : -INFINITY;   // select: poison rows never leak
                cmax = fmaxf(cmax, z[i]);
            }
            const float m_new = fmaxf(m_run[g], group_max(cmax));
            const float alpha = exp2f(m_run[g] - m_new);
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = exp2f(z[i] - m_new);
                psum += p;
                sP[(4 * blk + i) * G + 4 * g + m4] = val[i] ? p * vsc[i] : 0.0f;
            }
            l_run[g] = l_run[g] * alpha + group_sum(psum);
            m_run[g] = m_new;
            // P.V accumulators hold all four heads of the group: rescale head i
            // by the factor computed in lanes with m4 == i.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), i));
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[g][j][i] *= ai;
            }
        }
        __syncthreads();

        // ---- P . V: lane owns word pw of the tokens of phase ph ----
#pragma unroll 4
        for (int k = 0; k < HS4P; ++k) {
            const uint32_t tok = k * NPH + ph;
            const uint32_t vw = sV[tok * wpt + pw];
            const float c0 = code_f32(vw, 0), c1 = code_f32(vw, 1), c2 = code_f32(vw, 2), c3 = code_f32(vw, 3);
#pragma unroll
            for (int g = 0; g < NG4; ++g) {
                const float pa = sP[tok * G + 4 * g + m4];
                acc[g][0] = mfma4(pa, c0, acc[g][0]);
                acc[g][1] = mfma4(pa, c1, acc[g][1]);
                acc[g][2] = mfma4(pa, c2, acc[g][2]);
                acc[g][3] = mfma4(pa, c3, acc[g][3]);
            }
        }
        if (!more) break;
        __syncthreads();
        cs = ncs;
        nv = nnv;
        tiled = ntiled;
    }

    // ---- combine token phases: lanes with equal pw hold partial sums ----
#pragma unroll
    for (int off = HS4P; off < kWave; off <<= 1)
#pragma unroll
        for (int g = 0; g < NG4; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[g][j][i] += __shfl_xor(acc[g][j][i], off, 64);

    // m and l of head 4g+i live in lanes with lane % 4 == i.
    float mh[G], lh[G];
#pragma unroll
    for (int g = 0; g < NG4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mh[4 * g + i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_run[g]), i));
            lh[4 * g + i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_run[g]), i));
        }
    if (ph != 0 || pw >= hs4) return;
    const uint64_t row_sh = static_cast<uint64_t>(s) * a.num_heads;
#pragma unroll
    for (int g = 0; g < NG4; ++g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t hh = 4 * g + i;
            if (hh >= nh) continue;
            const uint64_t h = row_sh + h0 + hh;
            float4 v = make_float4(acc[g][0][i], acc[g][1][i], acc[g][2][i], acc[g][3][i]);
            if (n_split_s == 1) {
                const float inv = 1.0f / lh[hh];
                v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
                *reinterpret_cast<float4*>(a.out + h * hs + 4 * pw) = v;
            } else {
                const uint64_t rec = h * c.num_splits + split;
                *reinterpret_cast<float4*>(a.part_acc + rec * hs + 4 * pw) = v;
                if (pw == 0) {
                    a.part_ml[2 * rec] = mh[hh];
                    a.part_ml[2 * rec + 1] = lh[hh];
                }
            }
        }
    }
}

// One wavefront per (seq, head): combine the split partials of rows with more
// than one split, write zero rows for empty position sets.
template <bool VIS>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a, uint32_t split_tokens, uint32_t num_splits) {
    const uint32_t lane = threadIdx.x;
    const uint32_t s = blockIdx.x / a.num_heads;
    const uint64_t h = blockIdx.x;   // s * num_heads + head
    const uint32_t n_pos = positions_of<VIS>(a, s);
    const uint32_t ns = (n_pos + split_tokens - 1) / split_tokens;
    if (ns == 1) return;
    const uint32_t hs = a.head_size;
    float* o = a.out + h * hs;
    if (ns == 0) {
        for (uint32_t d = lane; d < hs; d += kWave) o[d] = 0.0f;
        return;
    }
    const float* ml = a.part_ml + 2 * h * num_splits;
    float M = -INFINITY;
    for (uint32_t i = 0; i < ns; ++i) M = fmaxf(M, ml[2 * i]);
    float L = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const bool act = 4 * lane < hs;
    for (uint32_t i = 0; i < ns; ++i) {
        const float w = exp2f(ml[2 * i] - M);
        L += w * ml[2 * i + 1];
        if (act) {
            const float4 v = *reinterpret_cast<const float4*>(a.part_acc + (h * num_splits + i) * hs + 4 * lane);
            acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
        }
    }
    if (act) {
        const float inv = 1.0f / L;
        *reinterpret_cast<float4*>(o + 4 * lane) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
}

template <int HS4P, bool EXACT, int G>
hipError_t launch_split_t(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st, bool vis) {
    if (vis)
        hipLaunchKernelGGL((decode_split_kernel<HS4P, EXACT, G, true>), grid, dim3(64), 0, st, a, c, nbm1);
    else
        hipLaunchKernelGGL((decode_split_kernel<HS4P, EXACT, G, false>), grid, dim3(64), 0, st, a, c, nbm1);
    return hipGetLastError();
}

template <int HS4P, bool EXACT>
hipError_t launch_split_g(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st, bool vis) {
    if (c.group == 8) return launch_split_t<HS4P, EXACT, 8>(a, c, nbm1, grid, st, vis);
    return launch_split_t<HS4P, EXACT, 4>(a, c, nbm1, grid, st, vis);
}

}  // namespace

DecodePlan plan_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                       uint32_t head_size, uint32_t block_size, uint32_t max_positions) {
    DecodePlan p{};
    const uint32_t n_rep = num_kv_heads ? num_heads / num_kv_heads : 1;
    p.group = n_rep > 4 ? 8 : 4;
    p.num_groups = (n_rep + p.group - 1) / p.group;
    (void)block_size;
    // Aim for about 8 work items per compute unit when every row is at the
    // longest length, with splits of 256..1024 positions (multiples of 64).
    const uint64_t units = static_cast<uint64_t>(num_seqs) * num_kv_heads * p.num_groups;
    const uint64_t target_items = 256ull * 8;
    uint64_t per = units ? (static_cast<uint64_t>(max_positions) * units + target_items - 1) / target_items : max_positions;
    per = (per + kChunk - 1) / kChunk * kChunk;
    if (per < 256) per = 256;
    if (per > 1024) per = 1024;
    if (const char* e = getenv("Q8KV_SPLIT_TOKENS")) {
        const long v = atol(e);
        if (v >= kChunk) per = static_cast<uint64_t>(v) / kChunk * kChunk;
    }
    p.split_tokens = static_cast<uint32_t>(per);
    p.num_splits = max_positions ? (max_positions + p.split_tokens - 1) / p.split_tokens : 0;
    const uint64_t recs = static_cast<uint64_t>(num_seqs) * num_heads * p.num_splits;
    p.acc_offset = 0;
    p.ml_offset = (recs * head_size * sizeof(float) + 255) / 256 * 256;
    p.bytes = p.num_splits > 1 ? p.ml_offset + recs * 2 * sizeof(float) : 0;
    return p;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
    const bool vis = a.visible_pos != nullptr;
    const uint32_t hs4 = a.head_size / 4;
    const uint32_t wpt = hs4 + 1;
    SplitConsts c{};
    c.split_tokens = p.split_tokens;
    c.num_splits = p.num_splits;
    c.group = p.group;
    c.num_groups = p.num_groups;
    c.seg_rows = a.block_size < static_cast<uint32_t>(kChunk) ? a.block_size : kChunk;
    const bool shape_ok = a.block_size % 4 == 0 &&
                          (kChunk % a.block_size == 0 || a.block_size % kChunk == 0);
    const bool align_ok = reinterpret_cast<uintptr_t>(a.key_cache) % 16 == 0 &&
                          reinterpret_cast<uintptr_t>(a.value_cache) % 16 == 0;
    c.tiled_ok = shape_ok && align_ok;
    c.seg_u4 = c.seg_rows * wpt / 4;
    if (c.seg_u4 == 0) c.seg_u4 = 1;
    c.seg_magic = static_cast<uint32_t>((0x100000000ull + c.seg_u4 - 1) / c.seg_u4);
    const uint32_t nbm1 = a.num_blocks - 1;
    if (p.num_splits > 0) {
        const uint64_t items = static_cast<uint64_t>(a.num_seqs) * a.num_kv_heads * p.num_groups * p.num_splits;
        const dim3 grid(static_cast<uint32_t>(items));
        hipError_t err;
        if (hs4 == 16) err = launch_split_g<16, true>(a, c, nbm1, grid, stream, vis);
        else if (hs4 == 32) err = launch_split_g<32, true>(a, c, nbm1, grid, stream, vis);
        else if (hs4 == 64) err = launch_split_g<64, true>(a, c, nbm1, grid, stream, vis);
        else if (hs4 < 16) err = launch_split_g<16, false>(a, c, nbm1, grid, stream, vis);
        else if (hs4 < 32) err = launch_split_g<32, false>(a, c, nbm1, grid, stream, vis);
        else err = launch_split_g<64, false>(a, c, nbm1, grid, stream, vis);
        if (err != hipSuccess) return err;
    }
    const uint32_t st = p.split_tokens ? p.split_tokens : 1;
    const dim3 mgrid(a.num_seqs * a.num_heads);
    if (vis)
        hipLaunchKernelGGL(decode_merge_kernel<true>, mgrid, dim3(64), 0, stream, a, st, p.num_splits);
    else
        hipLaunchKernelGGL(decode_merge_kernel<false>, mgrid, dim3(64), 0, stream, a, st, p.num_splits);
    return hipGetLastError();
}

}  // namespace q8kv
