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
//   * Work item = one wavefront for (seq, kv head, up to 8 query heads sharing
//     that kv head, context split).  Each K/V byte is read from HBM once for
//     the whole GQA group.
//   * Positions are processed in chunks of 64.  A chunk of consecutive,
//     64-aligned positions is a run of whole cache tiles (or one 64-row slice
//     of a larger tile): it is fetched with coalesced 16-byte loads into
//     registers one chunk ahead of use, then written to LDS.  Other chunks
//     (visible lists with gaps) are gathered row by row.
//   * Both contractions run on the int8 matrix cores
//     (v_mfma_i32_16x16x64_i8), whose operands include the cache's own codes:
//       q.K^T: each query head's q row is scaled by a power of two and rounded
//       to an integer below 2^30 in magnitude, written as four balanced
//       base-256 digits; the 16 MFMA rows are (4 heads x 4 digits), the
//       columns 16 tokens, k the head dimension.
//       P.V: the softmax weights of a chunk times the V token scales are
//       scaled by a power of two and rounded to integers below 2^29, again as
//       four digits; rows (4 heads x 4 digits), k = 64 tokens, columns 16 head
//       dimensions.  V codes are transposed to token-major bytes with v_perm.
//     The int32 digit sums are exact and are combined exactly in f64; q and
//     the weights keep 30 significant bits, finer than binary32, so the result
//     carries f32-level rounding error only.
//   * Online softmax in the exp2 domain (scale folded with log2 e).  Each
//     MFMA output row group is one head, so the per-head max and sum reduce
//     over the 16 lanes of a DPP row.  Running max, sum and the unnormalized
//     output of each split go to the workspace, and a merge kernel combines
//     the splits (single-split rows are written out directly).
#include "q8kv_internal.h"

namespace q8kv {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kDigitBias = 0x80808080u;

__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Four balanced base-256 digits of a signed integer |n| <= 2^30, one per
// byte, each read back as a signed int8: sum_k byte_k * 256^k == n.
__device__ __forceinline__ uint32_t to_digits(int32_t n) {
    return (static_cast<uint32_t>(n) + kDigitBias) ^ kDigitBias;
}

// Exact value of sum_k d[k] * 256^k for int32 digit sums |d[k]| < 2^22.
__device__ __forceinline__ double combine_digits(i32x4 d) {
    const int32_t d0 = d[0], d1 = d[1], d2 = d[2], d3 = d[3];
    const int32_t lo = d0 + d1 * 256;
    const int32_t hi = d2 + d3 * 256;
    return static_cast<double>(hi) * 65536.0 + static_cast<double>(lo);
}

// v_perm_b32: byte i of the result is byte sel_i of the 8-byte value (a:b),
// selectors 0-3 picking bytes of b and 4-7 bytes of a.
__device__ __forceinline__ uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) {
    return __builtin_amdgcn_perm(a, b, sel);
}

// 4x4 byte transpose: byte b of y[j] = byte j of x[b].
__device__ __forceinline__ void transpose4(const uint32_t x[4], uint32_t y[4]) {
    const uint32_t t01l = perm(x[1], x[0], 0x05010400u);   // x0.0 x1.0 x0.1 x1.1
    const uint32_t t01h = perm(x[1], x[0], 0x07030602u);   // x0.2 x1.2 x0.3 x1.3
    const uint32_t t23l = perm(x[3], x[2], 0x05010400u);
    const uint32_t t23h = perm(x[3], x[2], 0x07030602u);
    y[0] = perm(t23l, t01l, 0x05040100u);
    y[1] = perm(t23l, t01l, 0x07060302u);
    y[2] = perm(t23h, t01h, 0x05040100u);
    y[3] = perm(t23h, t01h, 0x07060302u);
}

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

// Exponent e with |x| < 2^e for finite nonzero x (frexp convention).
__device__ __forceinline__ int exponent_bound(float x) {
    int e = 0;
    (void)frexpf(x, &e);
    return e;
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

// Split-kernel lane roles.  Lane l = 16*g + r.
//   q.K^T (v_mfma_i32_16x16x64_i8): lane (r, g) supplies MFMA row r = (head
//   r/4, digit r%4) of the q digits and column r = token 16*tg + r of the
//   codes, both over the 16 head dimensions 64*kb + 16*g + 0..15, and
//   receives the digit sums of token 16*tg + r for head g.
//   P.V: lane (r, g) supplies row r = (head r/4, digit r%4) of the weight
//   digits and column r of the codes, both over the 16 tokens 4*g + w + 16*b
//   (w, b = 0..3; byte 4*w + b of the operand), where column r of column
//   block cw is dimension 4*NCW*r + 4*cw + j of MFMA j; it receives the digit
//   sums of those dimensions for head g.
//
// Data movement: a chunk of 64 consecutive, 64-aligned positions is a run of
// whole cache tiles (or a 64-row slice of a larger tile), so its K and V rows
// arrive with fully coalesced 16-byte loads (one KiB per instruction) into
// registers, one chunk ahead of use, and are then written to LDS, from where
// each lane reads its MFMA operands.  Chunks of a visible list that are not
// such runs are gathered row by row.  The block ids a chunk needs are read two
// chunks ahead, so no block-table read sits between a data load and its use.
//
// HS4P: code words per row rounded up to 16, 32, 48 or 64; EXACT: head_size /
// 4 == HS4P; NHS: sets of 4 query heads per work item (1 or 2).
template <int HS4P, bool EXACT, int NHS, bool VIS>
__global__ __launch_bounds__(64, (HS4P <= 32 && NHS == 1) ? 2 : 1) void decode_split_kernel(DecodeArgs a, SplitConsts c, uint32_t num_blocks_m1) {
    constexpr int NKB = HS4P / 16;             // 64-dimension k-blocks of q.K^T
    constexpr int NCW = HS4P / 16;             // V code words per lane and row
    constexpr int G = 4 * NHS;
    constexpr int QD = NKB * 64;               // padded q row length
    constexpr int WPT_MAX = HS4P + 1;
    constexpr int NU = (kChunk * WPT_MAX + 4 * kWave - 1) / (4 * kWave);   // 16-byte slots per lane

    __shared__ __align__(16) uint32_t sK[kChunk * WPT_MAX + 64];
    __shared__ __align__(16) uint32_t sV[kChunk * WPT_MAX + 64];
    __shared__ __align__(16) float sQ[G * QD];
    __shared__ __align__(16) uint32_t sA[NHS * 16 * 16];   // [set][head*4+digit][w]: weight digits, 4 tokens a word
    __shared__ int sEq[G];

    const uint32_t lane = threadIdx.x;
    const uint32_t r = lane & 15, g = lane >> 4;
    // Work item = ((s * num_splits + split) * num_kv_heads + kvh) * num_groups + grp:
    // the kv heads of one (seq, split) are dispatched together, so the slices of
    // each cache block that they read reach the memory controllers close in time.
    const uint32_t grp = blockIdx.x % c.num_groups;
    const uint32_t kvh = (blockIdx.x / c.num_groups) % a.num_kv_heads;
    const uint32_t ss = blockIdx.x / c.num_groups / a.num_kv_heads;
    const uint32_t split = ss % c.num_splits;
    const uint32_t s = ss / c.num_splits;
    const uint32_t n_pos = positions_of<VIS>(a, s);
    const uint32_t t0 = split * c.split_tokens;
    if (t0 >= n_pos) return;
    const uint32_t t1 = min(n_pos, t0 + c.split_tokens);
    const uint32_t n_split_s = (n_pos + c.split_tokens - 1) / c.split_tokens;
    const uint32_t n_chunks = (t1 - t0 + kChunk - 1) / kChunk;

    const uint32_t hs = a.head_size, hs4 = EXACT ? HS4P : hs / 4, wpt = hs4 + 1;
    const uint32_t n_rep = a.num_heads / a.num_kv_heads;
    const uint32_t h0 = kvh * n_rep + grp * G;
    const uint32_t nh = min(static_cast<uint32_t>(G), n_rep - grp * G);
    const uint64_t seq_bt = static_cast<uint64_t>(s) * a.max_num_blocks_per_seq;
    const uint64_t kv_stride = static_cast<uint64_t>(a.num_kv_heads) * a.block_size * wpt;  // words per block
    const uint64_t kvh_off = static_cast<uint64_t>(kvh) * a.block_size * wpt;
    const uint32_t chunk_u4 = kChunk * wpt / 4;
    const uint32_t nseg = kChunk / c.seg_rows;            // tile segments per tiled chunk

    // ---- stage q rows (zero for padded dims and absent heads) ----
    for (uint32_t i = lane; i < G * QD; i += kWave) {
        const uint32_t hi = i / QD, d = i % QD;
        float v = 0.0f;
        if (hi < nh && d < hs) v = a.q[static_cast<uint64_t>(s) * a.q_stride + static_cast<uint64_t>(h0 + hi) * hs + d];
        sQ[i] = v;
    }
    __syncthreads();

    // ---- q digits: MFMA row r = (head r/4, digit r%4), k = dims 64kb+16g+0..15 ----
    i32x4 qa[NHS][NKB];
#pragma unroll
    for (int hset = 0; hset < NHS; ++hset) {
        const uint32_t hq = 4 * hset + r / 4, dig = r % 4;
        const float* row = &sQ[hq * QD];
        float amax = 0.0f;
        for (int d = 0; d < QD; d += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + d);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
        const int eq = amax > 0.0f ? 30 - exponent_bound(amax) : 0;    // |q * 2^eq| < 2^30
        if (g == 0 && dig == 0) sEq[hq] = eq;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            uint32_t packed[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float4 v = *reinterpret_cast<const float4*>(row + 64 * kb + 16 * g + 4 * w);
                const uint32_t b0 = (to_digits(static_cast<int32_t>(rintf(ldexpf(v.x, eq)))) >> (8 * dig)) & 0xFFu;
                const uint32_t b1 = (to_digits(static_cast<int32_t>(rintf(ldexpf(v.y, eq)))) >> (8 * dig)) & 0xFFu;
                const uint32_t b2 = (to_digits(static_cast<int32_t>(rintf(ldexpf(v.z, eq)))) >> (8 * dig)) & 0xFFu;
                const uint32_t b3 = (to_digits(static_cast<int32_t>(rintf(ldexpf(v.w, eq)))) >> (8 * dig)) & 0xFFu;
                packed[w] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
            }
            qa[hset][kb] = i32x4{static_cast<int32_t>(packed[0]), static_cast<int32_t>(packed[1]),
                                 static_cast<int32_t>(packed[2]), static_cast<int32_t>(packed[3])};
        }
    }
    __syncthreads();
    int eq_out[NHS];       // q exponent of this lane's output head 4*hset + g
#pragma unroll
    for (int hset = 0; hset < NHS; ++hset) eq_out[hset] = sEq[4 * hset + g];

    // ---- chunk metadata, prepared two chunks ahead ----
    // Tiled chunk: lane k holds the block id of segment k.  Row-gathered chunk:
    // lane i holds the block id and in-block row of the chunk's i-th position.
    struct Meta {
        uint32_t cs, nv, p0, id, row, tiled;
    };
    auto meta_of = [&](uint32_t cs_) __attribute__((always_inline)) -> Meta {
        Meta m;
        m.cs = cs_;
        m.nv = min(static_cast<uint32_t>(kChunk), t1 - cs_);
        m.p0 = position_at<VIS>(a, s, cs_);
        m.tiled = c.tiled_ok;
        if (VIS && m.tiled) {
            const uint32_t pl = position_at<VIS>(a, s, cs_ + m.nv - 1);
            m.tiled = (m.p0 % kChunk == 0) && (pl - m.p0 == m.nv - 1) ? 1u : 0u;
        }
        uint32_t j;
        m.row = 0;
        if (m.tiled) {
            const uint32_t k = min(lane, nseg - 1);
            j = m.p0 / a.block_size + (a.block_size <= kChunk ? k : 0);
        } else {
            const uint32_t pos = position_at<VIS>(a, s, cs_ + min(lane, m.nv - 1));
            j = pos / a.block_size;
            m.row = pos % a.block_size;
        }
        j = j < a.max_num_blocks_per_seq ? j : a.max_num_blocks_per_seq - 1;
        m.id = a.block_tables[seq_bt + j];
        return m;
    };

    // ---- tiled chunk: 16-byte slot u = lane + 64*i lies in segment u / seg_u4 ----
    u32x4 kreg[NU], vreg[NU];
    auto issue_data = [&](const Meta& m) __attribute__((always_inline)) {
        const uint32_t row0 = m.p0 % a.block_size;     // nonzero only when block_size > 64
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const uint32_t u = lane + kWave * i;
            const uint32_t k = __umulhi(u, c.seg_magic);
            uint32_t phys = __shfl(m.id, static_cast<int>(min(k, nseg - 1)), 64);
            phys = phys < num_blocks_m1 ? phys : num_blocks_m1;
            if ((u < chunk_u4) && (k * c.seg_rows < m.nv)) {
                const uint32_t off = (u - k * c.seg_u4) * 4;
                const uint64_t w = phys * kv_stride + kvh_off + static_cast<uint64_t>(row0) * wpt + off;
                kreg[i] = *reinterpret_cast<const u32x4*>(a.key_cache + w);
                vreg[i] = *reinterpret_cast<const u32x4*>(a.value_cache + w);
            }
        }
    };
    auto store = [&](const Meta& m) __attribute__((always_inline)) {
        if (m.tiled) {
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                const uint32_t u = lane + kWave * i;
                if (u < chunk_u4 && __umulhi(u, c.seg_magic) * c.seg_rows < m.nv) {
                    *reinterpret_cast<u32x4*>(&sK[4 * u]) = kreg[i];
                    *reinterpret_cast<u32x4*>(&sV[4 * u]) = vreg[i];
                }
            }
        } else {
            const uint32_t phys = m.id < num_blocks_m1 ? m.id : num_blocks_m1;
            const uint64_t my_row = ((static_cast<uint64_t>(phys) * a.num_kv_heads + kvh) * a.block_size + m.row) * wpt;
            for (uint32_t rr = 0; rr < m.nv; ++rr) {
                const uint32_t lo = __shfl(static_cast<uint32_t>(my_row), rr, 64);
                const uint32_t hi = __shfl(static_cast<uint32_t>(my_row >> 32), rr, 64);
                const uint64_t base = (static_cast<uint64_t>(hi) << 32) | lo;
                for (uint32_t w = lane; w < wpt; w += kWave) {
                    sK[rr * wpt + w] = a.key_cache[base + w];
                    sV[rr * wpt + w] = a.value_cache[base + w];
                }
            }
        }
    };

    // Online-softmax state (log2 units) of head 4*hset + g, uniform across the lane's row.
    float m_run[NHS], l_run[NHS];
    float acc[NHS][NCW][4];      // dims 4*NCW*r + 4*cw + j of head 4*hset + g
#pragma unroll
    for (int hset = 0; hset < NHS; ++hset) {
        m_run[hset] = -INFINITY;
        l_run[hset] = 0.0f;
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[hset][cw][j] = 0.0f;
    }

    // One chunk from LDS: q.K^T, online softmax, P.V.
    auto process = [&](uint32_t nv) __attribute__((always_inline)) {
        // ---- q . K^T ----
        i32x4 dsum[NHS][4];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            const uint32_t* krow = &sK[(16 * tg + r) * wpt + 4 * g];
#pragma unroll
            for (int hset = 0; hset < NHS; ++hset) dsum[hset][tg] = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                i32x4 b;
                if (EXACT) {
                    __builtin_memcpy(&b, krow + 16 * kb, 16);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        b[q] = (16 * kb + 4 * g + q < hs4) ? static_cast<int32_t>(krow[16 * kb + q]) : 0;
                }
#pragma unroll
                for (int hset = 0; hset < NHS; ++hset) dsum[hset][tg] = mfma_i8(qa[hset][kb], b, dsum[hset][tg]);
            }
        }

        // ---- token scales of rows 16*tg + r ----
        float ksc[4], vsc[4];
        bool val[4];
        float vmax = 0.0f;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg) {
            const uint32_t t = 16 * tg + r;
            val[tg] = t < nv;
            ksc[tg] = __uint_as_float(sK[t * wpt + hs4]);
            vsc[tg] = __uint_as_float(sV[t * wpt + hs4]);
            vmax = val[tg] ? fmaxf(vmax, vsc[tg]) : vmax;     // select: unwritten rows never leak
        }
        vmax = row_max(vmax);
        const int ep = 29 - exponent_bound(vmax);             // weight * 2^ep < 2^29

        // ---- online softmax; weights to integers, digits to LDS ----
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset) {
            float z[4];
            float cmax = -INFINITY;
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
                const float zq = ldexpf(static_cast<float>(combine_digits(dsum[hset][tg])), -eq_out[hset]);
                z[tg] = val[tg] ? zq * (ksc[tg] * a.scale_log2) : -INFINITY;
                cmax = fmaxf(cmax, z[tg]);
            }
            const float m_new = fmaxf(m_run[hset], row_max(cmax));
            const float alpha = exp2f(m_run[hset] - m_new);
            float psum = 0.0f;
            uint32_t wd[4];
#pragma unroll
            for (int tg = 0; tg < 4; ++tg) {
                const float p = exp2f(z[tg] - m_new);
                psum += p;
                const float pv = val[tg] ? p * vsc[tg] : 0.0f;
                wd[tg] = to_digits(static_cast<int32_t>(rintf(ldexpf(pv, ep))));
            }
            l_run[hset] = l_run[hset] * alpha + row_sum(psum);
            m_run[hset] = m_new;
            uint32_t td[4];
            transpose4(wd, td);       // byte tg of td[digit] = digit of token r + 16*tg
#pragma unroll
            for (int dg = 0; dg < 4; ++dg) sA[(hset * 16 + 4 * g + dg) * 16 + r] = td[dg];
#pragma unroll
            for (int cw = 0; cw < NCW; ++cw)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[hset][cw][j] *= alpha;
        }
        __syncthreads();

        // ---- P . V ----
        i32x4 pa[NHS];
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset)
            pa[hset] = *reinterpret_cast<const i32x4*>(&sA[(hset * 16 + r) * 16 + 4 * g]);
        const double pscale = ldexp(1.0, -ep);
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) {
            uint32_t bj[4][4];      // [byte j][w]: codes of tokens 4g + w + 16*b (byte b)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t x[4], y[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t word = NCW * r + cw;
                    x[b] = (EXACT || word < hs4) ? sV[(4 * g + w + 16 * b) * wpt + word] : 0u;
                }
                transpose4(x, y);
#pragma unroll
                for (int j = 0; j < 4; ++j) bj[j][w] = y[j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const i32x4 b = i32x4{static_cast<int32_t>(bj[j][0]), static_cast<int32_t>(bj[j][1]),
                                      static_cast<int32_t>(bj[j][2]), static_cast<int32_t>(bj[j][3])};
#pragma unroll
                for (int hset = 0; hset < NHS; ++hset) {
                    const i32x4 d = mfma_i8(pa[hset], b, i32x4{0, 0, 0, 0});
                    acc[hset][cw][j] += static_cast<float>(combine_digits(d) * pscale);
                }
            }
        }
    };

    // ---- pipeline: data one chunk ahead, block ids two chunks ahead ----
    Meta cur = meta_of(t0);
    if (cur.tiled) issue_data(cur);
    Meta nxt = cur;
    if (n_chunks > 1) nxt = meta_of(t0 + kChunk);
    for (uint32_t ci = 0;; ++ci) {
        store(cur);
        const bool more = ci + 1 < n_chunks;
        Meta nxt2 = nxt;
        if (ci + 2 < n_chunks) nxt2 = meta_of(cur.cs + 2 * kChunk);
        if (more && nxt.tiled) issue_data(nxt);
        __syncthreads();
        process(cur.nv);
        if (!more) break;
        __syncthreads();
        cur = nxt;
        nxt = nxt2;
    }

    // ---- write: lane (r, g) holds dims 4*NCW*r + 4*cw + j of head 4*hset + g ----
    const uint64_t row_sh = static_cast<uint64_t>(s) * a.num_heads;
#pragma unroll
    for (int hset = 0; hset < NHS; ++hset) {
        const uint32_t hh = 4 * hset + g;
        if (hh >= nh) continue;
        const uint64_t h = row_sh + h0 + hh;
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) {
            const uint32_t word = NCW * r + cw;
            if (word >= hs4) continue;
            float4 v = make_float4(acc[hset][cw][0], acc[hset][cw][1], acc[hset][cw][2], acc[hset][cw][3]);
            if (n_split_s == 1) {
                const float inv = 1.0f / l_run[hset];
                v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
                *reinterpret_cast<float4*>(a.out + h * hs + 4 * word) = v;
            } else {
                const uint64_t rec = h * c.num_splits + split;
                *reinterpret_cast<float4*>(a.part_acc + rec * hs + 4 * word) = v;
                if (word == 0) {
                    a.part_ml[2 * rec] = m_run[hset];
                    a.part_ml[2 * rec + 1] = l_run[hset];
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

template <int HS4P, bool EXACT, int NHS>
hipError_t launch_split_t(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st, bool vis) {
    if (vis)
        hipLaunchKernelGGL((decode_split_kernel<HS4P, EXACT, NHS, true>), grid, dim3(64), 0, st, a, c, nbm1);
    else
        hipLaunchKernelGGL((decode_split_kernel<HS4P, EXACT, NHS, false>), grid, dim3(64), 0, st, a, c, nbm1);
    return hipGetLastError();
}

template <int HS4P, bool EXACT>
hipError_t launch_split_g(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st, bool vis) {
    if (c.group == 8) return launch_split_t<HS4P, EXACT, 2>(a, c, nbm1, grid, st, vis);
    return launch_split_t<HS4P, EXACT, 1>(a, c, nbm1, grid, st, vis);
}

}  // namespace

DecodePlan plan_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                       uint32_t head_size, uint32_t block_size, uint32_t max_positions) {
    DecodePlan p{};
    const uint32_t n_rep = num_kv_heads ? num_heads / num_kv_heads : 1;
    p.group = n_rep > 4 ? 8 : 4;
    p.num_groups = (n_rep + p.group - 1) / p.group;
    (void)block_size;
    // Aim for about 16 work items per compute unit when every row is at the
    // longest length, with splits of 256..1024 positions (multiples of 64).
    const uint64_t units = static_cast<uint64_t>(num_seqs) * num_kv_heads * p.num_groups;
    const uint64_t target_items = 256ull * 16;
    uint64_t per = units ? (static_cast<uint64_t>(max_positions) * units + target_items - 1) / target_items : max_positions;
    per = (per + kChunk - 1) / kChunk * kChunk;
    if (per < 256) per = 256;
    if (per > 1024) per = 1024;
    if (const char* e = getenv("Q8KV_SPLIT_TOKENS")) {
        const long v = atol(e);
        if (v >= kChunk) per = static_cast<uint64_t>(v) / kChunk * kChunk;
    }
    if (per > kMaxSplit) per = kMaxSplit;
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
        else if (hs4 == 48) err = launch_split_g<48, true>(a, c, nbm1, grid, stream, vis);
        else if (hs4 == 64) err = launch_split_g<64, true>(a, c, nbm1, grid, stream, vis);
        else if (hs4 < 16) err = launch_split_g<16, false>(a, c, nbm1, grid, stream, vis);
        else if (hs4 < 32) err = launch_split_g<32, false>(a, c, nbm1, grid, stream, vis);
        else if (hs4 < 48) err = launch_split_g<48, false>(a, c, nbm1, grid, stream, vis);
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
