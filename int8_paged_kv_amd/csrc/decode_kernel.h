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
//   * Positions are processed in chunks of 32 or 64.  For one row group (kv
//     head, up to 16 of its query heads; in multi-row decode, up to 16 (row,
//     head) pairs) the chunks of all sequences form one sequence of C chunks, and a
//     fixed number of persistent wavefronts per row group each take an equal
//     contiguous range of it, weighted by cost (a chunk, plus the fixed work
//     of each nonempty sequence).  This is the split-context idea of the
//     "attention.rs" page, balanced over the whole batch instead of per
//     sequence.  A wave that covers a whole sequence writes its output
//     directly; otherwise it writes a softmax partial (running max, sum,
//     unnormalized output) with device-coherent stores, and the last wave to
//     arrive for that sequence combines the partials.  Wavefronts are numbered
//     kv head fastest, so the kv-head slices of the same cache blocks are
//     requested together.  Each K/V byte is read once per row group.
//   * A chunk of CH (32 or 64) consecutive, CH-aligned positions is a run of
//     whole cache tiles (or one CH-row slice of a larger tile), fetched one
//     chunk ahead with coalesced 16-byte loads: at head sizes up to 128
//     straight into one of two LDS buffers (LDS-direct loads), otherwise into
//     registers and then LDS.  Visible lists with gaps are gathered row by
//     row.  32-position chunks (one set of 4 query heads, up to 128
//     dimensions) let two workgroups share a compute unit.
//   * Both contractions run on the int8 matrix cores
//     (v_mfma_i32_16x16x64_i8), whose operands include the cache's own codes:
//       q.K^T: each query head's q row is scaled by a power of two and rounded
//       to an integer below 2^30 in magnitude, written as four balanced
//       base-256 digits; the 16 MFMA rows are (4 heads x 4 digits), the
//       columns 16 tokens, k the head dimension.
//       P.V: the softmax weights of a chunk times the V token scales are
//       scaled by a power of two and rounded to integers below 2^29, again as
//       four digits; rows (4 heads x 4 digits), k = 64 tokens (a 32-position
//       chunk fills half with zero weights), columns 16 head dimensions.  V
//       codes are transposed to token-major bytes with v_perm.
//     The int32 digit sums are exact; they are combined in binary32 with a
//     single rounding per step, so q and the weights keep about 30
//     significant bits and the result carries f32-level rounding error only.
//   * Online softmax in the exp2 domain (scale folded with log2 e).  Each
//     MFMA output row group is one head, so the per-head max and sum reduce
//     over the 16 lanes of a DPP row.
#pragma once
#include "bounds.h"
#include "decode_split.h"
#include "norm_rope_ops.h"
#include "q8_pack.h"
#include "wave_ops.h"

namespace q8kv {
namespace {


typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kDigitBias = 0x80808080u;

// Cost units that split a row group's work evenly among its waves: a chunk,
// and a sequence's start (its q digits, the output or partial record of the
// previous sequence, the append of the step's new row).  Per-wave stamps on
// the Llama-shaped batch: with 64-position chunks a start costs about 1.8
// chunks of wave time; with 32-position chunks a weight of 1.5 chunks gave
// the shortest launch (weights of 1 to 2 chunks timed).
constexpr uint32_t kCostChunk = 4;
constexpr uint32_t cost_seq(int ch) { return ch == 64 ? 7u : 6u; }

__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Four balanced base-256 digits of a signed integer |n| <= 2^30, one per
// byte, each read back as a signed int8: sum_k byte_k * 256^k == n.
__device__ __forceinline__ uint32_t to_digits(int32_t n) {
    return (static_cast<uint32_t>(n) + kDigitBias) ^ kDigitBias;
}

// sum_k d[k] * 256^k for int32 digit sums |d[k]| < 2^22, rounded to binary32:
// the two halves are exact int32 values; each conversion and the final fma
// round once, so the result is within 2^-23 relative of the exact sum.
__device__ __forceinline__ float combine_digits(i32x4 d) {
    const int32_t lo = d[0] + d[1] * 256;
    const int32_t hi = d[2] + d[3] * 256;
    return fmaf(static_cast<float>(hi), 65536.0f, static_cast<float>(lo));
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

// Exponent e with |x| < 2^e for finite nonzero x (frexp convention).
__device__ __forceinline__ int exponent_bound(float x) {
    int e = 0;
    (void)frexpf(x, &e);
    return e;
}

// Number of positions sequence s attends (in multi-row decode, its last row);
// in dense mode *len (when given) receives context_lens[s] itself.
template <bool VIS>
__device__ __forceinline__ uint32_t positions_of(const DecodeArgs& a, uint32_t s, uint32_t* len = nullptr) {
    uint32_t n;
    if (VIS) {
        n = a.num_visible[s];
        bounds_report(a.bounds_flags, n > a.vis_stride, kBoundVisible);
        n = n < a.vis_stride ? n : a.vis_stride;
    } else {
        n = a.context_lens[s];
        if (len) *len = n;
        n = n < a.max_context_len ? n : a.max_context_len;
        const uint64_t cap = static_cast<uint64_t>(a.max_num_blocks_per_seq) * a.block_size;
        bounds_report(a.bounds_flags, n > cap, kBoundTable);
        if (n > cap) n = static_cast<uint32_t>(cap);   // defensive: never index past a table row
    }
    return n;
}

template <bool VIS, int CH>
__device__ __forceinline__ uint32_t chunks_of(const DecodeArgs& a, uint32_t s) {
    return (positions_of<VIS>(a, s) + CH - 1) / CH;
}

template <bool VIS>
__device__ __forceinline__ uint32_t position_at(const DecodeArgs& a, uint32_t s, uint32_t idx) {
    return VIS ? a.visible_pos[static_cast<uint64_t>(s) * a.vis_stride + idx] : idx;
}

// Device-coherent (agent scope, "sc1") 16- and 8-byte accesses for the
// partial records handed between wavefronts that may run on different XCDs:
// they bypass the XCD's non-coherent L2 copies, so no whole-cache write-back
// or invalidation is needed.  A record is laid out in lane order, so each
// store or load instruction covers whole contiguous lines.  The loads wait
// for their own completion inside the same asm block.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void coherent_store4(float* p, f32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void coherent_store2(float* p, f32x2 v) {
    asm volatile("global_store_dwordx2 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
// Byte offset of an LDS location (the value M0 takes for LDS-direct loads).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}
// LDS-direct 16-byte load: lane l's 16 bytes at g land at LDS byte lds + 16*l.
// The compiler does not see these loads: the caller waits for them with
// wait_vmem() before reading the LDS they fill.
__device__ __forceinline__ void load_lds16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(g), "s"(lds) : "memory", "m0");
}
// A load through the scalar data cache from a wave-uniform address of data no
// kernel writes during the launch (read only: nothing is stored that way).
__device__ __forceinline__ uint32_t scalar_load(const uint32_t* p) {
    typedef const __attribute__((address_space(4))) uint32_t* ConstPtr;
    return *(ConstPtr)p;     // (a C-style cast: the only one that changes address space)
}
// Waits for every outstanding vector memory operation of the wavefront.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }
// Device-coherent loads the compiler tracks (relaxed agent-scope atomic
// loads of 8 bytes compile to sc1 loads): a 16-byte unit as two halves, and an
// 8-byte (max, sum) pair.
__device__ __forceinline__ f32x4 coherent_load4(const float* p) {
    uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(p));
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float(static_cast<uint32_t>(lo)), __uint_as_float(static_cast<uint32_t>(lo >> 32)),
                 __uint_as_float(static_cast<uint32_t>(hi)), __uint_as_float(static_cast<uint32_t>(hi >> 32))};
}
__device__ __forceinline__ f32x2 coherent_load2(const float* p) {
    const uint64_t x = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return f32x2{__uint_as_float(static_cast<uint32_t>(x)), __uint_as_float(static_cast<uint32_t>(x >> 32))};
}

// Query heads of a row group: pairs p = (row p / n_rep, head kvh*n_rep +
// p % n_rep) of a sequence's rows (one row except in multi-row decode) and the
// kv head's query heads.  Output row (a row of [rows, num_heads, head_size])
// of pair p of sequence s.
__device__ __forceinline__ uint64_t pair_out_row(const DecodeArgs& a, uint32_t s, uint32_t kvh, uint32_t n_rep,
                                                 uint32_t nrow, uint32_t p) {
    return (static_cast<uint64_t>(s) * nrow + p / n_rep) * a.num_heads + kvh * n_rep + p % n_rep;
}

// Zero output rows of sequences [s_begin, s_end) for pairs p0 .. p0+np-1.
__device__ void zero_rows(const DecodeArgs& a, uint32_t lane, uint32_t s_begin, uint32_t s_end, uint32_t kvh,
                          uint32_t n_rep, uint32_t nrow, uint32_t p0, uint32_t np) {
    const uint32_t hs4 = a.head_size / 4;
    for (uint32_t s = s_begin; s < s_end; ++s)
        for (uint32_t p = lane; p < np * hs4; p += kWave) {
            const uint64_t row = pair_out_row(a, s, kvh, n_rep, nrow, p0 + p / hs4);
            *reinterpret_cast<float4*>(a.out + row * a.head_size + 4 * (p % hs4)) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
}

// Chunk sequence of one row group: the chunks of sequence 0, then sequence 1,
// ...  Wave-uniform results.
//   chunk_totals: total chunk count C and the chunks of sequences before s.
template <bool VIS, int CH>
__device__ void chunk_totals(const DecodeArgs& a, uint32_t lane, uint32_t s, uint32_t& total, uint32_t& before) {
    total = 0;
    before = 0;
    for (uint32_t b = 0; b < a.num_seqs; b += kWave) {
        const uint32_t t = b + lane;
        const uint32_t nc = t < a.num_seqs ? chunks_of<VIS, CH>(a, t) : 0u;
        const uint32_t incl = wave_incl_scan(nc, lane);
        const uint32_t wt = lane_value(incl, kWave - 1);
        if (s >= b + kWave) before += wt;
        else if (s > b) before += lane_value(incl, s - b - 1);
        total += wt;
    }
}

//   locate_chunk: the sequence holding chunk x (x < C) and the chunks before it.
template <bool VIS, int CH>
__device__ void locate_chunk(const DecodeArgs& a, uint32_t lane, uint32_t x, uint32_t& row, uint32_t& before) {
    uint32_t base = 0;
    row = a.num_seqs;
    before = 0;
    for (uint32_t b = 0; b < a.num_seqs; b += kWave) {
        const uint32_t t = b + lane;
        const uint32_t nc = t < a.num_seqs ? chunks_of<VIS, CH>(a, t) : 0u;
        const uint32_t incl = wave_incl_scan(nc, lane);
        const uint32_t wt = lane_value(incl, kWave - 1);
        if (x < base + wt) {
            const uint64_t m = __ballot(base + incl > x);
            const uint32_t l = static_cast<uint32_t>(__builtin_ctzll(m));
            row = b + l;
            before = base + lane_value(incl - nc, l);
            return;
        }
        base += wt;
    }
}

// Shares of a row group's U cost units among its W waves.  Waves j < H weigh
// kShareOld and the others kShareYoung: with two workgroups per compute unit,
// the second half of the grid is the second workgroup on each CU, whose
// waves start behind the first ones (their first loads queue behind those
// waves' tile loads) and are issued second on their SIMDs; per-wave stamps
// show them finishing about 7% later on equal shares.  Wave j covers units
// [floor(P(j)*U/T), floor(P(j+1)*U/T)) with P(j) = kShareOld*min(j, H) +
// kShareYoung*max(j - H, 0) and T = P(W); H >= W gives equal shares.
constexpr uint32_t kShareOld = 23, kShareYoung = 21;
struct Shares {
    uint32_t W, H, U;
    uint64_t T;
    __device__ __forceinline__ uint64_t P(uint32_t j) const {
        return static_cast<uint64_t>(kShareOld) * min(j, H) + static_cast<uint64_t>(kShareYoung) * (j > H ? j - H : 0u);
    }
    __device__ __forceinline__ uint32_t bound(uint32_t j) const { return static_cast<uint32_t>(P(j) * U / T); }
    // the wave whose range holds unit x: the largest j with bound(j) <= x
    __device__ __forceinline__ uint32_t wave_of(uint32_t x) const {
        const uint64_t A = (static_cast<uint64_t>(x) + 1) * T;
        const uint64_t oldU = static_cast<uint64_t>(kShareOld) * H * U;
        const uint64_t j = A <= oldU ? (A - 1) / (static_cast<uint64_t>(kShareOld) * U)
                                     : H + (A - oldU - 1) / (static_cast<uint64_t>(kShareYoung) * U);
        return static_cast<uint32_t>(j < W - 1 ? j : W - 1);
    }
};

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
// HS4P: code words per row rounded up to 16, 32, 48 or 64; EXACT: head_size /
// 4 == HS4P; NHS: sets of 4 query heads per wavefront (1, 2 or 4); VIS: visible
// list positions; TILED: every chunk is known to be a tile run (dense
// positions, aligned caches, block_size dividing or a multiple of 64); SEGR:
// when nonzero (16 or 32, with EXACT), the rows per tile segment, for which
// each segment of a chunk fills whole 64-lane slots (SEGR*HS4P/256 of them)
// plus SEGR/4 trailing 16-byte units: every full slot then loads from one
// segment with a scalar base address and a fixed per-lane offset.  NR: the
// decode step with the per-head RMSNorm + partial rotary step (head_size 64,
// 128 or 256, dense positions): q rows and the new K row are normalized and
// rotated at the sequence's last position as they are staged, as the
// standalone norm + rotary kernels do it.
template <int HS4P, bool EXACT, int NHS, bool VIS, bool TILED, int SEGR, int CH, bool NR = false>
__global__ __launch_bounds__(kWave * kWavesPerGroup, (HS4P <= 32 && (SEGR == 0 || CH == 32)) ? 2 : 1) void decode_split_kernel(DecodeArgs a, SplitConsts c, uint32_t num_blocks_m1) {
    constexpr int NKB = HS4P / 16;             // 64-dimension k-blocks of q.K^T
    constexpr int NCW = HS4P / 16;             // V code words per lane and row
    constexpr int G = 4 * NHS;
    constexpr uint64_t kRecFloats = static_cast<uint64_t>(NHS) * NCW * kWave * 4;   // floats per partial record (= G * 4 * HS4P)
    constexpr int QD = NKB * 64;               // padded q row length
    constexpr int WPT_MAX = HS4P + 1;
    constexpr int NTG = CH / 16;               // 16-token column groups of a chunk
    constexpr uint32_t kCostSeq = cost_seq(CH);
    static_assert(CH == 32 || CH == 64, "chunk size");
    static_assert(!NR || ((HS4P == 16 || HS4P == 32 || HS4P == 64) && EXACT && !VIS),
                  "norm + rotary step: 16, 32 or 64 lanes per q head, dense positions");
    constexpr int NU = (CH * WPT_MAX + 4 * kWave - 1) / (4 * kWave);   // 16-byte slots per lane
    // An exact head size makes a chunk CH*(HS4P+1) words: CH*HS4P/256 full
    // 16-byte slots per lane plus a 4-byte tail slot in CH lanes.
    constexpr int NF = EXACT ? CH * HS4P / 256 : NU;
    constexpr bool FAST = SEGR > 0;
    static_assert(!FAST || (EXACT && (SEGR * HS4P) % 256 == 0 && SEGR <= CH), "segment layout");
    static_assert(!EXACT || (CH * HS4P) % 256 == 0, "exact layout");
    // Segment loads go straight to LDS (no register staging), double-buffered:
    // the next chunk lands in one buffer while the other is processed.  Two
    // buffers of K and V fit for up to 32 code words per row.
    constexpr bool DMA = FAST && HS4P <= 32;
    constexpr int NBUF = DMA ? 2 : 1;
    constexpr int FSEG = FAST ? CH / SEGR : 1;              // segments per chunk
    constexpr int FS = FAST ? SEGR * HS4P / 256 : 0;         // full slots per segment (FSEG * FS == NF)
    constexpr int FLO = FAST ? SEGR / 4 : 1;                 // trailing 16-byte units per segment
    constexpr int SEG_U4 = FAST ? SEGR * (HS4P + 1) / 4 : 1; // 16-byte units per segment
    constexpr uint32_t NTAIL = FAST ? FSEG * FLO : 0;         // lanes holding the segments' trailing units (CH/4)
    struct Buf {
        u32x4 k[DMA ? 1 : NF], v[DMA ? 1 : NF];
        uint32_t kt, vt;        // EXACT generic layout: one 4-byte tail slot per lane
        u32x4 k4, v4;           // FAST layout: the segments' trailing units (lanes below NTAIL)
    };

    // Per-wavefront LDS regions: the wavefronts of a workgroup are independent.
    // Segment layouts fill a chunk's CH*(HS4P+1) words exactly; the others
    // use whole 64-lane slots.
    constexpr int BUFW = FAST ? CH * (HS4P + 1) : NU * 4 * kWave;
    __shared__ __align__(16) uint32_t sK_[kWavesPerGroup][NBUF][BUFW];   // also q-digit scratch at sequence changes
    __shared__ __align__(16) uint32_t sV_[kWavesPerGroup][NBUF][BUFW];
    __shared__ __align__(16) uint32_t sA_[kWavesPerGroup][NHS * 16 * 16];    // [set][head*4+digit][w]: weight digits; q maxima
    __shared__ int sEq_[kWavesPerGroup][G];
    // q-digit scratch of its own (LDS-direct loads, one set of 4 heads: it fits
    // the budget there), so that a sequence change can form the new q digits
    // while the next chunk's loads are already in flight; elsewhere the next
    // chunk's buffer serves, before those loads are issued.
    constexpr bool QSCR = DMA && NHS == 1;
    constexpr int QSCR_WORDS = NHS * NKB * 256;      // digits; the per-slot maxima go to sA
    __shared__ __align__(16) uint32_t sQs_[kWavesPerGroup][QSCR ? QSCR_WORDS : 1];
    const uint32_t wid = uniform(threadIdx.x / kWave);
    // sK/sV: the tiles of the chunk being processed; sKn/sVn: where the next
    // chunk's segments land (the same buffer without LDS-direct loads).
    uint32_t* sK = sK_[wid][0];
    uint32_t* sV = sV_[wid][0];
    uint32_t* sKn = sK_[wid][NBUF - 1];
    uint32_t* sVn = sV_[wid][NBUF - 1];
    uint32_t* const sA = sA_[wid];
    int* const sEq = sEq_[wid];

    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t r = lane & 15, g = lane >> 4;
    // Workgroups are dispatched to the XCDs in turn (workgroup b to XCD
    // b mod 8).  Within each span (the first and the second workgroup of
    // every CU), workgroup numbers are regrouped so that consecutive ones run
    // on one XCD: the row groups of the same chunk range (adjacent kv heads'
    // tiles of the same blocks, which share lines at the tile edges) then
    // meet in one L2.
    uint32_t bl = blockIdx.x;
    if (c.xcd_span) {
        const uint32_t span0 = bl - bl % c.xcd_span, b = bl % c.xcd_span;
        bl = span0 + (b % kXcds) * (c.xcd_span / kXcds) + b / kXcds;
    }
    const uint32_t gw = bl * kWavesPerGroup + wid;      // persistent wavefront index
    if (gw >= c.num_rg * c.waves_per_rg) return;
    const uint32_t rg = gw % c.num_rg;
    const uint32_t j = gw / c.num_rg;
    // The row groups of one kv head are adjacent: with several (multi-row
    // decode, or more query heads than a group holds), their waves for the
    // same range j share a workgroup, hence a CU and an L2, and read the same
    // tiles at about the same time.
    const uint32_t ngrp = c.num_rg / a.num_kv_heads;
    const uint32_t kvh = rg / ngrp;
    const uint32_t grp = rg % ngrp;

    // ---- this wave's chunk range [x0, x1) of the row group's chunk sequence ----
    // The waves split the row group's work into equal contiguous ranges of
    // cost units.  A chunk costs kCostChunk units; starting a new sequence
    // inside a range (closing the previous sequence's piece, forming the new
    // q) costs kCostSeq more, measured.  With up to 64 sequences and at least
    // kCostChunk + kCostSeq units per wave (the widest gap between two chunks'
    // cost indices) the units are weighted so; otherwise they are the chunks
    // alone.  Every range then holds at least one chunk.
    // Up to 64 sequences: one load and one scan give every sequence's chunk
    // count and offsets, kept in lane s.
    const bool one_window = a.num_seqs <= static_cast<uint32_t>(kWave);
    const bool append = !VIS && a.new_key != nullptr;     // decode step: append, then attend
    uint32_t C, U, win_np = 0, win_nc = 0, win_incl = 0, win_cinc = 0, win_len = 0;
    bool weighted = false;
    uint32_t ua = 1;      // cost units of a chunk (kCostChunk when weighted)
    if (one_window) {
        win_np = lane < a.num_seqs ? positions_of<VIS>(a, lane) : 0u;
        if ((append || a.rows_per_seq > 1) && lane < a.num_seqs) win_len = a.context_lens[lane];
        win_nc = (win_np + CH - 1) / CH;
        win_incl = wave_incl_scan(win_nc, lane);
        C = uniform(lane_value(win_incl, kWave - 1));
        const uint64_t ne = __ballot(win_np > 0);
        const uint32_t sne = static_cast<uint32_t>(__builtin_popcountll(ne));
        const uint64_t uw = static_cast<uint64_t>(kCostChunk) * C + static_cast<uint64_t>(kCostSeq) * sne;
        // every share, the smallest included, must span the widest gap
        // between two chunks' cost indices
        const Shares sh{c.waves_per_rg, min(c.young_from, c.waves_per_rg), 1u, 0u};
        weighted = uw * kShareYoung >= static_cast<uint64_t>(kCostChunk + kCostSeq) * sh.P(c.waves_per_rg) &&
                   uw < (1ull << 31);
        ua = weighted ? kCostChunk : 1u;
        U = weighted ? static_cast<uint32_t>(uw) : C;
        const uint64_t upto = lane == kWave - 1 ? ~0ull : (2ull << lane) - 1;
        win_cinc = ua * win_incl + (weighted ? kCostSeq * static_cast<uint32_t>(__builtin_popcountll(ne & upto)) : 0u);
    } else {
        uint32_t unused;
        chunk_totals<VIS, CH>(a, lane, 0, C, unused);
        C = uniform(C);
        U = C;
    }
    const uint32_t W = weighted ? c.waves_per_rg : min(c.waves_per_rg, C);
    // unequal shares only with cost weighting (the chunk-count split needs a
    // chunk in every share)
    Shares shares{W, weighted ? min(c.young_from, W) : W, U, 0u};
    shares.T = shares.P(W);
    const uint32_t n_rep = a.num_heads / a.num_kv_heads;
    // Multi-row decode: the nrow rows of a sequence share its K/V reads; the
    // row group's query heads are (row, head) pairs h0 .. h0+nh-1.
    const uint32_t nrow = a.rows_per_seq > 1 ? a.rows_per_seq : 1u;
    const uint32_t h0 = grp * G;
    const uint32_t nh = min(static_cast<uint32_t>(G), nrow * n_rep - grp * G);
    auto zero_seqs = [&](uint32_t s_begin, uint32_t s_end) __attribute__((always_inline)) {
        zero_rows(a, lane, s_begin, s_end, kvh, n_rep, nrow, h0, nh);
    };
    if (j >= W) {
        if (C == 0 && j == 0) zero_seqs(0, a.num_seqs);
        return;
    }
    // First chunk whose cost index is at least u (u < U, and when weighted
    // u <= U - kCostChunk - kCostSeq, as every range bound is), its sequence,
    // the chunks before that sequence and its positions.  Cost index of chunk
    // i of sequence s: the units of the sequences before s, plus kCostSeq when
    // weighted, plus ua*i.  Its sequence is the first whose last chunk's cost
    // index (its cumulative units minus ua) reaches u.
    auto chunk_at_cost = [&](uint32_t u, uint32_t& s_out, uint32_t& before_out, uint32_t& np_out) __attribute__((always_inline)) -> uint32_t {
        if (one_window) {
            const uint32_t l = static_cast<uint32_t>(__builtin_ctzll(__ballot(win_cinc > u + ua - 1)));
            s_out = l;
            before_out = lane_value(win_incl - win_nc, l);
            np_out = lane_value(win_np, l);
            const uint32_t cf = lane_value(win_cinc - ua * win_nc, l);     // cost index of its first chunk
            return before_out + (u > cf ? (u - cf + ua - 1) / ua : 0u);
        }
        locate_chunk<VIS, CH>(a, lane, u, s_out, before_out);
        np_out = 0;
        return u;
    };
    const uint32_t lo = uniform(shares.bound(j));
    const uint32_t hi = uniform(shares.bound(j + 1));
    uint32_t s0, p0c, np0, s1, p1c, np1;
    const uint32_t x0 = uniform(chunk_at_cost(lo, s0, p0c, np0));
    const uint32_t x1 = hi >= U ? C : uniform(chunk_at_cost(hi, s1, p1c, np1));
    const uint32_t n = x1 - x0;
    if (uniform(s0) >= a.num_seqs || n == 0) return;    // unreachable: every range holds a chunk
    // Cost index of the first chunk of the sequence at cursor state (s, before).
    auto first_cost = [&](uint32_t s_, uint32_t before_) __attribute__((always_inline)) -> uint32_t {
        return one_window ? lane_value(win_cinc - ua * win_nc, s_) : before_;
    };

    const uint32_t hs = a.head_size, hs4 = EXACT ? HS4P : hs / 4, wpt = hs4 + 1;
    // In segment layouts a block is exactly one tile segment (block_size ==
    // SEGR), so its size and the segment rows are compile-time constants.
    const uint32_t bsz = FAST ? static_cast<uint32_t>(SEGR) : a.block_size;
    const uint32_t segr = FAST ? static_cast<uint32_t>(SEGR) : c.seg_rows;
    const uint64_t kv_stride = static_cast<uint64_t>(a.num_kv_heads) * bsz * wpt;  // words per block
    const uint64_t kvh_off = static_cast<uint64_t>(kvh) * bsz * wpt;
    const uint32_t chunk_u4 = CH * wpt / 4;
    const uint32_t nseg = CH / segr;                  // tile segments per tiled chunk

    // ---- cursor over the chunk sequence (wave-uniform) ----
    struct Cursor {
        uint32_t s, ci, npos, before;    // sequence, chunk index in it, its positions, chunks before it
        uint32_t jf, nrec;               // first wave sharing the sequence, and their number
        uint32_t len;                    // norm + rotary step without one window: context_lens[s]
    };
    Cursor cur{uniform(s0), 0, 0, uniform(p0c), 0, 0, 0};
    cur.ci = x0 - cur.before;
    // Positions of the cursor's sequence (with one load window, from a lane).
    // The norm + rotary step also keeps the context length from the same
    // read, so its q position, append test and multi-row limits need no read
    // of their own (each would stall the wave on its round trip); the other
    // instantiations read it where they need it (one register fewer across
    // the loop, measurably faster at the headline shape).
    auto load_seq = [&](uint32_t s_) __attribute__((always_inline)) {
        if (one_window) {
            cur.npos = lane_value(win_np, s_);
        } else if constexpr (NR) {
            uint32_t raw = 0;
            cur.npos = uniform(positions_of<VIS>(a, s_, &raw));
            cur.len = uniform(raw);
        } else {
            cur.npos = uniform(positions_of<VIS>(a, s_));
        }
    };
    if (one_window) cur.npos = uniform(np0);
    else load_seq(cur.s);
    auto share = [&]() __attribute__((always_inline)) {
        const uint32_t cf = first_cost(cur.s, cur.before);
        cur.jf = shares.wave_of(cf);
        cur.nrec = shares.wave_of(cf + ua * ((cur.npos + CH - 1) / CH - 1)) - cur.jf + 1;
    };
    share();
    // Sequences with no positions get zero rows.  Each is written by exactly
    // one wave of the row group: the one whose range it falls inside, wave 0
    // for those before the first chunk, the last wave for those after it.
    auto advance = [&]() __attribute__((always_inline)) {
        ++cur.ci;
        if (cur.ci * CH >= cur.npos) {
            cur.before += (cur.npos + CH - 1) / CH;
            cur.ci = 0;
            while (true) {
                ++cur.s;
                if constexpr (NR) {
                    if (cur.s >= a.num_seqs) cur.npos = static_cast<uint32_t>(CH);
                    else load_seq(cur.s);
                } else {
                    cur.npos = cur.s >= a.num_seqs ? static_cast<uint32_t>(CH)
                               : one_window ? lane_value(win_np, cur.s)
                                            : uniform(positions_of<VIS>(a, cur.s));
                }
                if (cur.npos != 0) break;
                zero_seqs(cur.s, cur.s + 1);
            }
            if (cur.s < a.num_seqs) share();
        }
    };
    // A range that starts a sequence zeroes the empty sequences just before
    // it (those after the previous non-empty one); empty sequences between two
    // sequences of one range are zeroed as the cursor passes them, and those
    // after the last chunk by the last wave.
    if (cur.ci == 0) {
        uint32_t first;
        if (one_window) {
            const uint64_t below = cur.s >= 64u ? ~0ull : ((1ull << cur.s) - 1);
            const uint64_t ne = __ballot(win_np > 0) & below;
            first = ne ? 64u - static_cast<uint32_t>(__builtin_clzll(ne)) : 0u;
        } else {
            first = cur.s;
            while (first > 0 && uniform(positions_of<VIS>(a, first - 1)) == 0) --first;
        }
        if (first < cur.s) zero_seqs(first, cur.s);
    }

    // ---- chunk metadata (uniform except the block id of segment `lane`) ----
    // info: bits 0-6 valid positions (0 for a chunk past the wave's range),
    // bit 7 tiled chunk, bits 8-31 the number of waves whose ranges share the
    // sequence (1: it lies wholly in this wave's range); jf: the first of them.
    struct Meta {
        uint32_t s, cs, p0, info, jf, id;
        uint32_t app;            // decode step: the chunk's last row is its sequence's new token
        uint32_t lr;             // multi-row decode: context_lens[s] - cs (row b sees lr - (nrow-1-b) of the chunk)
        uint32_t len;            // norm + rotary step: context_lens[s]
    };
    auto meta_nv = [](const Meta& m) __attribute__((always_inline)) { return m.info & 0x7Fu; };
    auto meta_tiled = [](const Meta& m) __attribute__((always_inline)) { return TILED || (m.info & 0x80u) != 0; };
    auto meta_nrec = [](const Meta& m) __attribute__((always_inline)) { return m.info >> 8; };
    // Visible lists: the first and last listed position of 64 consecutive
    // chunks of one sequence, lane l holding chunk vc_c0 + l, loaded in one
    // round trip when the cursor leaves the cached span; a chunk's bounds are
    // then read from a lane instead of two dependent loads per chunk.
    uint32_t vc_s = ~0u, vc_c0 = 0, vc_first = 0, vc_last = 0;
    auto vis_bounds = [&](uint32_t s_, uint32_t ci, uint32_t npos, uint32_t& p0, uint32_t& pl)
        __attribute__((always_inline)) {
        if (s_ != vc_s || ci < vc_c0 || ci - vc_c0 >= static_cast<uint32_t>(kWave)) {
            vc_s = s_;
            vc_c0 = ci;
            const uint32_t cl = ci + lane;
            const uint64_t row = static_cast<uint64_t>(s_) * a.vis_stride;
            const bool in = static_cast<uint64_t>(cl) * CH < npos;
            const uint32_t f = in ? cl * CH : 0u;
            const uint32_t l = in ? min(cl * CH + CH - 1, npos - 1) : 0u;
            vc_first = a.visible_pos[row + f];
            vc_last = a.visible_pos[row + l];
        }
        p0 = lane_value(vc_first, ci - vc_c0);
        pl = lane_value(vc_last, ci - vc_c0);
    };
    auto meta_of = [&](bool live, bool first = false) __attribute__((always_inline)) -> Meta {
        Meta m;
        m.s = cur.s;
        m.cs = cur.ci * CH;
        const uint32_t nv = live ? min(static_cast<uint32_t>(CH), cur.npos - m.cs) : 0u;
        uint32_t pl = 0;
        if (VIS) vis_bounds(m.s, cur.ci, cur.npos, m.p0, pl);
        else m.p0 = m.cs;
        uint32_t tiled = 1;
        if (!TILED) {
            tiled = c.tiled_ok;
            // ascending distinct positions from a 64-aligned p0 to p0 + nv - 1
            // are exactly the tile rows p0 .. p0 + nv - 1
            if (VIS && tiled && nv > 0) tiled = (m.p0 % CH == 0) && (pl - m.p0 == nv - 1) ? 1u : 0u;
        }
        m.jf = cur.jf;
        m.info = nv | (tiled << 7) | (cur.nrec << 8);
        // The new token sits at position context_lens[s]-1, the sequence's last
        // attended position when it is not clamped.
        m.lr = 0;
        auto seq_len = [&]() __attribute__((always_inline)) -> uint32_t {
            if (one_window) return lane_value(win_len, m.s);
            return NR ? cur.len : uniform(a.context_lens[m.s]);
        };
        if constexpr (NR) m.len = seq_len();
        if (nrow > 1 && nv > 0) m.lr = seq_len() - m.cs;
        m.app = 0;
        if (append && nv > 0 && m.cs + nv == cur.npos) {
            m.app = seq_len() == cur.npos ? 1u : 0u;
        }
        const uint32_t k = min(lane, nseg - 1);
        uint32_t jb = m.p0 / bsz + (bsz <= static_cast<uint32_t>(CH) ? k : 0u);
        // a segment holding attended positions (its first row below nv)
        const bool used = lane < nseg && k * segr < nv;
        bounds_report(a.bounds_flags, used && jb >= a.max_num_blocks_per_seq, kBoundTable);
        jb = jb < a.max_num_blocks_per_seq ? jb : a.max_num_blocks_per_seq - 1;
        if (first && nseg <= 2) {
            // The first chunk's (at most two) block ids as scalar loads: they
            // skip the vector-memory queue, where the tile loads the CU's
            // other waves have already issued sit ahead of them.
            const uint64_t row = static_cast<uint64_t>(m.s) * a.max_num_blocks_per_seq;
            const uint32_t j0 = uniform(lane_value(jb, 0)), j1 = uniform(lane_value(jb, 1));
            const uint32_t id0 = scalar_load(a.block_tables + row + j0);
            const uint32_t id1 = scalar_load(a.block_tables + row + j1);
            m.id = lane == 0 ? id0 : id1;
        } else {
            m.id = a.block_tables[static_cast<uint64_t>(m.s) * a.max_num_blocks_per_seq + jb];
        }
#ifdef Q8_DEBUG_BOUNDS
        bounds_report(a.bounds_flags, used && (tiled != 0) && m.id > num_blocks_m1, kBoundBlock);
        if (VIS && nv > 0 && tiled) {
            // a tile run must be exactly the listed positions p0 .. p0 + nv - 1
            const uint32_t pl_ = position_at<VIS>(a, m.s, m.cs + min(lane, nv - 1));
            bounds_report(a.bounds_flags, lane < nv && pl_ != m.p0 + lane, kBoundVisible);
        }
#endif
        return m;
    };

    // ---- tiled chunk loads: 16-byte slot u = lane + 64*i lies in segment u / seg_u4 ----
    auto issue_data = [&](const Meta& m, Buf& b, uint32_t* dK, uint32_t* dV) __attribute__((always_inline)) {
        if (FAST) {
            // Segment k's tile (block id from lane k) starts at a uniform
            // address; an invalid segment reads the cache's first bytes.
            const bool ok = meta_tiled(m);
            const uint32_t nv = meta_nv(m);
            const char* kb[FSEG];
            const char* vb[FSEG];
#pragma unroll
            for (int k = 0; k < FSEG; ++k) {
                uint32_t ph = lane_value(m.id, k);
                ph = ph < num_blocks_m1 ? ph : num_blocks_m1;
                const bool valid = ok && static_cast<uint32_t>(k * SEGR) < nv;
                const uint64_t off = valid ? static_cast<uint64_t>(ph) * kv_stride + kvh_off : 0;
                kb[k] = reinterpret_cast<const char*>(a.key_cache + off);
                vb[k] = reinterpret_cast<const char*>(a.value_cache + off);
            }
            const uint32_t lb = lane * 16;
            if (DMA && nv == 0) return;   // past the range: nothing is stored from this chunk
            if (DMA) {
                const uint32_t lk = lds_offset(dK), lv = lds_offset(dV);
#pragma unroll
                for (int k = 0; k < FSEG; ++k)
#pragma unroll
                    for (int f = 0; f < FS; ++f) {
                        const uint32_t o = (k * SEG_U4 + f * 64) * 16;
                        load_lds16(kb[k] + lb + f * 1024, lk + o);
                        load_lds16(vb[k] + lb + f * 1024, lv + o);
                    }
            } else {
#pragma unroll
                for (int k = 0; k < FSEG; ++k)
#pragma unroll
                    for (int f = 0; f < FS; ++f) {
                        b.k[k * FS + f] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb[k] + lb + f * 1024));
                        b.v[k * FS + f] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb[k] + lb + f * 1024));
                    }
            }
            // Trailing units: lane l < NTAIL takes unit l % FLO of segment l / FLO.
            const uint32_t kk = lane / FLO;
            const char* pk = reinterpret_cast<const char*>(a.key_cache);
            const char* pv = reinterpret_cast<const char*>(a.value_cache);
#pragma unroll
            for (int k = 0; k < FSEG; ++k)
                if (kk == static_cast<uint32_t>(k)) { pk = kb[k]; pv = vb[k]; }
            const uint32_t tb = (lane < NTAIL) ? (FS * 64 + lane % FLO) * 16 : lb;
            b.k4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pk + tb));
            b.v4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pv + tb));
            return;
        }
        if (!TILED && !c.tiled_ok) return;     // no tile loads at all (caches not 16-byte aligned, odd block_size)
        const uint32_t row0 = m.p0 % bsz;              // nonzero only when block_size > 64
        const bool ok = meta_tiled(m);
        const uint32_t nv = meta_nv(m);
        const uint64_t base = kvh_off + static_cast<uint64_t>(row0) * wpt;
        // Recompute the slot geometry per chunk (a few VALU ops) rather than
        // keeping it live across the loop.
        uint32_t ln = lane;
        asm volatile("" : "+v"(ln));
        // All block-id exchanges first (one LDS round trip), then the loads.
        // An invalid slot's word offset is masked to 0, so it reads the
        // cache's first line: branch-free, in bounds, and one cached line.
        constexpr int NS = NF + (EXACT ? 1 : 0);
        uint32_t kseg[NS], phys[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const uint32_t u = (i < NF) ? ln + kWave * i : (4 * kWave * NF + ln) >> 2;
            kseg[i] = __umulhi(u, c.seg_magic);
            phys[i] = __shfl(m.id, static_cast<int>(min(kseg[i], nseg - 1)), 64);
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const uint32_t k = kseg[i];
            const uint32_t ph = phys[i] < num_blocks_m1 ? phys[i] : num_blocks_m1;
            uint64_t w;
            bool valid;
            if (i < NF) {
                const uint32_t u = ln + kWave * i;
                valid = ok && (EXACT || u < chunk_u4) && (k * segr < nv);
                w = ph * kv_stride + base + (u - k * c.seg_u4) * 4;
            } else {
                const uint32_t wi = 4 * kWave * NF + ln;
                valid = ok && (k * segr < nv);
                w = ph * kv_stride + base + (wi - 4 * k * c.seg_u4);
            }
            w &= 0ull - static_cast<uint64_t>(valid);
            if (i < NF) {
                b.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.key_cache + w));
                b.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.value_cache + w));
            } else {
                b.kt = __builtin_nontemporal_load(a.key_cache + w);
                b.vt = __builtin_nontemporal_load(a.value_cache + w);
            }
        }
    };
    // ---- decode step: the new token's K and V rows, staged one chunk ahead ----
    // Lane w < head_size/4 holds elements 4w .. 4w+3.  Quantized in the chunk's
    // step exactly as the cache writer does, they replace the row the tile
    // loads brought in (the cache still held the old one) and, for the first
    // query-head group of the kv head, are written to the caches.
    float4 nkx = make_float4(0.f, 0.f, 0.f, 0.f), nvx = nkx;
    // Norm + rotary step: the table row of a position (clamped to the table);
    // the staged q rows' weights and cos/sin (q_op, at the position of their
    // sequence's last row); the new K row's weights for lane w = lane (64-lane
    // group), staged with it.
    auto nr_row = [&](uint32_t pos) __attribute__((always_inline)) -> const float* {
        if (a.nr_rot == 0) return a.nr_table;
        const uint32_t p = pos < a.nr_num_positions ? pos : a.nr_num_positions - 1;
        return a.nr_table + static_cast<uint64_t>(p) * a.nr_rot;
    };
    RopeLane q_op{};
    float4 nk_wt = make_float4(0.f, 0.f, 0.f, 0.f);
    auto issue_new = [&](const Meta& m) __attribute__((always_inline)) {
        if (!append || !m.app) return;
        nkx = make_float4(0.f, 0.f, 0.f, 0.f);
        nvx = nkx;
        if constexpr (NR) nk_wt = load_weight4(a.nr_k_weight, lane, hs4, a.nr_params_vec4 != 0);
        if (lane < hs4) {
            const float* pk = a.new_key + static_cast<uint64_t>(m.s) * a.new_key_stride + static_cast<uint64_t>(kvh) * hs + 4 * lane;
            const float* pv = a.new_value + static_cast<uint64_t>(m.s) * a.new_value_stride + static_cast<uint64_t>(kvh) * hs + 4 * lane;
            if (a.new_vec4) {
                nkx = *reinterpret_cast<const float4*>(pk);
                nvx = *reinterpret_cast<const float4*>(pv);
            } else {
                nkx = make_float4(pk[0], pk[1], pk[2], pk[3]);
                nvx = make_float4(pv[0], pv[1], pv[2], pv[3]);
            }
        }
    };
    auto store_new = [&](const Meta& m) __attribute__((always_inline)) {
        if (!append || !m.app) return;
        // The appended row sits at the q rows' position, context_lens[s] - 1,
        // and the staged q rows are still this sequence's (the next
        // sequence's are staged after this store), so their cos/sin serve:
        // rotated lanes lie below 2 * (rot / 8) <= HS4P, where the q lane
        // w = lane % HS4P equals lane.  Lanes at and above head_size/4 hold
        // zeros and weight 0: they add nothing to the sum of squares and stay 0.
        if constexpr (NR)
            nkx = norm_rope4<kWave>(nkx, lane, RowMean(hs), RopeLane{nk_wt, q_op.c, q_op.s}, a.nr_rot, a.nr_eps);
        uint32_t ks, vs;
        const uint32_t kw = quantize_word<kWave>(nkx, ks);
        const uint32_t vw = quantize_word<kWave>(nvx, vs);
        const uint32_t row = (meta_nv(m) - 1) * wpt;
        if (lane < hs4) { sK[row + lane] = kw; sV[row + lane] = vw; }
        if (lane == 0) { sK[row + hs4] = ks; sV[row + hs4] = vs; }
        if (grp == 0) {
            const uint32_t pos = m.cs + meta_nv(m) - 1;
            // When blocks and chunks nest (a block size dividing the chunk, or
            // a multiple of it), the row's block id is the one its chunk's
            // segment was read with (lane k of m.id holds segment k's): no new
            // load.  Otherwise it is read from the table.
            const uint32_t bs = bsz;
            const bool nested = bs <= static_cast<uint32_t>(CH) ? CH % bs == 0 : bs % CH == 0;
            const uint32_t blk = nested ? lane_value(m.id, bs <= static_cast<uint32_t>(CH) ? (meta_nv(m) - 1) / bs : 0u)
                                        : uniform(a.block_tables[static_cast<uint64_t>(m.s) * a.max_num_blocks_per_seq +
                                                                 pos / bs]);
            // An out-of-range block id breaks the caller contract: nothing is
            // written for it (a clamped id would overwrite another block's row).
            bounds_report(a.bounds_flags, lane == 0 && blk > num_blocks_m1, kBoundBlock);
            if (blk > num_blocks_m1) return;
            const uint64_t dst = ((static_cast<uint64_t>(blk) * a.num_kv_heads + kvh) * bsz + pos % bsz) * wpt;
            if (lane < hs4) { a.key_cache_w[dst + lane] = kw; a.value_cache_w[dst + lane] = vw; }
            if (lane == 0) { a.key_cache_w[dst + hs4] = ks; a.value_cache_w[dst + hs4] = vs; }
        }
    };

    auto store = [&](const Meta& m, const Buf& b) __attribute__((always_inline)) {
        if (DMA) wait_vmem();           // this chunk's LDS-direct segment loads have landed
        if (FAST && meta_tiled(m)) {
            if (!DMA) {
#pragma unroll
                for (int k = 0; k < FSEG; ++k)
#pragma unroll
                    for (int f = 0; f < FS; ++f) {
                        const uint32_t u = k * SEG_U4 + f * 64 + lane;
                        *reinterpret_cast<u32x4*>(&sK[4 * u]) = b.k[k * FS + f];
                        *reinterpret_cast<u32x4*>(&sV[4 * u]) = b.v[k * FS + f];
                    }
            }
            if (lane < NTAIL) {
                const uint32_t u = (lane / FLO) * SEG_U4 + FS * 64 + lane % FLO;
                *reinterpret_cast<u32x4*>(&sK[4 * u]) = b.k4;
                *reinterpret_cast<u32x4*>(&sV[4 * u]) = b.v4;
            }
        } else if (meta_tiled(m)) {
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                const uint32_t u = lane + kWave * i;
                *reinterpret_cast<u32x4*>(&sK[4 * u]) = b.k[i];
                *reinterpret_cast<u32x4*>(&sV[4 * u]) = b.v[i];
            }
            if (EXACT) {
                sK[4 * kWave * NF + lane] = b.kt;
                sV[4 * kWave * NF + lane] = b.vt;
            }
        } else {
            // Row gather: lane i resolves the chunk's i-th position, then the
            // wave copies the rows one after another.
            const uint32_t nv = meta_nv(m);
            const uint32_t pos = position_at<VIS>(a, m.s, m.cs + min(lane, nv - 1));
            uint32_t jb = pos / bsz;
            bounds_report(a.bounds_flags, lane < nv && jb >= a.max_num_blocks_per_seq, kBoundTable);
#ifdef Q8_DEBUG_BOUNDS
            // listed positions ascending and distinct within the chunk
            const uint32_t prev = __shfl(pos, lane > 0 ? lane - 1 : 0, 64);
            bounds_report(a.bounds_flags, lane > 0 && lane < nv && pos <= prev, kBoundVisible);
#endif
            jb = jb < a.max_num_blocks_per_seq ? jb : a.max_num_blocks_per_seq - 1;
            uint32_t phys = a.block_tables[static_cast<uint64_t>(m.s) * a.max_num_blocks_per_seq + jb];
            bounds_report(a.bounds_flags, lane < nv && phys > num_blocks_m1, kBoundBlock);
            phys = phys < num_blocks_m1 ? phys : num_blocks_m1;
            const uint64_t my_row = ((static_cast<uint64_t>(phys) * a.num_kv_heads + kvh) * bsz +
                                     pos % bsz) * wpt;
            for (uint32_t rr = 0; rr < nv; ++rr) {
                const uint32_t lo = __shfl(static_cast<uint32_t>(my_row), rr, 64);
                const uint32_t hi = __shfl(static_cast<uint32_t>(my_row >> 32), rr, 64);
                const uint64_t base = (static_cast<uint64_t>(hi) << 32) | lo;
                for (uint32_t w = lane; w < wpt; w += kWave) {
                    sK[rr * wpt + w] = a.key_cache[base + w];
                    sV[rr * wpt + w] = a.value_cache[base + w];
                }
            }
        }
        store_new(m);
    };

    // ---- q digits of the current sequence: MFMA row r = (head r/4, digit r%4) ----
    i32x4 qa[NHS][NKB];
    int eq_out[NHS];       // q exponent of this lane's output head 4*hset + g
    // q rows of the query heads h0 .. h0+nh-1 (padded to G heads of QD
    // values) staged per lane as QF 16-byte slots: lane l, slot t holds padded
    // elements 4*(l + 64*t) .. +3.
    constexpr int QF = G * QD / (4 * kWave);
    static_assert(QF * kWave <= NHS * 16 * 16 && (QSCR || NHS * NKB * 256 <= BUFW), "q scratch");
    float4 qv[QF];
    // Norm + rotary step on the staged q rows: an exact head fills HS4P lanes
    // of a slot (QD == 4 * HS4P), lane w = lane % HS4P holding its elements
    // 4w .. 4w+3, so one set of weights and cos/sin per lane (q_op, staged
    // with the rows) serves every slot.
    auto q_issue = [&](uint32_t s, uint32_t L) __attribute__((always_inline)) {
        const uint64_t row = static_cast<uint64_t>(s) * nrow * a.q_stride;
        if constexpr (NR) {
            // position L - 1, L = context_lens[s] (a staged sequence has
            // positions, so L >= 1)
            const uint32_t w = lane % static_cast<uint32_t>(HS4P);
            q_op.wt = load_weight4(a.nr_q_weight, w, hs4, a.nr_params_vec4 != 0);
            load_cs4(nr_row(L - 1), w, a.nr_rot, a.nr_params_vec4 != 0, q_op.c, q_op.s);
        }
#pragma unroll
        for (int t = 0; t < QF; ++t) {
            const uint32_t e = 4 * (lane + kWave * t);
            const uint32_t hi = e / QD, d = e % QD;
            const bool ok = hi < nh && d < hs;               // d % 4 == 0 and hs % 4 == 0: all four or none
            const uint32_t pq = h0 + hi;                     // pair: row pq / n_rep, head kvh*n_rep + pq % n_rep
            const float* src = a.q + (ok ? row + static_cast<uint64_t>(pq / n_rep) * a.q_stride +
                                           static_cast<uint64_t>(kvh * n_rep + pq % n_rep) * a.q_head_stride + d
                                         : row);
            float4 v;
            if (c.q_vec_ok) {
                v = *reinterpret_cast<const float4*>(src);
            } else {
                v = make_float4(src[0], ok ? src[1] : 0.f, ok ? src[2] : 0.f, ok ? src[3] : 0.f);
            }
            qv[t] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    // Digits of the staged q rows.  Each head's exponent comes from its
    // largest |q|: the lanes write per-slot maxima to LDS and the 16 lanes of a
    // head reduce their share.  Then every lane converts its own staged values
    // once and scatters each value's four digits to the lanes whose MFMA rows
    // hold them, through LDS in the operand layout [set][k-block][lane][w].
    auto q_finish = [&]() __attribute__((always_inline)) {
        if constexpr (NR) {
            // slots of heads past nh stay zero (they are padding, not vectors)
            const RowMean mean(hs);
#pragma unroll
            for (int t = 0; t < QF; ++t) {
                const uint32_t hi = 4 * (lane + kWave * t) / QD;
                const float4 y = norm_rope4<HS4P>(qv[t], lane % static_cast<uint32_t>(HS4P), mean, q_op, a.nr_rot,
                                                  a.nr_eps);
                qv[t] = hi < nh ? y : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        uint32_t* const scratch = QSCR ? sQs_[wid] : sKn;   // sKn: no loads are landing in it yet
        uint32_t* const sDig = scratch;
        // per-slot maxima: in sA (not in use outside a chunk's processing)
        float* const sMax = reinterpret_cast<float*>(sA);
#pragma unroll
        for (int t = 0; t < QF; ++t) {
            const float4 v = qv[t];
            sMax[lane + kWave * t] = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        }
        wave_sync();
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset) {
            const uint32_t h = 4 * hset + r / 4;
            const uint32_t i = 4 * g + r % 4;                 // this lane's share of the head's 16*NKB maxima
            float m = 0.0f;
#pragma unroll
            for (int k = 0; k < NKB; ++k) m = fmaxf(m, sMax[h * 16 * NKB + i * NKB + k]);
            m = fmaxf(m, __shfl_xor(m, 1, 64));
            m = fmaxf(m, __shfl_xor(m, 2, 64));
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (g == 0 && r % 4 == 0) sEq[h] = m > 0.0f ? 30 - exponent_bound(m) : 0;   // |q * 2^eq| < 2^30
        }
        wave_sync();
#pragma unroll
        for (int t = 0; t < QF; ++t) {
            const uint32_t f = lane + kWave * t;              // staged float4 index: head f / (16*NKB)
            const uint32_t hi = f / (16 * NKB), d0 = 4 * (f % (16 * NKB));
            const int eq = sEq[hi];
            const float4 v = qv[t];
            const uint32_t dw[4] = {to_digits(static_cast<int32_t>(rintf(ldexpf(v.x, eq)))),
                                    to_digits(static_cast<int32_t>(rintf(ldexpf(v.y, eq)))),
                                    to_digits(static_cast<int32_t>(rintf(ldexpf(v.z, eq)))),
                                    to_digits(static_cast<int32_t>(rintf(ldexpf(v.w, eq))))};
            uint32_t pk[4];
            transpose4(dw, pk);                              // byte e of pk[dig] = digit dig of value e
            const uint32_t kb = d0 / 64, gq = (d0 % 64) / 16, w = (d0 % 16) / 4;
            const uint32_t base = (((hi / 4) * NKB + kb) * kWave + 16 * gq + 4 * (hi % 4)) * 4 + w;
#pragma unroll
            for (int dg = 0; dg < 4; ++dg) sDig[base + 4 * dg] = pk[dg];
        }
        wave_sync();
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                qa[hset][kb] = *reinterpret_cast<const i32x4*>(&sDig[((hset * NKB + kb) * kWave + lane) * 4]);
            eq_out[hset] = sEq[4 * hset + g];
        }
        wave_sync();
    };

    // Online-softmax state (log2 units) of head 4*hset + g, uniform across the lane's row.
    float m_run[NHS], l_run[NHS];
    float acc[NHS][NCW][4];      // dims 4*NCW*r + 4*cw + j of head 4*hset + g
    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset) {
            m_run[hset] = -INFINITY;
            l_run[hset] = 0.0f;
#pragma unroll
            for (int cw = 0; cw < NCW; ++cw)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[hset][cw][jj] = 0.0f;
        }
    };

    // One chunk from LDS: q.K^T, online softmax, P.V.
    auto process = [&](const Meta& pm) __attribute__((always_inline)) {
        const uint32_t nv = meta_nv(pm);
        // Tokens of the chunk each of the lane's pairs attends: all nv, except in
        // multi-row decode, where row b of nrow stops nrow-1-b positions early.
        uint32_t nvh[NHS];
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset) {
            const uint32_t pq = h0 + 4 * hset + g;
            const uint32_t dl = nrow - 1 - min(pq / n_rep, nrow - 1);
            nvh[hset] = nrow > 1 ? min(nv, pm.lr > dl ? pm.lr - dl : 0u) : nv;
        }
        // ---- q . K^T (NTG groups of 16 tokens) ----
        i32x4 dsum[NHS][4];
#pragma unroll
        for (int tg = 0; tg < NTG; ++tg) {
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
        for (int tg = 0; tg < NTG; ++tg) {
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
            bool vh[4];
            float cmax = -INFINITY;
#pragma unroll
            for (int tg = 0; tg < NTG; ++tg) {
                vh[tg] = 16 * tg + r < nvh[hset];
                const float zq = ldexpf(combine_digits(dsum[hset][tg]), -eq_out[hset]);
                z[tg] = vh[tg] ? zq * (ksc[tg] * a.scale_log2) : -INFINITY;
                cmax = fmaxf(cmax, z[tg]);
            }
            const float m_new = fmaxf(m_run[hset], row_max(cmax));
            // -inf only while a multi-row pair has attended nothing: no NaN from exp2(-inf + inf)
            const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_run[hset] - m_new);
            float psum = 0.0f;
            uint32_t wd[4] = {0u, 0u, 0u, 0u};      // groups past the chunk (CH = 32): weight 0
#pragma unroll
            for (int tg = 0; tg < NTG; ++tg) {
                const float p = vh[tg] ? exp2f(z[tg] - m_new) : 0.0f;
                psum += p;
                const float pv = vh[tg] ? p * vsc[tg] : 0.0f;
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
                for (int jj = 0; jj < 4; ++jj) acc[hset][cw][jj] *= alpha;
        }
        wave_sync();

        // ---- P . V ----
        i32x4 pa[NHS];
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset)
            pa[hset] = *reinterpret_cast<const i32x4*>(&sA[(hset * 16 + r) * 16 + 4 * g]);
#pragma unroll
        for (int cw = 0; cw < NCW; ++cw) {
            uint32_t bj[4][4];      // [byte j][w]: codes of tokens 4g + w + 16*b (byte b)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t x[4], y[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t word = NCW * r + cw;
                    x[b] = (b < NTG && (EXACT || word < hs4)) ? sV[(4 * g + w + 16 * b) * wpt + word] : 0u;
                }
                transpose4(x, y);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) bj[jj][w] = y[jj];
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const i32x4 b = i32x4{static_cast<int32_t>(bj[jj][0]), static_cast<int32_t>(bj[jj][1]),
                                      static_cast<int32_t>(bj[jj][2]), static_cast<int32_t>(bj[jj][3])};
#pragma unroll
                for (int hset = 0; hset < NHS; ++hset) {
                    const i32x4 d = mfma_i8(pa[hset], b, i32x4{0, 0, 0, 0});
                    acc[hset][cw][jj] += ldexpf(combine_digits(d), -ep);
                }
            }
        }
    };

    // Combine the nrec records of sequence ms (waves jf .. jf+nrec-1) into its
    // output rows.  Each lane combines, for each of its (head, 4 dims) items
    // in the records' lane-order layout, a batch of records at a time (8 when
    // the lane holds up to four 16-byte values per record, else 4) with a
    // running max and rescaling as in the online softmax.  A batch's loads for all the
    // lane's items are issued together (device-coherent 8-byte loads the
    // compiler tracks), so a batch costs one memory round trip whatever the
    // number of items.
    auto merge = [&](uint32_t ms, uint32_t jf, uint32_t nrec) __attribute__((always_inline)) {
        // records per batch: MB * NHS * NCW 16-byte values in registers
        constexpr int MB = NHS * NCW <= 4 ? 8 : NHS * NCW <= 8 ? 4 : 2;
        const uint64_t rec0 = static_cast<uint64_t>(rg) * c.recs_per_rg + ms + jf;      // record of wave jf
        float M[NHS], L[NHS];
        f32x4 o[NHS][NCW];
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset) {
            M[hset] = -INFINITY;
            L[hset] = 0.0f;
#pragma unroll
            for (int cw = 0; cw < NCW; ++cw) o[hset][cw] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (uint32_t i0 = 0; i0 < nrec; i0 += MB) {
            f32x4 v[MB][NHS][NCW];
            f32x2 ml[MB][NHS];
#pragma unroll
            for (int k = 0; k < MB; ++k) {
                const uint64_t rec = rec0 + min(i0 + k, nrec - 1);
#pragma unroll
                for (int hset = 0; hset < NHS; ++hset) {
                    ml[k][hset] = coherent_load2(a.part_ml + 2 * (rec * G + 4 * hset + g));
#pragma unroll
                    for (int cw = 0; cw < NCW; ++cw)
                        v[k][hset][cw] = coherent_load4(a.part_acc + rec * kRecFloats +
                                                        4 * ((hset * NCW + cw) * kWave + lane));
                }
            }
#pragma unroll
            for (int hset = 0; hset < NHS; ++hset) {
                float bm = M[hset];
#pragma unroll
                for (int k = 0; k < MB; ++k)
                    if (i0 + k < nrec) bm = fmaxf(bm, ml[k][hset].x);
                // A record whose row attended nothing (multi-row decode) has
                // max -inf and sum 0: it gets weight 0, never exp2(nan).
                const float sc = bm == -INFINITY ? 1.0f : exp2f(M[hset] - bm);
                L[hset] *= sc;
#pragma unroll
                for (int cw = 0; cw < NCW; ++cw) o[hset][cw] *= sc;
#pragma unroll
                for (int k = 0; k < MB; ++k) {
                    const float w = (i0 + k < nrec && ml[k][hset].x != -INFINITY) ? exp2f(ml[k][hset].x - bm) : 0.0f;
                    L[hset] += w * ml[k][hset].y;
#pragma unroll
                    for (int cw = 0; cw < NCW; ++cw) o[hset][cw] += w * v[k][hset][cw];
                }
                M[hset] = bm;
            }
        }
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset) {
            const uint32_t hh = 4 * hset + g;
            const float inv = L[hset] > 0.0f ? 1.0f / L[hset] : 0.0f;      // an empty prefix gives a zero row
#pragma unroll
            for (int cw = 0; cw < NCW; ++cw) {
                const uint32_t word = NCW * r + cw;
                if (hh < nh && word < hs4) {
                    const f32x4 x = o[hset][cw];
                    *reinterpret_cast<float4*>(a.out + pair_out_row(a, ms, kvh, n_rep, nrow, h0 + hh) * hs + 4 * word) =
                        make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv);
                }
            }
        }
    };

    uint32_t npend = 0, pend_s0 = 0, pend_jf0 = 0, pend_n0 = 0, pend_s1 = 0, pend_jf1 = 0, pend_n1 = 0;

    // ---- end of a sequence's share: final output or a partial record ----
    // Lane (r, g) holds dims 4*NCW*r + 4*cw + j of head 4*hset + g.  Record id
    // j + s is unique within the row group: a wave's sequences increase, and a
    // later wave starts at or after the sequence where the previous one ended.
    // The last of the sequence's waves to arrive (a counter per (row group,
    // sequence), which it sets back to zero) later combines all its records.
    auto flush = [&](const Meta& m) __attribute__((always_inline)) {
        const uint32_t nrec = meta_nrec(m);
        const uint64_t rec0 = static_cast<uint64_t>(rg) * c.recs_per_rg + m.s;    // record of wave jj: rec0 + jj
#pragma unroll
        for (int hset = 0; hset < NHS; ++hset) {
            const uint32_t hh = 4 * hset + g;
#pragma unroll
            for (int cw = 0; cw < NCW; ++cw) {
                const uint32_t word = NCW * r + cw;
                float4 v = make_float4(acc[hset][cw][0], acc[hset][cw][1], acc[hset][cw][2], acc[hset][cw][3]);
                if (nrec == 1) {
                    if (hh >= nh || word >= hs4) continue;
                    const float inv = l_run[hset] > 0.0f ? 1.0f / l_run[hset] : 0.0f;   // empty prefix: zero row
                    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
                    *reinterpret_cast<float4*>(a.out + pair_out_row(a, m.s, kvh, n_rep, nrow, h0 + hh) * hs + 4 * word) = v;
                } else {
                    // record layout: [head set][column word][lane] 16-byte units
                    float* pa_ = a.part_acc + (rec0 + j) * kRecFloats + 4 * ((hset * NCW + cw) * kWave + lane);
                    coherent_store4(pa_, f32x4{v.x, v.y, v.z, v.w});
                    if (cw == 0 && r == 0)
                        coherent_store2(a.part_ml + 2 * ((rec0 + j) * G + hh), f32x2{m_run[hset], l_run[hset]});
                }
            }
        }
        reset();
        if (nrec == 1) return;
        // The record was written with device-coherent stores; once they have
        // completed, count this wave in.  No cache maintenance is needed (a
        // device-scope fence would write back and invalidate the whole L2).
        wait_vmem();
        uint32_t prev = 0;
        if (lane == 0)
            prev = __hip_atomic_fetch_add(a.counters + static_cast<uint64_t>(rg) * a.num_seqs + m.s, 1u,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = uniform(prev);
        if (prev != nrec - 1) return;
        // Last arrival: reset the counter for the next call; the records are
        // combined after the main loop, when the tile registers are free.  A
        // sequence shared with other waves extends past one end of this
        // wave's range, so there are at most two such sequences per wave.
        if (lane == 0)
            __hip_atomic_store(a.counters + static_cast<uint64_t>(rg) * a.num_seqs + m.s, 0u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (npend == 0) { pend_s0 = m.s; pend_jf0 = m.jf; pend_n0 = nrec; }
        else { pend_s1 = m.s; pend_jf1 = m.jf; pend_n1 = nrec; }
        ++npend;
    };

    // ---- pipeline over the wave's chunks x0 .. x1-1 ----
    // Step for chunk x (relative index xr): its tiles sit in registers; the
    // step stores them to LDS, reads the block ids of chunk x+2, issues the
    // tile loads of chunk x+1 into the freed registers (and the q rows of its
    // sequence when that changes), and processes chunk x.
    reset();
    // Prologue order: q of the first sequence, block ids of chunk x0, chunk
    // x0's tiles, block ids of x0+1; the q digits are formed while tiles arrive.
    Buf bA;
    q_issue(cur.s, one_window ? lane_value(win_len, cur.s) : cur.len);   // q first: the first chunk's block-id wait below would delay it
    Meta mc = meta_of(true, true);
    issue_data(mc, bA, sK, sV);
    issue_new(mc);
    Meta mn1;
    if (n > 1) advance();
    mn1 = meta_of(n > 1);
    q_finish();
    uint32_t q_seq_prev = mc.s;
    for (uint32_t xr = 0;; ++xr) {
        // Issue priority by the chunks left: of the waves sharing a SIMD, the
        // one with more work left issues first, so they tend to finish
        // together (the arbiter otherwise favours the older wave, and the
        // latest waves of a launch were the younger workgroups').
        if (n - xr > 12) __builtin_amdgcn_s_setprio(3);
        else if (n - xr > 6) __builtin_amdgcn_s_setprio(2);
        else if (n - xr > 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        // q of mc.s was staged one step ago; its digits are formed before the
        // next sequence's q rows are staged into the same registers.
        const bool new_q = xr > 0 && mc.s != q_seq_prev;
        if (!QSCR && new_q) q_finish();
        store(mc, bA);
        if (QSCR && new_q) {
            // The staged q rows have landed (store waited for every load).  Use
            // them here so that the compiler's wait for them sits here, before
            // the next chunk's LDS-direct loads it does not count; placed at
            // q_finish it would also wait for those.
#pragma unroll
            for (int t = 0; t < QF; ++t) asm volatile("" : : "v"(qv[t].x), "v"(qv[t].y), "v"(qv[t].z), "v"(qv[t].w));
            if constexpr (NR) {
                asm volatile("" : : "v"(q_op.wt.x), "v"(q_op.wt.y), "v"(q_op.wt.z), "v"(q_op.wt.w));
                asm volatile("" : : "v"(q_op.c.x), "v"(q_op.c.y), "v"(q_op.c.z), "v"(q_op.c.w));
                asm volatile("" : : "v"(q_op.s.x), "v"(q_op.s.y), "v"(q_op.s.z), "v"(q_op.s.w));
            }
        }
        if (xr + 2 < n) advance();
        const Meta mn2 = meta_of(xr + 2 < n);
        issue_data(mn1, bA, sKn, sVn);
        issue_new(mn1);
        if (QSCR && new_q) q_finish();                        // with the next chunk's loads in flight
        if (mn1.s != mc.s) q_issue(mn1.s, mn1.len);                    // q of the next chunk's sequence
        wave_sync();
        process(mc);
        if (xr + 1 == n || mn1.s != mc.s) flush(mc);
        if (xr + 1 == n) break;
        wave_sync();
        q_seq_prev = mc.s;
        mc = mn1;
        mn1 = mn2;
        if (DMA) {
            uint32_t* t = sK; sK = sKn; sKn = t;
            t = sV; sV = sVn; sVn = t;
        }
    }
    if (DMA) wait_vmem();      // no LDS-direct load may still be landing when the wave ends
    if (npend > 0) merge(pend_s0, pend_jf0, pend_n0);
    if (npend > 1) merge(pend_s1, pend_jf1, pend_n1);
    if (j == W - 1) zero_seqs(mc.s + 1, a.num_seqs);
}

template <int HS4P, bool EXACT, int NHS, bool VIS, bool TILED>
const void* split_kernel_seg(bool tiled, uint32_t seg_rows) {
    constexpr int CH = decode_chunk(HS4P, NHS);
    // Scalar-addressed segment loads need an exact head size, 16-byte aligned
    // caches and tile segments of 16 or 32 rows.
    const uint32_t segr = EXACT && tiled ? seg_rows : 0;
    if (EXACT && segr == 16)
        return reinterpret_cast<const void*>(&decode_split_kernel<HS4P, EXACT, NHS, VIS, TILED, EXACT ? 16 : 0, CH>);
    if (EXACT && segr == 32)
        return reinterpret_cast<const void*>(&decode_split_kernel<HS4P, EXACT, NHS, VIS, TILED, EXACT ? 32 : 0, CH>);
    return reinterpret_cast<const void*>(&decode_split_kernel<HS4P, EXACT, NHS, VIS, TILED, 0, CH>);
}

template <int HS4P, bool EXACT, int NHS>
const void* split_kernel_t(bool vis, bool tiled, uint32_t seg_rows) {
    if (vis) return split_kernel_seg<HS4P, EXACT, NHS, true, false>(tiled, seg_rows);
    if (EXACT && tiled) return split_kernel_seg<HS4P, EXACT, NHS, false, EXACT>(tiled, seg_rows);
    return reinterpret_cast<const void*>(
        &decode_split_kernel<HS4P, EXACT, NHS, false, false, 0, decode_chunk(HS4P, NHS)>);
}

template <int HS4P, bool EXACT>
const void* split_kernel_g(bool vis, bool tiled, uint32_t group, uint32_t seg_rows) {
    if (group == 16) return split_kernel_t<HS4P, EXACT, 4>(vis, tiled, seg_rows);
    if (group == 8) return split_kernel_t<HS4P, EXACT, 2>(vis, tiled, seg_rows);
    return split_kernel_t<HS4P, EXACT, 1>(vis, tiled, seg_rows);
}

// The norm + rotary decode step (exact head sizes of HS4P code words, dense,
// tiled chunks) for sets of NHS query heads.
template <int HS4P, int NHS>
const void* split_kernel_nr_seg(uint32_t seg_rows) {
    constexpr int CH = decode_chunk(HS4P, NHS);
    if (seg_rows == 16)
        return reinterpret_cast<const void*>(&decode_split_kernel<HS4P, true, NHS, false, true, 16, CH, true>);
    if (seg_rows == 32)
        return reinterpret_cast<const void*>(&decode_split_kernel<HS4P, true, NHS, false, true, 32, CH, true>);
    return reinterpret_cast<const void*>(&decode_split_kernel<HS4P, true, NHS, false, true, 0, CH, true>);
}

template <int HS4P>
const void* split_kernel_nr(uint32_t group, uint32_t seg_rows) {
    if (group == 16) {
        // none for 16 heads at head_size 256: the plain kernel already spills there
        if constexpr (HS4P == 64) return nullptr;
        else return split_kernel_nr_seg<HS4P, 4>(seg_rows);
    }
    if (group == 8) return split_kernel_nr_seg<HS4P, 2>(seg_rows);
    return split_kernel_nr_seg<HS4P, 1>(seg_rows);
}

}  // namespace
}  // namespace q8kv
