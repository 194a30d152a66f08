// Full-width paged-cache baselines (f32 and bfloat16): cache writer and
// single-query decode.
//
// The "paged_attn_q8.comp" page's header says the int8 decode keeps the math
// and workgroup structure of an f32 paged decode whose cache holds 4 bytes per
// element (the int8 cache's point being the 4x smaller read), and the
// "reshape_and_cache_q8.comp" page's header says its pad-slot rule mirrors the
// f32 writer.  The f32 layout is not printed there; it is taken to be the int8
// layout with one f32 per element: [num_blocks, num_kv_heads, block_size,
// head_size].  The bfloat16 cache (not on the pages; the half-width cache most
// serving stacks keep) is the same layout with 2-byte elements, each the
// nearest bfloat16 to the f32 input (ties to even).  These kernels serve to
// measure the int8 cache against both on the same batch.
//
// Decode, MI355X mapping.  The work is a stream of rows with one multiply-add
// per element and query head for q.k and one for p.v, on the VALU.  For f32
// that is below the rate at which HBM delivers elements; bfloat16 delivers
// twice the elements per byte for the same arithmetic and is bound by VALU
// issue at four query heads per row group.  Laid out for the loads:
//   * A row of head_size elements is read by LPT lanes with 16-byte loads of
//     EPL elements (4 f32 or 8 bfloat16, widened to f32 on use), LPT =
//     head_size/EPL; one load instruction covers 64/LPT consecutive
//     positions, and a chunk is 8 such loads per tensor (8 KiB of K and 8 KiB
//     of V per wave; 4 loads for bfloat16, whose q slices and accumulators
//     take twice the registers), fetched into registers one chunk ahead, the
//     block ids two chunks ahead.
//   * A wave handles one row group: a kv head and G = 4, 2 or 1 of its query
//     heads, whose q slices stay in registers.  q.k is an EPL-element partial
//     per lane, summed over the row's LPT lanes with DPP and a swizzle; the
//     softmax runs in the exp2 domain with the running max uniform over the
//     wave and the running sum and output kept per lane group until the end
//     of a sequence.
//   * The chunks of all sequences form one list of C chunks per row group;
//     persistent waves take equal contiguous ranges of it.  A wave that covers
//     a whole sequence writes the output; otherwise it leaves a partial record
//     (running max, sum, unnormalized output) through device-coherent stores
//     and counts itself in, and the last wave to arrive combines the records.
#include "q8kv_internal.h"
#include "wave_ops.h"

#include <cstdlib>
#include <type_traits>

namespace q8kv {
namespace {

constexpr int kLoadsPerChunk = 8;       // 16-byte loads per lane and tensor per chunk
constexpr int kRowMirror = 0x140;       // DPP: lane i of a row reads lane 15 - i
constexpr int kRowHalfMirror = 0x141;   // DPP: lane i of a half row reads lane 7 - i
constexpr int kQuadSwap1 = 0xB1;        // DPP quad_perm [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;        // DPP quad_perm [2, 3, 0, 1]
constexpr int kSwizzleXor16 = 0x401F;   // ds_swizzle: lane i of 32 reads lane i ^ 16

__device__ __forceinline__ float swizzle_xor16(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kSwizzleXor16));
}
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, kWave); }
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over each aligned group of LPT lanes; every lane of a group receives
// the same value (each step adds a lane's partner symmetrically).
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
    if (LPT >= 2) v += dpp_mov<kQuadSwap1>(v);
    if (LPT >= 4) v += dpp_mov<kQuadSwap2>(v);
    if (LPT >= 8) v += dpp_mov<kRowHalfMirror>(v);
    if (LPT >= 16) v += dpp_mov<kRowMirror>(v);
    if (LPT >= 32) v += swizzle_xor16(v);
    if (LPT >= 64) v += xor32(v);
    return v;
}

// For a value that is equal within each group of LPT lanes: the maximum over
// the groups, uniform over the wave.
template <int LPT>
__device__ __forceinline__ float groups_max(float v) {
    if (LPT <= 2) v = fmaxf(v, dpp_mov<kRowRor2>(v));
    if (LPT <= 4) v = fmaxf(v, dpp_mov<kRowRor4>(v));
    if (LPT <= 8) v = fmaxf(v, dpp_mov<kRowRor8>(v));
    if (LPT >= 64) return readlane_f(v, 0);
    if (LPT == 32) return fmaxf(readlane_f(v, 0), readlane_f(v, 32));
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// Sum over the groups of LPT lanes of the lanes at the same position in their
// group: lane i receives sum_g v[g*LPT + i % LPT].
template <int LPT>
__device__ __forceinline__ float groups_sum(float v) {
    if (LPT <= 2) v += dpp_mov<kRowRor2>(v);
    if (LPT <= 4) v += dpp_mov<kRowRor4>(v);
    if (LPT <= 8) v += dpp_mov<kRowRor8>(v);
    if (LPT <= 16) v += swizzle_xor16(v);
    if (LPT <= 32) v += xor32(v);
    return v;
}

__device__ __forceinline__ float4 f4_zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }


// Device-coherent (agent scope) element accesses for the partial records
// handed between waves that may run on different XCDs; they compile to sc1
// loads and stores, which bypass the XCD's non-coherent L2 copies.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

// ---------------------------------------------------------------- writer ----

// Element type of a cache: E = float (4 per 16-byte unit) or uint16_t holding
// a bfloat16 (8 per unit).
template <typename E>
constexpr int epl() { return 16 / static_cast<int>(sizeof(E)); }

// The bfloat16 nearest to finite x, ties to even, as its 16 bits: adding
// 0x7FFF plus the lowest kept bit carries into the upper half exactly when the
// dropped half is above half an ulp, or exactly half with an odd kept part.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) { return bf16_bits(lo) | (bf16_bits(hi) << 16); }

__device__ __forceinline__ float4 load_f4(const float* p, bool vec4) {
    return vec4 ? *reinterpret_cast<const float4*>(p) : make_float4(p[0], p[1], p[2], p[3]);
}

// One thread per 16-byte unit of a (token, kv head) row of the cache.
template <typename E>
__global__ __launch_bounds__(256) void baseline_write_kernel(BaselineWriteArgs a, bool vec4) {
    constexpr int EPL = epl<E>();
    const uint32_t units = a.head_size / EPL;
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads * units) return;
    const uint32_t w = static_cast<uint32_t>(i % units);
    const uint64_t th = i / units;
    const uint32_t h = static_cast<uint32_t>(th % a.num_kv_heads);
    const uint32_t t = static_cast<uint32_t>(th / a.num_kv_heads);
    const uint32_t slot = a.slot_mapping[t];
    if (slot == kPadSlot) return;
    const uint64_t block = slot / a.block_size, off = slot % a.block_size;
    if (block >= a.num_blocks) return;   // out of contract; skipped rather than written out of bounds
    const float* ks = a.key + static_cast<uint64_t>(t) * a.key_stride + static_cast<uint64_t>(h) * a.head_size + EPL * w;
    const float* vs = a.value + static_cast<uint64_t>(t) * a.value_stride + static_cast<uint64_t>(h) * a.head_size + EPL * w;
    const uint64_t dst = ((block * a.num_kv_heads + h) * a.block_size + off) * a.head_size + EPL * w;
    if constexpr (EPL == 4) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.key_cache) + dst) = load_f4(ks, vec4);
        *reinterpret_cast<float4*>(static_cast<float*>(a.value_cache) + dst) = load_f4(vs, vec4);
    } else {
        const float4 k0 = load_f4(ks, vec4), k1 = load_f4(ks + 4, vec4);
        const float4 v0 = load_f4(vs, vec4), v1 = load_f4(vs + 4, vec4);
        *reinterpret_cast<uint4*>(static_cast<E*>(a.key_cache) + dst) =
            make_uint4(bf16_pair(k0.x, k0.y), bf16_pair(k0.z, k0.w), bf16_pair(k1.x, k1.y), bf16_pair(k1.z, k1.w));
        *reinterpret_cast<uint4*>(static_cast<E*>(a.value_cache) + dst) =
            make_uint4(bf16_pair(v0.x, v0.y), bf16_pair(v0.z, v0.w), bf16_pair(v1.x, v1.y), bf16_pair(v1.z, v1.w));
    }
}

// ---------------------------------------------------------------- decode ----

// Positions of sequence s (the context clamp applied).
__device__ __forceinline__ uint32_t seq_positions(const BaselineDecodeArgs& a, uint32_t s) {
    const uint32_t L = a.context_lens[s];
    return L < a.max_context_len ? L : a.max_context_len;
}

// A 16-byte unit of a cache row as loaded: four f32, or eight bfloat16 as
// four words.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
template <typename E>
using unit_t = typename std::conditional<epl<E>() == 4, f32x4, u32x4v>::type;

// Element e of a unit, as f32 (a bfloat16 is the upper half of its binary32
// encoding, so widening is exact).
__device__ __forceinline__ float unit_elem(const f32x4& w, int e) { return w[e]; }
__device__ __forceinline__ float unit_elem(const u32x4v& w, int e) {
    return __uint_as_float((e & 1) ? (w[e / 2] & 0xFFFF0000u) : (w[e / 2] << 16));
}

template <typename E, int LPT, int G>
__global__ __launch_bounds__(256, 2) void baseline_decode_kernel(BaselineDecodeArgs a) {
    constexpr int EPL = epl<E>();                       // elements per 16-byte unit
    // 16-byte loads per lane and tensor per chunk: 8, or 4 for bfloat16,
    // whose q slices and accumulators take twice the registers
    constexpr int NL = EPL == 4 ? kLoadsPerChunk : kLoadsPerChunk / 2;
    constexpr int TPI = kWave / LPT;                    // positions per load instruction
    constexpr uint32_t T = NL * TPI;                    // positions per chunk
    constexpr uint32_t HS = EPL * LPT;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wid = uniform(blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave);
    // Row group fastest: the groups of one kv head, which read the same rows,
    // share a workgroup.
    const uint32_t W = a.waves_per_rg;
    const uint32_t num_rg = a.num_kv_heads * a.num_groups;
    const uint32_t rg = wid % num_rg, j = wid / num_rg;
    if (j >= W) return;
    const uint32_t kvh = rg / a.num_groups;
    const uint32_t n_rep = a.num_heads / a.num_kv_heads;
    const uint32_t h0 = kvh * n_rep + (rg % a.num_groups) * G;
    const uint32_t S = a.num_seqs;
    const uint32_t col = lane % LPT, grp_l = lane / LPT;

    // EPL floats of an output row, from lane group column c
    auto store_out = [&](uint64_t row, uint32_t c, const float (&x)[EPL]) {
#pragma unroll
        for (int u = 0; u < EPL / 4; ++u)
            *reinterpret_cast<float4*>(a.out + row * HS + EPL * c + 4 * u) =
                make_float4(x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]);
    };

    // ---- chunk count C of the row group; empty sequences s = j (mod W) get zero rows ----
    uint32_t C = 0;
    for (uint32_t base = 0; base < S; base += kWave) {
        const uint32_t s = base + lane;
        const uint32_t L = s < S ? seq_positions(a, s) : 0;
        const uint32_t nc = (L + T - 1) / T;
        const uint32_t incl = wave_incl_scan(nc, lane);
        C += lane_value(incl, kWave - 1);
        uint64_t zmask = __ballot(s < S && L == 0 && s % W == j);
        while (zmask) {
            const uint32_t zs = base + static_cast<uint32_t>(__builtin_ctzll(zmask));
            zmask &= zmask - 1;
            for (uint32_t e = lane; e < G * LPT; e += kWave) {
                const uint32_t g = e / LPT, c = e % LPT;
#pragma unroll
                for (int u = 0; u < EPL / 4; ++u)
                    *reinterpret_cast<float4*>(a.out + (static_cast<uint64_t>(zs) * a.num_heads + h0 + g) * HS +
                                               EPL * c + 4 * u) = f4_zero();
            }
        }
    }
    C = uniform(C);
    // With fewer chunks than waves only the first C waves work, so that
    // every working wave's range holds at least one chunk.
    const uint32_t Wc = W < C ? W : C;
    if (j >= Wc) return;
    const uint32_t x0 = uniform(static_cast<uint32_t>(static_cast<uint64_t>(j) * C / Wc));
    const uint32_t x1 = uniform(static_cast<uint32_t>(static_cast<uint64_t>(j + 1) * C / Wc));

    // ---- the sequence holding chunk x0 ----
    uint32_t cs = 0, ck = 0, cbefore = 0;   // cursor: sequence, chunk within it, chunks before it
    {
        uint32_t acc = 0;
        for (uint32_t base = 0; base < S; base += kWave) {
            const uint32_t s = base + lane;
            const uint32_t nc = s < S ? (seq_positions(a, s) + T - 1) / T : 0;
            const uint32_t incl = acc + wave_incl_scan(nc, lane);
            const uint64_t hit = __ballot(incl > x0);
            if (hit) {
                const uint32_t f = static_cast<uint32_t>(__builtin_ctzll(hit));
                cs = base + f;
                cbefore = lane_value(incl - nc, f);
                break;
            }
            acc = lane_value(incl, kWave - 1);
        }
        cs = uniform(cs);
        cbefore = uniform(cbefore);
        ck = x0 - cbefore;
    }
    uint32_t cL = uniform(seq_positions(a, cs));

    struct Meta {
        uint32_t s, k, L, before;   // sequence, chunk within it, its positions, chunks before it
    };
    // Next chunk of the row group's list (only called while one remains).
    auto advance = [&]() {
        ++ck;
        if (static_cast<uint64_t>(ck) * T >= cL) {
            cbefore += (cL + T - 1) / T;
            ck = 0;
            do {
                ++cs;
                cL = uniform(seq_positions(a, cs));
            } while (cL == 0);
        }
    };

    const E* kbase = static_cast<const E*>(a.key_cache) + static_cast<uint64_t>(kvh) * a.block_size * HS + EPL * col;
    const E* vbase = static_cast<const E*>(a.value_cache) + static_cast<uint64_t>(kvh) * a.block_size * HS + EPL * col;
    const uint64_t block_stride = static_cast<uint64_t>(a.num_kv_heads) * a.block_size * HS;

    // Row offsets (elements from kbase) of the lane's positions in chunk m; an
    // invalid position gets ~0u.
    auto rows_of = [&](const Meta& m, uint64_t (&row)[NL]) {
        const uint32_t c0 = m.k * T;
        const uint32_t q0 = c0 / a.block_size, r0 = c0 % a.block_size;
        const uint32_t* bt = a.block_tables + static_cast<uint64_t>(m.s) * a.max_num_blocks_per_seq;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint32_t d = i * TPI + grp_l;
            const uint32_t t = r0 + d;
            // t < block_size + T: one step when block_size >= T, else an exact
            // float quotient (t < 512, so t + 1/2 is at least 1/512 of a block
            // away from a multiple of block_size).
            const uint32_t qt = a.block_size >= T ? static_cast<uint32_t>(t >= a.block_size)
                                                 : static_cast<uint32_t>((static_cast<float>(t) + 0.5f) * a.inv_block_size);
            const uint32_t off = t - qt * a.block_size;
            uint64_t r = ~0ull;
            if (c0 + d < m.L) {
                uint32_t jb = q0 + qt;
                jb = jb < a.max_num_blocks_per_seq ? jb : a.max_num_blocks_per_seq - 1;   // out of contract
                uint32_t ph = bt[jb];
                ph = ph < a.num_blocks ? ph : a.num_blocks - 1;                            // out of contract
                r = ph * block_stride + static_cast<uint64_t>(off) * HS;
            }
            row[i] = r;
        }
    };

    typedef unit_t<E> U;
    struct Buf {
        U k[NL], v[NL];
    };
    auto issue = [&](const uint64_t (&row)[NL], Buf& b) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            if (row[i] != ~0ull) {
                b.k[i] = __builtin_nontemporal_load(reinterpret_cast<const U*>(kbase + row[i]));
                b.v[i] = __builtin_nontemporal_load(reinterpret_cast<const U*>(vbase + row[i]));
            } else {
                b.k[i] = U{};
                b.v[i] = U{};
            }
        }
    };
    auto load_q = [&](uint32_t s, float (&qv)[G][EPL]) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int u = 0; u < EPL / 4; ++u) {
                const float4 x = *reinterpret_cast<const float4*>(a.q + static_cast<uint64_t>(s) * a.q_stride +
                                                                  static_cast<uint64_t>(h0 + g) * HS + EPL * col + 4 * u);
                qv[g][4 * u] = x.x * a.scale_log2;
                qv[g][4 * u + 1] = x.y * a.scale_log2;
                qv[g][4 * u + 2] = x.z * a.scale_log2;
                qv[g][4 * u + 3] = x.w * a.scale_log2;
            }
    };

    // Online-softmax state of the current piece.
    float m_run[G], l_run[G];
    float acc[G][EPL];
    auto reset = [&]() {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m_run[g] = -INFINITY;
            l_run[g] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
        }
    };

    auto process = [&](const Meta& m, const Buf& b, const float (&qv)[G][EPL]) {
        const uint32_t c0 = m.k * T;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float z[NL];
            float cmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                float p = qv[g][0] * unit_elem(b.k[i], 0);
#pragma unroll
                for (int e = 1; e < EPL; ++e) p = fmaf(qv[g][e], unit_elem(b.k[i], e), p);
                p = group_sum<LPT>(p);
                z[i] = c0 + i * TPI + grp_l < m.L ? p : -INFINITY;
                cmax = fmaxf(cmax, z[i]);
            }
            const float mn = fmaxf(m_run[g], groups_max<LPT>(cmax));   // finite: the chunk holds a position
            const float alpha = exp2f(m_run[g] - mn);
            m_run[g] = mn;
            float l = l_run[g] * alpha;
            float o[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[e] = acc[g][e] * alpha;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const float p = exp2f(z[i] - mn);
                l += p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, unit_elem(b.v[i], e), o[e]);
            }
            l_run[g] = l;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = o[e];
        }
    };

    // Wave holding chunk x of the row group's list.
    auto wave_of = [&](uint32_t x) -> uint32_t {
        return static_cast<uint32_t>(((static_cast<uint64_t>(x) + 1) * Wc + C - 1) / C - 1);
    };
    const uint64_t rec_base = static_cast<uint64_t>(rg) * a.recs_per_rg;

    // End of the wave's piece of sequence m.s, whose chunks kfirst .. m.k it covered.
    auto flush = [&](const Meta& m, uint32_t kfirst) {
        const uint32_t nc = (m.L + T - 1) / T;
        float l_tot[G];
        float o[G][EPL];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            l_tot[g] = groups_sum<LPT>(l_run[g]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[g][e] = groups_sum<LPT>(acc[g][e]);
        }
        if (kfirst == 0 && m.k + 1 == nc) {
            if (grp_l == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float inv = 1.0f / l_tot[g];
                    float x[EPL];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) x[e] = o[g][e] * inv;
                    store_out(static_cast<uint64_t>(m.s) * a.num_heads + h0 + g, col, x);
                }
            }
            return;
        }
        // Partial record j + s of the row group (wave ranges are monotone in
        // the sequence, so j + s is distinct for every (wave, sequence) piece).
        const uint64_t rec = rec_base + j + m.s;
        if (grp_l == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float* pa = a.part_acc + (rec * G + g) * HS + EPL * col;
#pragma unroll
                for (int e = 0; e < EPL; ++e) store_coherent(pa + e, o[g][e]);
                if (col == 0) {
                    store_coherent(a.part_ml + (rec * G + g) * 2 + 0, m_run[g]);
                    store_coherent(a.part_ml + (rec * G + g) * 2 + 1, l_tot[g]);
                }
            }
        }
        // Count this wave in once its record has reached the coherent level.
        wait_stores();
        const uint32_t xf = m.before;                 // the sequence's first chunk in the list
        const uint32_t jf = wave_of(xf);
        const uint32_t nrec = wave_of(xf + nc - 1) - jf + 1;
        uint32_t* counter = a.counters + static_cast<uint64_t>(rg) * S + m.s;
        uint32_t prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = lane_value(prev, 0);
        if (prev != nrec - 1) return;
        if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // Last arrival: lane group grp_l combines records r = grp_l, grp_l + TPI, ...
        const uint64_t r0 = rec_base + jf + m.s;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float M = -INFINITY, Lsum = 0.0f;
            float A[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) A[e] = 0.0f;
            for (uint32_t r = grp_l; r < nrec; r += 4 * TPI) {
                float mr[4], lr[4];
                float ar[4][EPL];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t ri = r + u * TPI;
                    if (ri < nrec) {
                        const float* pa = a.part_acc + ((r0 + ri) * G + g) * HS + EPL * col;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) ar[u][e] = load_coherent(pa + e);
                        mr[u] = load_coherent(a.part_ml + ((r0 + ri) * G + g) * 2);
                        lr[u] = load_coherent(a.part_ml + ((r0 + ri) * G + g) * 2 + 1);
                    } else {
#pragma unroll
                        for (int e = 0; e < EPL; ++e) ar[u][e] = 0.0f;
                        mr[u] = -INFINITY;
                        lr[u] = 0.0f;
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (mr[u] == -INFINITY) continue;
                    const float Mn = fmaxf(M, mr[u]);
                    const float s0 = exp2f(M - Mn), s1 = exp2f(mr[u] - Mn);
                    Lsum = Lsum * s0 + lr[u] * s1;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) A[e] = A[e] * s0 + ar[u][e] * s1;
                    M = Mn;
                }
            }
            const float Mg = groups_max<LPT>(M);
            const float sc = M == -INFINITY ? 0.0f : exp2f(M - Mg);
            Lsum = groups_sum<LPT>(Lsum * sc);
#pragma unroll
            for (int e = 0; e < EPL; ++e) A[e] = groups_sum<LPT>(A[e] * sc);
            if (grp_l == 0) {
                const float inv = 1.0f / Lsum;
#pragma unroll
                for (int e = 0; e < EPL; ++e) A[e] *= inv;
                store_out(static_cast<uint64_t>(m.s) * a.num_heads + h0 + g, col, A);
            }
        }
    };

    // ---- pipeline: block ids two chunks ahead, rows one chunk ahead ----
    reset();
    Meta mc{cs, ck, cL, cbefore};
    uint64_t row_c[NL], row_n[NL];
    rows_of(mc, row_c);
    float qv[G][EPL], qn[G][EPL];
    load_q(mc.s, qv);
    Buf bA, bB;
    issue(row_c, bA);
    Meta mn = mc;
    if (x0 + 1 < x1) {
        advance();
        mn = Meta{cs, ck, cL, cbefore};
        rows_of(mn, row_n);
    }
    uint32_t kfirst = mc.k;

    auto step = [&](uint32_t x, Buf& cur, Buf& nxt) -> bool {
        const bool more = x + 1 < x1;
        if (more) {
            issue(row_n, nxt);
            if (mn.s != mc.s) load_q(mn.s, qn);
        }
        Meta m2 = mn;
        if (x + 2 < x1) {
            advance();
            m2 = Meta{cs, ck, cL, cbefore};
            rows_of(m2, row_n);
        }
        process(mc, cur, qv);
        if (!more || mn.s != mc.s) {
            flush(mc, kfirst);
            reset();
            kfirst = mn.k;
            if (more) {
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) qv[g][e] = qn[g][e];
            }
        }
        mc = mn;
        mn = m2;
        return more;
    };
    for (uint32_t x = x0;; x += 2) {
        if (!step(x, bA, bB)) break;
        if (!step(x + 1, bB, bA)) break;
    }
}

template <typename E, int LPT>
hipError_t launch_lpt(const BaselineDecodeArgs& a, dim3 grid, hipStream_t st) {
    switch (a.group) {
        case 4: hipLaunchKernelGGL((baseline_decode_kernel<E, LPT, 4>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((baseline_decode_kernel<E, LPT, 2>), grid, dim3(256), 0, st, a); break;
        default: hipLaunchKernelGGL((baseline_decode_kernel<E, LPT, 1>), grid, dim3(256), 0, st, a); break;
    }
    return hipGetLastError();
}

// head_size / EPL lanes per row
template <typename E>
hipError_t launch_elem(const BaselineDecodeArgs& a, dim3 grid, hipStream_t st) {
    constexpr int EPL = epl<E>();
    switch (a.head_size) {
        case 16: return launch_lpt<E, 16 / EPL>(a, grid, st);
        case 32: return launch_lpt<E, 32 / EPL>(a, grid, st);
        case 64: return launch_lpt<E, 64 / EPL>(a, grid, st);
        case 128: return launch_lpt<E, 128 / EPL>(a, grid, st);
        case 256: return launch_lpt<E, 256 / EPL>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_baseline_write(const BaselineWriteArgs& a, hipStream_t stream) {
    const uint32_t epl_ = a.elem_bytes == 2 ? 8u : 4u;
    const uint64_t n = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads * (a.head_size / epl_);
    const bool vec4 = (reinterpret_cast<uintptr_t>(a.key) % 16 == 0) && (reinterpret_cast<uintptr_t>(a.value) % 16 == 0) &&
                      a.key_stride % 4 == 0 && a.value_stride % 4 == 0;
    const dim3 grid(static_cast<uint32_t>((n + 255) / 256));
    if (a.elem_bytes == 2) hipLaunchKernelGGL(baseline_write_kernel<uint16_t>, grid, dim3(256), 0, stream, a, vec4);
    else hipLaunchKernelGGL(baseline_write_kernel<float>, grid, dim3(256), 0, stream, a, vec4);
    return hipGetLastError();
}

BaselineDecodePlan plan_baseline_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                                        uint32_t head_size) {
    BaselineDecodePlan p{};
    const uint32_t n_rep = num_heads / num_kv_heads;
    p.group = n_rep % 4 == 0 ? 4 : (n_rep % 2 == 0 ? 2 : 1);
    p.num_groups = n_rep / p.group;
    // Q8KV_F32_DECODE_WAVES overrides the persistent wave count of the f32
    // and bf16 decodes (tests use it to move the boundaries between the
    // waves' chunk ranges).
    uint64_t target = kBaselineDecodeWaves;
    if (const char* e = getenv("Q8KV_F32_DECODE_WAVES")) {
        const long v = atol(e);
        if (v >= 1 && v <= (1L << 20)) target = static_cast<uint64_t>(v);
    }
    const uint64_t num_rg = static_cast<uint64_t>(num_kv_heads) * p.num_groups;
    p.waves_per_rg = static_cast<uint32_t>(num_rg >= target ? 1 : target / num_rg);
    p.recs_per_rg = static_cast<uint64_t>(p.waves_per_rg) + (num_seqs ? num_seqs - 1 : 0);
    p.num_waves = num_rg * p.waves_per_rg;
    auto r256 = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t slots = static_cast<size_t>(num_rg) * p.recs_per_rg * p.group;
    p.counters_offset = 0;
    p.acc_offset = r256(static_cast<size_t>(num_rg) * num_seqs * 4);
    p.ml_offset = p.acc_offset + r256(slots * head_size * 4);
    p.bytes = p.ml_offset + slots * 2 * 4;
    return p;
}

hipError_t launch_baseline_decode(const BaselineDecodeArgs& a, const BaselineDecodePlan& p, hipStream_t st) {
    const dim3 grid(static_cast<uint32_t>((p.num_waves + 3) / 4));
    return a.elem_bytes == 2 ? launch_elem<uint16_t>(a, grid, st) : launch_elem<float>(a, grid, st);
}

}  // namespace q8kv
