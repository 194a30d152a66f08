// f32 paged-cache baseline: cache writer and single-query decode.
//
// The "paged_attn_q8.comp" page's header says the int8 decode keeps the math
// and workgroup structure of an f32 paged decode whose cache holds 4 bytes per
// element (the int8 cache's point being the 4x smaller read), and the
// "reshape_and_cache_q8.comp" page's header says its pad-slot rule mirrors the
// f32 writer.  The f32 layout is not printed there; it is taken to be the int8
// layout with one f32 per element: [num_blocks, num_kv_heads, block_size,
// head_size].  These kernels serve to measure the int8 cache against the f32
// one on the same batch.
//
// Decode, MI355X mapping.  The work is a pure stream of f32 rows with about
// one multiply-add per byte, far below the VALU rate, so it stays on the VALU
// and is laid out for the loads:
//   * A row of head_size f32 is read by LPT = head_size/4 lanes with 16-byte
//     loads; one load instruction covers 64/LPT consecutive positions, and a
//     chunk is 8 such loads per tensor (8 KiB of K and 8 KiB of V per wave),
//     fetched into registers one chunk ahead, the block ids two chunks ahead.
//   * A wave handles one row group: a kv head and G = 4, 2 or 1 of its query
//     heads, whose q slices stay in registers.  q.k is a 4-element partial
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
    if (LPT <= 4) v += dpp_mov<kRowRor4>(v);
    if (LPT <= 8) v += dpp_mov<kRowRor8>(v);
    if (LPT <= 16) v += swizzle_xor16(v);
    if (LPT <= 32) v += xor32(v);
    return v;
}

__device__ __forceinline__ float4 f4_zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }

typedef float f32x4 __attribute__((ext_vector_type(4)));   // vector type the nontemporal builtins accept

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

__global__ __launch_bounds__(256) void f32_cache_write_kernel(F32CacheWriteArgs a, bool vec4) {
    const uint32_t hs4 = a.head_size / 4;
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads * hs4) return;
    const uint32_t w = static_cast<uint32_t>(i % hs4);
    const uint64_t th = i / hs4;
    const uint32_t h = static_cast<uint32_t>(th % a.num_kv_heads);
    const uint32_t t = static_cast<uint32_t>(th / a.num_kv_heads);
    const uint32_t slot = a.slot_mapping[t];
    if (slot == kPadSlot) return;
    const uint64_t block = slot / a.block_size, off = slot % a.block_size;
    if (block >= a.num_blocks) return;   // out of contract; skipped rather than written out of bounds
    const float* ks = a.key + static_cast<uint64_t>(t) * a.key_stride + static_cast<uint64_t>(h) * a.head_size + 4 * w;
    const float* vs = a.value + static_cast<uint64_t>(t) * a.value_stride + static_cast<uint64_t>(h) * a.head_size + 4 * w;
    const float4 k = vec4 ? *reinterpret_cast<const float4*>(ks) : make_float4(ks[0], ks[1], ks[2], ks[3]);
    const float4 v = vec4 ? *reinterpret_cast<const float4*>(vs) : make_float4(vs[0], vs[1], vs[2], vs[3]);
    const uint64_t dst = ((block * a.num_kv_heads + h) * a.block_size + off) * a.head_size + 4 * w;
    *reinterpret_cast<float4*>(a.key_cache + dst) = k;
    *reinterpret_cast<float4*>(a.value_cache + dst) = v;
}

// ---------------------------------------------------------------- decode ----

// Positions of sequence s (the context clamp applied).
__device__ __forceinline__ uint32_t f32_positions(const F32DecodeArgs& a, uint32_t s) {
    const uint32_t L = a.context_lens[s];
    return L < a.max_context_len ? L : a.max_context_len;
}

template <int LPT, int G>
__global__ __launch_bounds__(256, 2) void f32_decode_kernel(F32DecodeArgs a) {
    constexpr int TPI = kWave / LPT;                    // positions per load instruction
    constexpr uint32_t T = kLoadsPerChunk * TPI;        // positions per chunk
    constexpr uint32_t HS = 4 * LPT;
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

    // ---- chunk count C of the row group; empty sequences s = j (mod W) get zero rows ----
    uint32_t C = 0;
    for (uint32_t base = 0; base < S; base += kWave) {
        const uint32_t s = base + lane;
        const uint32_t L = s < S ? f32_positions(a, s) : 0;
        const uint32_t nc = (L + T - 1) / T;
        const uint32_t incl = wave_incl_scan(nc, lane);
        C += lane_value(incl, kWave - 1);
        uint64_t zmask = __ballot(s < S && L == 0 && s % W == j);
        while (zmask) {
            const uint32_t zs = base + static_cast<uint32_t>(__builtin_ctzll(zmask));
            zmask &= zmask - 1;
            for (uint32_t e = lane; e < G * LPT; e += kWave) {
                const uint32_t g = e / LPT, c4 = e % LPT;
                *reinterpret_cast<float4*>(a.out + (static_cast<uint64_t>(zs) * a.num_heads + h0 + g) * HS + 4 * c4) =
                    f4_zero();
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
            const uint32_t nc = s < S ? (f32_positions(a, s) + T - 1) / T : 0;
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
    uint32_t cL = uniform(f32_positions(a, cs));

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
                cL = uniform(f32_positions(a, cs));
            } while (cL == 0);
        }
    };

    const float* kbase = a.key_cache + static_cast<uint64_t>(kvh) * a.block_size * HS + 4 * col;
    const float* vbase = a.value_cache + static_cast<uint64_t>(kvh) * a.block_size * HS + 4 * col;
    const uint64_t block_stride = static_cast<uint64_t>(a.num_kv_heads) * a.block_size * HS;

    // Row offsets (floats from kbase) of the lane's positions in chunk m; an
    // invalid position gets ~0u.
    auto rows_of = [&](const Meta& m, uint64_t (&row)[kLoadsPerChunk]) {
        const uint32_t c0 = m.k * T;
        const uint32_t q0 = c0 / a.block_size, r0 = c0 % a.block_size;
        const uint32_t* bt = a.block_tables + static_cast<uint64_t>(m.s) * a.max_num_blocks_per_seq;
#pragma unroll
        for (int i = 0; i < kLoadsPerChunk; ++i) {
            const uint32_t d = i * TPI + grp_l;
            const uint32_t t = r0 + d;
            // t < block_size + T: one step when block_size >= T, else an exact
            // float quotient (t < 256, so t + 1/2 is at least 1/256 of a block
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

    struct Buf {
        f32x4 k[kLoadsPerChunk], v[kLoadsPerChunk];
    };
    auto issue = [&](const uint64_t (&row)[kLoadsPerChunk], Buf& b) {
#pragma unroll
        for (int i = 0; i < kLoadsPerChunk; ++i) {
            if (row[i] != ~0ull) {
                b.k[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kbase + row[i]));
                b.v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vbase + row[i]));
            } else {
                b.k[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                b.v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto load_q = [&](uint32_t s, float4 (&qv)[G]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float4 x = *reinterpret_cast<const float4*>(a.q + static_cast<uint64_t>(s) * a.q_stride +
                                                        static_cast<uint64_t>(h0 + g) * HS + 4 * col);
            qv[g] = make_float4(x.x * a.scale_log2, x.y * a.scale_log2, x.z * a.scale_log2, x.w * a.scale_log2);
        }
    };

    // Online-softmax state of the current piece.
    float m_run[G], l_run[G];
    float4 acc[G];
    auto reset = [&]() {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m_run[g] = -INFINITY;
            l_run[g] = 0.0f;
            acc[g] = f4_zero();
        }
    };

    auto process = [&](const Meta& m, const Buf& b, const float4 (&qv)[G]) {
        const uint32_t c0 = m.k * T;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float z[kLoadsPerChunk];
            float cmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < kLoadsPerChunk; ++i) {
                float p = qv[g].x * b.k[i].x;
                p = fmaf(qv[g].y, b.k[i].y, p);
                p = fmaf(qv[g].z, b.k[i].z, p);
                p = fmaf(qv[g].w, b.k[i].w, p);
                p = group_sum<LPT>(p);
                z[i] = c0 + i * TPI + grp_l < m.L ? p : -INFINITY;
                cmax = fmaxf(cmax, z[i]);
            }
            const float mn = fmaxf(m_run[g], groups_max<LPT>(cmax));   // finite: the chunk holds a position
            const float alpha = exp2f(m_run[g] - mn);
            m_run[g] = mn;
            float l = l_run[g] * alpha;
            float4 o = make_float4(acc[g].x * alpha, acc[g].y * alpha, acc[g].z * alpha, acc[g].w * alpha);
#pragma unroll
            for (int i = 0; i < kLoadsPerChunk; ++i) {
                const float p = exp2f(z[i] - mn);
                l += p;
                o.x = fmaf(p, b.v[i].x, o.x);
                o.y = fmaf(p, b.v[i].y, o.y);
                o.z = fmaf(p, b.v[i].z, o.z);
                o.w = fmaf(p, b.v[i].w, o.w);
            }
            l_run[g] = l;
            acc[g] = o;
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
        float4 o[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            l_tot[g] = groups_sum<LPT>(l_run[g]);
            o[g] = make_float4(groups_sum<LPT>(acc[g].x), groups_sum<LPT>(acc[g].y), groups_sum<LPT>(acc[g].z),
                               groups_sum<LPT>(acc[g].w));
        }
        if (kfirst == 0 && m.k + 1 == nc) {
            if (grp_l == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float inv = 1.0f / l_tot[g];
                    *reinterpret_cast<float4*>(a.out + (static_cast<uint64_t>(m.s) * a.num_heads + h0 + g) * HS +
                                               4 * col) =
                        make_float4(o[g].x * inv, o[g].y * inv, o[g].z * inv, o[g].w * inv);
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
                float* pa = a.part_acc + (rec * G + g) * HS + 4 * col;
                store_coherent(pa + 0, o[g].x);
                store_coherent(pa + 1, o[g].y);
                store_coherent(pa + 2, o[g].z);
                store_coherent(pa + 3, o[g].w);
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
            float4 A = f4_zero();
            for (uint32_t r = grp_l; r < nrec; r += 4 * TPI) {
                float mr[4], lr[4];
                float4 ar[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t ri = r + u * TPI;
                    if (ri < nrec) {
                        const float* pa = a.part_acc + ((r0 + ri) * G + g) * HS + 4 * col;
                        ar[u] = make_float4(load_coherent(pa), load_coherent(pa + 1), load_coherent(pa + 2),
                                            load_coherent(pa + 3));
                        mr[u] = load_coherent(a.part_ml + ((r0 + ri) * G + g) * 2);
                        lr[u] = load_coherent(a.part_ml + ((r0 + ri) * G + g) * 2 + 1);
                    } else {
                        ar[u] = f4_zero();
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
                    A = make_float4(A.x * s0 + ar[u].x * s1, A.y * s0 + ar[u].y * s1, A.z * s0 + ar[u].z * s1,
                                    A.w * s0 + ar[u].w * s1);
                    M = Mn;
                }
            }
            const float Mg = groups_max<LPT>(M);
            const float sc = M == -INFINITY ? 0.0f : exp2f(M - Mg);
            Lsum = groups_sum<LPT>(Lsum * sc);
            A = make_float4(groups_sum<LPT>(A.x * sc), groups_sum<LPT>(A.y * sc), groups_sum<LPT>(A.z * sc),
                            groups_sum<LPT>(A.w * sc));
            if (grp_l == 0) {
                const float inv = 1.0f / Lsum;
                *reinterpret_cast<float4*>(a.out + (static_cast<uint64_t>(m.s) * a.num_heads + h0 + g) * HS +
                                           4 * col) = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
            }
        }
    };

    // ---- pipeline: block ids two chunks ahead, rows one chunk ahead ----
    reset();
    Meta mc{cs, ck, cL, cbefore};
    uint64_t row_c[kLoadsPerChunk], row_n[kLoadsPerChunk];
    rows_of(mc, row_c);
    float4 qv[G], qn[G];
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
                for (int g = 0; g < G; ++g) qv[g] = qn[g];
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

template <int LPT>
hipError_t launch_lpt(const F32DecodeArgs& a, dim3 grid, hipStream_t st) {
    switch (a.group) {
        case 4: hipLaunchKernelGGL((f32_decode_kernel<LPT, 4>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((f32_decode_kernel<LPT, 2>), grid, dim3(256), 0, st, a); break;
        default: hipLaunchKernelGGL((f32_decode_kernel<LPT, 1>), grid, dim3(256), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_f32_cache_write(const F32CacheWriteArgs& a, hipStream_t stream) {
    const uint64_t n = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads * (a.head_size / 4);
    const bool vec4 = (reinterpret_cast<uintptr_t>(a.key) % 16 == 0) && (reinterpret_cast<uintptr_t>(a.value) % 16 == 0) &&
                      a.key_stride % 4 == 0 && a.value_stride % 4 == 0;
    hipLaunchKernelGGL(f32_cache_write_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream, a, vec4);
    return hipGetLastError();
}

F32DecodePlan plan_f32_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads, uint32_t head_size) {
    F32DecodePlan p{};
    const uint32_t n_rep = num_heads / num_kv_heads;
    p.group = n_rep % 4 == 0 ? 4 : (n_rep % 2 == 0 ? 2 : 1);
    p.num_groups = n_rep / p.group;
    // Q8KV_F32_DECODE_WAVES overrides the persistent wave count (tests use it
    // to move the boundaries between the waves' chunk ranges).
    uint64_t target = kF32DecodeWaves;
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

hipError_t launch_f32_decode(const F32DecodeArgs& a, const F32DecodePlan& p, hipStream_t st) {
    const dim3 grid(static_cast<uint32_t>((p.num_waves + 3) / 4));
    switch (a.head_size) {
        case 16: return launch_lpt<4>(a, grid, st);
        case 32: return launch_lpt<8>(a, grid, st);
        case 64: return launch_lpt<16>(a, grid, st);
        case 128: return launch_lpt<32>(a, grid, st);
        case 256: return launch_lpt<64>(a, grid, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace q8kv
