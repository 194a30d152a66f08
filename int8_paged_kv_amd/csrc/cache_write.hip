// Quantize + pack new K/V vectors into the int8 paged cache.
//
// Follows the "reshape_and_cache_q8.comp" page, main(), for each (token, kv
// head) and for K then V (the quantizer is in q8_pack.h).  A pad slot
// (0xFFFFFFFF) skips the token: nothing is read or written for it.
//
// MI355X mapping: one wavefront per (token, kv head) in small writes.  In
// large ones a workgroup takes 16 consecutive tokens of one kv head, four per
// wave with all their loads in flight together: when those tokens fill a block
// in order (a prefill), the workgroup writes that block's whole tile for the
// head from one compute unit, so its L2 assembles full lines before they go
// to memory (rows written from different XCDs leave partial lines, which cost
// the memory a read-modify-write each).  When head_size <= 128 the two 32-lane
// halves quantize K and V side by side; otherwise the whole wave does K and
// then V.  Each lane owns one code word: a 16-byte load of four f32 values,
// an amax reduction across the lanes of its half (or wave), four IEEE
// multiplies, v_rndne, clamp and a byte pack.
#include "q8kv_internal.h"
#include "bounds.h"
#include "q8_pack.h"
#include "wave_ops.h"

namespace q8kv {
namespace {

__device__ __forceinline__ float4 load4(const float* p, bool vec4) {
    if (vec4) return *reinterpret_cast<const float4*>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
}

// NP (token, kv head) pairs per wave.  TILES: workgroup b takes tokens
// 16*(b / num_kv_heads) .. +15 of kv head b % num_kv_heads, wave w the NP = 4
// consecutive tokens from 16*(b / num_kv_heads) + 4*w.  Otherwise a wave takes
// NP consecutive pairs of the (token, kv head) order.  Every pair's slot, then
// every non-pad pair's rows, are loaded before any is packed, so a wave keeps
// NP rows in flight.
template <bool HALF, int NP, bool TILES>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a, bool vec4) {
    static_assert(!TILES || NP * 4 == 16, "a workgroup of four waves covers 16 tokens");
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = uniform(threadIdx.x / kWave);
    const uint32_t hs4 = a.head_size / 4, wpt = hs4 + 1;
    // The slots come first (scalar loads of the wave's tokens); then only the
    // rows of non-pad tokens are loaded, all of them before any is packed.
    float4 x0[NP], x1[NP];
    uint32_t slot[NP], head[NP], tok[NP];
    if (TILES) {
        const uint32_t h = blockIdx.x % a.num_kv_heads;
        const uint64_t t0 = static_cast<uint64_t>(blockIdx.x / a.num_kv_heads) * 16 + wave * NP;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            slot[i] = kPadSlot;
            head[i] = h;
            tok[i] = static_cast<uint32_t>(t0 + i);
            if (t0 + i < a.num_tokens) slot[i] = a.slot_mapping[t0 + i];     // wave-uniform
        }
    } else {
        // Wave-uniform pair indices (slots become scalar loads); one division
        // per wave, the later pairs step through the heads.
        const uint64_t first = (static_cast<uint64_t>(blockIdx.x) * (blockDim.x / kWave) + wave) * NP;
        const uint64_t pairs = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads;
        if (first >= pairs) return;
        uint32_t t = static_cast<uint32_t>(first / a.num_kv_heads);
        uint32_t h = static_cast<uint32_t>(first - static_cast<uint64_t>(t) * a.num_kv_heads);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            slot[i] = kPadSlot;
            if (i > 0 && ++h == a.num_kv_heads) h = 0, ++t;
            head[i] = h;
            tok[i] = t;
            if (first + i < pairs) slot[i] = a.slot_mapping[t];     // wave-uniform
        }
    }
    uint32_t t, h;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        x0[i] = x1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (slot[i] == kPadSlot) continue;           // wave-uniform: nothing is read for a pad token
        t = tok[i];
        h = head[i];
        const float* ksrc = a.key + static_cast<uint64_t>(t) * a.key_stride + static_cast<uint64_t>(h) * a.head_size;
        const float* vsrc = a.value + static_cast<uint64_t>(t) * a.value_stride + static_cast<uint64_t>(h) * a.head_size;
        if (HALF) {
            const uint32_t w = lane & 31;
            if (w < hs4) x0[i] = load4((lane >= 32 ? vsrc : ksrc) + 4 * w, vec4);
        } else if (lane < hs4) {
            x0[i] = load4(ksrc + 4 * lane, vec4);
            x1[i] = load4(vsrc + 4 * lane, vec4);
        }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        if (slot[i] == kPadSlot) continue;
        const uint32_t block = slot[i] / a.block_size, off = slot[i] - block * a.block_size;
        bounds_report(a.bounds_flags, block >= a.num_blocks, kBoundSlot);
        if (block >= a.num_blocks) continue;         // out of contract; skipped rather than written out of bounds
        const uint64_t dst = ((static_cast<uint64_t>(block) * a.num_kv_heads + head[i]) * a.block_size + off) * wpt;
        if (HALF) {
            pack_vector<32>(x0[i], (lane >= 32 ? a.value_cache : a.key_cache) + dst, hs4, lane & 31);
        } else {
            pack_vector<64>(x0[i], a.key_cache + dst, hs4, lane);
            pack_vector<64>(x1[i], a.value_cache + dst, hs4, lane);
        }
    }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
    const uint64_t pairs = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads;
    const bool vec4 = (reinterpret_cast<uintptr_t>(a.key) % 16 == 0) &&
                      (reinterpret_cast<uintptr_t>(a.value) % 16 == 0) &&
                      a.key_stride % 4 == 0 && a.value_stride % 4 == 0;
    const bool half = a.head_size / 4 <= 32;
    const uint64_t blocks = cache_write_blocks(a.num_tokens, a.num_kv_heads);
    if (blocks == 0 || blocks > kMaxGridBlocks) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<uint32_t>(blocks));
    if (pairs >= kWriteBatchMinPairs) {
        if (half) hipLaunchKernelGGL((cache_write_kernel<true, kWritePairsPerWave, true>), grid, dim3(256), 0, stream, a, vec4);
        else hipLaunchKernelGGL((cache_write_kernel<false, kWritePairsPerWave, true>), grid, dim3(256), 0, stream, a, vec4);
    } else {
        if (half) hipLaunchKernelGGL((cache_write_kernel<true, 1, false>), grid, dim3(256), 0, stream, a, vec4);
        else hipLaunchKernelGGL((cache_write_kernel<false, 1, false>), grid, dim3(256), 0, stream, a, vec4);
    }
    return hipGetLastError();
}

}  // namespace q8kv
