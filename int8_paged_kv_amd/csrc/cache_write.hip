// Quantize + pack new K/V vectors into the int8 paged cache.
//
// Follows the "reshape_and_cache_q8.comp" page, main(), for each (token, kv
// head) and for K then V (the quantizer is in q8_pack.h).  A pad slot
// (0xFFFFFFFF) skips the token: nothing is written for it (its source rows
// may be read).
//
// MI355X mapping: one wavefront per (token, kv head).  When head_size <= 128
// the two 32-lane halves quantize K and V side by side; otherwise the whole
// wave does K and then V.  Each lane owns one code word: a 16-byte load of four
// f32 values, an amax reduction across the lanes of its half (or wave), four
// IEEE multiplies, v_rndne, clamp and a byte pack.
#include "q8kv_internal.h"
#include "q8_pack.h"

namespace q8kv {
namespace {

__device__ __forceinline__ float4 load4(const float* p, bool vec4) {
    if (vec4) return *reinterpret_cast<const float4*>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
}

template <bool HALF>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a, bool vec4) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t pair = static_cast<uint64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (pair >= static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads) return;
    const uint32_t t = static_cast<uint32_t>(pair / a.num_kv_heads);
    const uint32_t h = static_cast<uint32_t>(pair % a.num_kv_heads);
    const uint32_t hs4 = a.head_size / 4, wpt = hs4 + 1;
    const float* ksrc = a.key + static_cast<uint64_t>(t) * a.key_stride + static_cast<uint64_t>(h) * a.head_size;
    const float* vsrc = a.value + static_cast<uint64_t>(t) * a.value_stride + static_cast<uint64_t>(h) * a.head_size;
    // The source rows are loaded together with the slot (one memory round
    // trip instead of two); a pad token's rows may thus be read, but nothing
    // is written for it.
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (HALF) {
        const uint32_t w = lane & 31;
        if (w < hs4) x0 = load4((lane >= 32 ? vsrc : ksrc) + 4 * w, vec4);
    } else {
        if (lane < hs4) {
            x0 = load4(ksrc + 4 * lane, vec4);
            x1 = load4(vsrc + 4 * lane, vec4);
        }
    }
    const uint32_t slot = a.slot_mapping[t];
    if (slot == kPadSlot) return;
    const uint64_t block = slot / a.block_size, off = slot % a.block_size;
    if (block >= a.num_blocks) return;   // out of contract; skipped rather than written out of bounds
    const uint64_t dst = ((block * a.num_kv_heads + h) * a.block_size + off) * wpt;
    if (HALF) {
        pack_vector<32>(x0, (lane >= 32 ? a.value_cache : a.key_cache) + dst, hs4, lane & 31);
    } else {
        pack_vector<64>(x0, a.key_cache + dst, hs4, lane);
        pack_vector<64>(x1, a.value_cache + dst, hs4, lane);
    }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
    const uint64_t pairs = static_cast<uint64_t>(a.num_tokens) * a.num_kv_heads;
    const uint64_t blocks = (pairs + 3) / 4;
    const bool vec4 = (reinterpret_cast<uintptr_t>(a.key) % 16 == 0) &&
                      (reinterpret_cast<uintptr_t>(a.value) % 16 == 0) &&
                      a.key_stride % 4 == 0 && a.value_stride % 4 == 0;
    if (a.head_size / 4 <= 32)
        hipLaunchKernelGGL(cache_write_kernel<true>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, a, vec4);
    else
        hipLaunchKernelGGL(cache_write_kernel<false>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, a, vec4);
    return hipGetLastError();
}

}  // namespace q8kv
