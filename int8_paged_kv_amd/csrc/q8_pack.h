// Quantize + pack of one K or V vector, shared by the cache writer and the
// decode step that appends a token while it attends.
//
// Follows the "reshape_and_cache_q8.comp" page, main(): amax = max|x| (from
// 0), inv = amax > 0 ? 127/amax : 0, code = clamp(round(x * inv), -127, 127)
// packed four per u32 word with element 4w+l in byte l, then one word with the
// bits of amax/127 (1.0 when amax == 0).  round() is round-half-even.  Every
// step is a single binary32 operation with round-to-nearest, so the packed
// words are bit-exact (no FMA contraction applies: there is no add).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "lane_reduce.h"

namespace q8kv {

__device__ __forceinline__ uint32_t pack_code(float x, float inv, uint32_t lane_byte) {
    float r = __builtin_rintf(x * inv);          // nearest, ties to even
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu) << (8u * lane_byte);
}

// Lane w of a group of WIDTH lanes holds elements 4w .. 4w+3 of the vector in
// x (zeros for w >= head_size/4).  Returns the lane's code word and sets
// scale_bits, the bits of the vector's scale word (the same in every lane).
// Every lane of the wave must be active.
template <int WIDTH>
__device__ __forceinline__ uint32_t quantize_word(float4 x, uint32_t& scale_bits) {
    const float amax = group_max<WIDTH>(fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    const float inv = amax > 0.0f ? __fdiv_rn(127.0f, amax) : 0.0f;
    scale_bits = __float_as_uint(amax > 0.0f ? __fdiv_rn(amax, 127.0f) : 1.0f);
    return pack_code(x.x, inv, 0) | pack_code(x.y, inv, 1) | pack_code(x.z, inv, 2) | pack_code(x.w, inv, 3);
}

// Packs the vector into dst[0 .. hs4] (hs4 = head_size/4 code words, then
// the scale word) with the lanes [0, WIDTH) of a group; lane w is w.
template <int WIDTH>
__device__ __forceinline__ void pack_vector(float4 x, uint32_t* dst, uint32_t hs4, uint32_t w) {
    uint32_t scale_bits;
    const uint32_t word = quantize_word<WIDTH>(x, scale_bits);
    if (w < hs4) dst[w] = word;
    if (w == 0) dst[hs4] = scale_bits;
}

}  // namespace q8kv
