// Measurement kernels for the practical HBM ceiling next to the decode
// (libq8kv_bench.so; only the benchmark loads it).  Neither computes anything
// of the method: each reads device memory with 16-byte nontemporal loads,
// folds what it read into one word per wavefront so the loads are not
// removed, and writes that word.
//   q8b_stream_read  -- one contiguous buffer, read once (the streaming rate).
//   q8b_tile_gather  -- the decode's access pattern without its arithmetic: a
//                       list of cache tiles (one (block, kv head) run of rows
//                       each) read from the K and the V cache.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* src, uint64_t n16, uint32_t* sink) {
    const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    uint32_t acc = 0;
    for (uint64_t i = tid; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // one word per wave
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if (threadIdx.x % 64 == 0) sink[tid / 64] = acc;
}

// Wave w of W reads the contiguous range [w*n/W, (w+1)*n/W) of the tile
// list, two tiles at a time with all their loads in flight; tile t is
// tile_u4 16-byte units (at most 192) at unit offset tiles[t] of both caches.
// (The best of the structures measured for the decode's tiles: ranges of
// pairs over 2048 waves.)
__global__ __launch_bounds__(256) void tile_gather_kernel(const u32x4* kc, const u32x4* vc, const uint64_t* tiles,
                                                          uint32_t num_tiles, uint32_t tile_u4, uint32_t* sink) {
    const uint32_t lane = threadIdx.x % 64;
    const uint32_t wave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const uint32_t nw = gridDim.x * (blockDim.x / 64);
    const uint32_t t0 = static_cast<uint32_t>(static_cast<uint64_t>(wave) * num_tiles / nw);
    const uint32_t t1 = static_cast<uint32_t>(static_cast<uint64_t>(wave + 1) * num_tiles / nw);
    uint32_t acc = 0;
    for (uint32_t t = t0; t < t1; t += 2) {
        u32x4 a[2][3], b[2][3];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint64_t base = tiles[t + i < t1 ? t + i : t1 - 1];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const uint32_t u = lane + 64 * j;
                const uint32_t uu = u < tile_u4 ? u : 0;     // units past the tile re-read its first one
                a[i][j] = __builtin_nontemporal_load(kc + base + uu);
                b[i][j] = __builtin_nontemporal_load(vc + base + uu);
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) acc ^= a[i][j].x ^ a[i][j].y ^ a[i][j].z ^ a[i][j].w ^ b[i][j].x ^ b[i][j].y ^
                                               b[i][j].z ^ b[i][j].w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if (lane == 0) sink[wave] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at 16-byte aligned `src`; writes
// `waves` words to sink (waves = grid_blocks * 4).  Returns a hipError_t.
int q8b_stream_read(const void* src, uint64_t bytes, uint32_t* sink, uint32_t grid_blocks, void* stream) {
    if (!src || !sink || bytes % 16 != 0 || grid_blocks == 0) return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid_blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    return static_cast<int>(hipGetLastError());
}

// Reads num_tiles tiles of tile_u4 16-byte units (1 to 192) from each cache
// at the unit offsets tiles[0 .. num_tiles) (device array); the caller keeps
// every tile inside both caches.  Writes grid_blocks * 4 words to sink.
int q8b_tile_gather(const void* key_cache, const void* value_cache, const uint64_t* tiles, uint32_t num_tiles,
                    uint32_t tile_u4, uint32_t* sink, uint32_t grid_blocks, void* stream) {
    if (!key_cache || !value_cache || !tiles || !sink || grid_blocks == 0 || tile_u4 == 0 || tile_u4 > 192)
        return static_cast<int>(hipErrorInvalidValue);
    hipLaunchKernelGGL(tile_gather_kernel, dim3(grid_blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(key_cache), static_cast<const u32x4*>(value_cache), tiles, num_tiles,
                       tile_u4, sink);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
