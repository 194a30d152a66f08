// Device-side checks of the callers' array contents, compiled in only when
// Q8_DEBUG_BOUNDS is defined (libq8kv_debug.so).  The release library trusts
// the contents, as the pages' shaders do; it only clamps reads and skips
// writes that would leave the caches.  A failed check sets its bit in a
// device flag word (q8_bounds_flags reads it back) and changes nothing else:
// every kernel still clamps or skips as in the release build.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8kv {

constexpr uint32_t kBoundSlot = 1u;      // cache write: slot past the cache that is not the pad value
constexpr uint32_t kBoundBlock = 2u;     // decode / step: block id of an attended or appended position past the cache
constexpr uint32_t kBoundTable = 4u;     // decode: positions of a sequence past its block-table row
constexpr uint32_t kBoundVisible = 8u;   // visible list: count past vis_stride, or a chunk not ascending and distinct

__device__ __forceinline__ void bounds_report(uint32_t* flags, bool bad, uint32_t bit) {
#ifdef Q8_DEBUG_BOUNDS
    if (bad && flags != nullptr) {
        // a vector atomic by the failing lanes (the address goes through a
        // vector register)
        uintptr_t p = reinterpret_cast<uintptr_t>(flags);
        asm volatile("" : "+v"(p));
        __hip_atomic_fetch_or(reinterpret_cast<uint32_t*>(p), bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#else
    (void)flags;
    (void)bad;
    (void)bit;
#endif
}

}  // namespace q8kv
