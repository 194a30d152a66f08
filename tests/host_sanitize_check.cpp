// Host-side checks of libq8kv's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure; no GPU is touched).
//
// Built by tests/test_host_sanitize.py from the library's own api.hip,
// decode.hip and baseline_cache.hip (their validation, split planning and
// workspace sizing), with the host pass instrumented.  The launchers of the
// other translation units are replaced below by stubs that report an error:
// no call here reaches a kernel.  Each entry point is called with arguments
// that fail validation (every documented error code, in exactly sized heap
// argument blocks where arrays are read), and the workspace queries over a
// grid of shapes up to 32-bit extremes, checking the properties the launches
// rely on (a workspace sized at the wave bound is never smaller than a
// launch's own plan; no workspace for at most 32 positions; offsets inside
// the buffer).  Prints "ok"; a sanitizer report or a failed check aborts.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <initializer_list>

#include "q8kv.h"
#include "decode_split.h"

namespace q8kv {
hipError_t launch_cache_write(const CacheWriteArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_index_select(const IndexSelectArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_rope_table(float*, uint32_t, uint32_t, double, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_norm_rope(const NormRopeArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_norm_rope_cache_write(const NormRopeCacheWriteArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_norm_rope_qk_cache_write(const NormRopeArgs&, const NormRopeCacheWriteArgs&, hipStream_t) {
    return hipErrorInvalidValue;
}
const void* split_kernel_hs16(bool, bool, bool, uint32_t, uint32_t) { return nullptr; }
const void* split_kernel_hs32(bool, bool, bool, uint32_t, uint32_t) { return nullptr; }
const void* split_kernel_hs48(bool, bool, bool, uint32_t, uint32_t) { return nullptr; }
const void* split_kernel_hs64(bool, bool, bool, uint32_t, uint32_t) { return nullptr; }
const void* split_kernel_nr_hs16(uint32_t, uint32_t) { return nullptr; }
const void* split_kernel_nr_hs32(uint32_t, uint32_t) { return nullptr; }
const void* split_kernel_nr_hs64(uint32_t, uint32_t) { return nullptr; }
}  // namespace q8kv

static int failures = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "line %d: %s\n", __LINE__, #cond);                \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

// Never dereferenced: every call below stops in validation.
static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static void workspace_properties() {
    const uint32_t seqs[] = {0, 1, 2, 63, 64, 65, 1000, 65535, 0xFFFFFFFFu};
    const uint32_t heads[][2] = {{1, 1}, {4, 2}, {32, 8}, {64, 8}, {16, 16}, {128, 1}, {0xFFFFu, 0xFFFFu}};
    const uint32_t hss[] = {4, 64, 68, 128, 192, 256};
    const uint32_t poss[] = {0, 1, 32, 33, 64, 4096, 32768, 0xFFFFFFFFu};
    for (uint32_t S : seqs)
        for (auto& hh : heads)
            for (uint32_t hs : hss)
                for (uint32_t mp : poss) {
                    const size_t b = q8_paged_decode_workspace_bytes(S, hh[0], hh[1], hs, 16, mp);
                    if (mp <= 32) EXPECT(b == 0);
                    // the launch's own plan for any wave count up to the bound fits the query's bytes
                    for (uint64_t w : {uint64_t(1), uint64_t(7), uint64_t(256), uint64_t(q8kv::kMaxDecodeWaves)}) {
                        const q8kv::DecodePlan p = q8kv::plan_decode(S, hh[0], hh[1], hs, 16, mp, w);
                        EXPECT(p.bytes <= b);
                        if (p.bytes) {
                            EXPECT(p.acc_offset % 256 == 0 && p.ml_offset % 256 == 0);
                            EXPECT(p.counters_offset < p.acc_offset || S == 0);
                            EXPECT(p.ml_offset >= p.acc_offset && p.ml_offset <= p.bytes);
                        }
                    }
                }
    EXPECT(q8_paged_decode_workspace_bytes(4, 3, 2, 128, 16, 1000) == 0);     // heads not a multiple of kv heads
    EXPECT(q8_paged_decode_workspace_bytes(4, 3, 0, 128, 16, 1000) == 0);
    EXPECT(q8_f32_paged_decode_workspace_bytes(4, 3, 2, 128) == 0);
    for (uint32_t S : seqs)
        for (auto& hh : heads) (void)q8_f32_paged_decode_workspace_bytes(S, hh[0], hh[1], 128);
}

static void decode_validation() {
    float* out = static_cast<float*>(fake(0x1000));
    const float* q = static_cast<const float*>(fake(0x2000));
    const uint32_t* u = static_cast<const uint32_t*>(fake(0x3000));
    void* ws = fake(0x4000);
    // shape errors
    EXPECT(q8_paged_decode(out, q, 512, u, u, u, 8, u, 100, nullptr, nullptr, 0, 2, 4, 2, 130, 16, 64, 0.1f, ws, 1u << 30,
                           nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_paged_decode(out, q, 512, u, u, u, 8, u, 100, nullptr, nullptr, 0, 2, 5, 2, 128, 16, 64, 0.1f, ws, 1u << 30,
                           nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_paged_decode(out, q, 100, u, u, u, 8, u, 100, nullptr, nullptr, 0, 2, 4, 2, 128, 16, 64, 0.1f, ws, 1u << 30,
                           nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_paged_decode(out, q, 512, u, u, u, 8, u, 100, u, u, 0, 2, 4, 2, 128, 16, 64, 0.1f, ws, 1u << 30,
                           nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_paged_decode(out, q, 512, u, u, u, 8, u, 100, nullptr, nullptr, 0, 2, 4, 2, 128, 16, 64, 0.0f / 0.0f, ws,
                           1u << 30, nullptr) == Q8_ERR_SHAPE);
    // null and workspace errors
    EXPECT(q8_paged_decode(nullptr, q, 512, u, u, u, 8, u, 100, nullptr, nullptr, 0, 2, 4, 2, 128, 16, 64, 0.1f, ws,
                           1u << 30, nullptr) == Q8_ERR_NULL);
    EXPECT(q8_paged_decode(out, q, 512, u, u, u, 8, u, 100, nullptr, nullptr, 0, 2, 4, 2, 128, 16, 64, 0.1f, nullptr, 0,
                           nullptr) == Q8_ERR_WORKSPACE);
    EXPECT(q8_paged_decode(out, q, 512, u, u, u, 8, u, 100, nullptr, nullptr, 0, 2, 4, 2, 128, 16, 64, 0.1f, fake(0x4004),
                           1u << 30, nullptr) == Q8_ERR_WORKSPACE);
    EXPECT(q8_paged_decode(static_cast<float*>(fake(0x1004)), q, 512, u, u, u, 8, u, 100, nullptr, nullptr, 0, 2, 4, 2,
                           128, 16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_UNSUPPORTED);
    EXPECT(q8_paged_decode(out, q, 512, u, u, u, 8, u, 100, nullptr, nullptr, 0, 0, 4, 2, 128, 16, 64, 0.1f, ws, 1u << 30,
                           nullptr) == Q8_OK);
    // extremes: 2^32-1 sequences and heads, huge strides (64-bit sizing, no overflow)
    const q8_status st = q8_paged_decode(out, q, 0xFFFFFFFFu, u, u, u, 0xFFFFFFFFu, u, 0xFFFFFFFFu, nullptr, nullptr, 0,
                                         0xFFFFFFFFu, 0xFFFF0000u, 0xFFFF0000u, 256, 0xFFFFFFFFu, 0xFFFFFFFFu, 1.0f, ws,
                                         1u << 30, nullptr);
    EXPECT(st == Q8_ERR_SHAPE || st == Q8_ERR_UNSUPPORTED || st == Q8_ERR_WORKSPACE);
    // the decode without a workspace: sizes beyond its scratch rejected before any device call
    EXPECT(q8_paged_decode_noalloc(out, q, 16 * 256, u, u, u, 8, u, 5000, nullptr, nullptr, 0, 100000, 16, 16, 256, 16,
                                   64, 0.1f, nullptr) == Q8_ERR_WORKSPACE);
    // decode step and multi-row decode
    const float* k = q;
    EXPECT(q8_decode_step(out, q, 512, nullptr, 256, k, 256, const_cast<uint32_t*>(u), const_cast<uint32_t*>(u), u, 8,
                          u, 100, 2, 4, 2, 128, 16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_NULL);
    EXPECT(q8_decode_step(out, q, 512, k, 255, k, 256, const_cast<uint32_t*>(u), const_cast<uint32_t*>(u), u, 8, u,
                          100, 2, 4, 2, 128, 16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_paged_decode_rows(out, q, 512, u, u, u, 8, u, 100, 0, 2, 4, 2, 128, 16, 64, 0.1f, ws, 1u << 30, nullptr) ==
           Q8_ERR_SHAPE);
    EXPECT(q8_paged_decode_rows(out, q, 512, u, u, u, 8, u, 100, 0xFFFFFFFFu, 0xFFFFFFFFu, 4, 2, 128, 16, 64, 0.1f, ws,
                                1u << 30, nullptr) == Q8_ERR_UNSUPPORTED);
    // f32 baseline
    EXPECT(q8_f32_paged_decode(out, q, 512, reinterpret_cast<const float*>(u), reinterpret_cast<const float*>(u), u, 8, u,
                               100, 2, 4, 2, 96, 16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_UNSUPPORTED);
    EXPECT(q8_f32_paged_decode(out, q, 512, reinterpret_cast<const float*>(u), reinterpret_cast<const float*>(u), u, 8, u,
                               100, 2, 4, 2, 128, 16, 64, 0.1f, nullptr, 0, nullptr) == Q8_ERR_WORKSPACE);
    // bf16 baseline
    const uint16_t* b = reinterpret_cast<const uint16_t*>(u);
    EXPECT(q8_bf16_paged_decode(out, q, 512, b, b, u, 8, u, 100, 2, 4, 2, 96, 16, 64, 0.1f, ws, 1u << 30, nullptr) ==
           Q8_ERR_UNSUPPORTED);
    EXPECT(q8_bf16_paged_decode(out, q, 512, b, b, u, 8, u, 100, 2, 4, 2, 128, 16, 64, 0.1f, nullptr, 0, nullptr) ==
           Q8_ERR_WORKSPACE);
    EXPECT(q8_bf16_paged_decode_workspace_bytes(4, 3, 2, 128) == 0);
}

static void writer_and_step_validation() {
    const float* k = static_cast<const float*>(fake(0x2000));
    uint32_t* c = static_cast<uint32_t*>(fake(0x3000));
    const uint32_t* sl = c;
    for (uint32_t hs : {0u, 6u, 260u}) EXPECT(q8_cache_write(k, 1024, k, 1024, c, c, sl, 4, 2, hs, 16, 8, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_cache_write(k, 255, k, 256, c, c, sl, 4, 2, 128, 16, 8, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_cache_write(nullptr, 256, k, 256, c, c, sl, 4, 2, 128, 16, 8, nullptr) == Q8_ERR_NULL);
    EXPECT(q8_cache_write(nullptr, 256, nullptr, 256, nullptr, nullptr, nullptr, 0, 2, 128, 16, 8, nullptr) == Q8_OK);
    EXPECT(q8_cache_write(k, 256, k, 256, c, c, sl, 4, 2, 128, 16, 0, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_cache_write(k, 1024, k, 1024, c, c, sl, 0xFFFFFFFFu, 8, 128, 16, 8, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_f32_cache_write(k, 256, k, 256, reinterpret_cast<float*>(fake(0x3004)), reinterpret_cast<float*>(c), sl, 4,
                              2, 128, 16, 8, nullptr) == Q8_ERR_UNSUPPORTED);
    uint16_t* bc = reinterpret_cast<uint16_t*>(c);
    EXPECT(q8_bf16_cache_write(k, 256, k, 256, bc, bc, sl, 4, 2, 20, 16, 8, nullptr) == Q8_ERR_UNSUPPORTED);
    EXPECT(q8_bf16_cache_write(k, 256, k, 256, reinterpret_cast<uint16_t*>(fake(0x3008)), bc, sl, 4, 2, 128, 16, 8,
                               nullptr) == Q8_ERR_UNSUPPORTED);
    EXPECT(q8_bf16_cache_write(nullptr, 256, k, 256, bc, bc, sl, 4, 2, 128, 16, 8, nullptr) == Q8_ERR_NULL);
    // norm + rotary
    float* o = static_cast<float*>(fake(0x5000));
    const float* w = k;
    EXPECT(q8_norm_rope(o, 512, k, 512, 128, 3, 4, 128, sl, w, w, 12, 100, 1e-6f, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_norm_rope(o, 512, k, 512, 100, 3, 4, 128, sl, w, w, 64, 100, 1e-6f, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_norm_rope(o, 512, k, 512, 128, 3, 4, 128, sl, w, w, 64, 0, 1e-6f, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_norm_rope(o, 512, k, 512, 128, 3, 4, 128, sl, w, w, 64, 100, -1.0f, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_norm_rope(o, 512, k, 512, 128, 3, 4, 128, nullptr, w, w, 64, 100, 1e-6f, nullptr) == Q8_ERR_NULL);
    EXPECT(q8_norm_rope(o, 512, k, 0xFFFFFFFFu, 0xFFFFFFFFu, 3, 0xFFFFFFFFu, 128, sl, w, w, 64, 100, 1e-6f, nullptr) ==
           Q8_ERR_SHAPE);
    EXPECT(q8_rope_table(o, 100, 7, 10000.0f, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_rope_table(o, 100, 8, -1.0f, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_rope_table(nullptr, 100, 8, 10000.0f, nullptr) == Q8_ERR_NULL);
    EXPECT(q8_norm_rope_cache_write(k, 256, k, 256, c, c, sl, sl, w, w, 64, 100, 1e-6f, 4, 2, 128, 16, 0, nullptr) ==
           Q8_ERR_SHAPE);
    EXPECT(q8_norm_rope_qk_cache_write(o, 512, k, 512, 128, 2, 4, sl, w, k, 255, k, 256, c, c, sl, sl, w, w, 64, 100, 1e-6f,
                                       4, 2, 128, 16, 8, nullptr) == Q8_ERR_SHAPE);
    // the decode step with the norm + rotary step
    void* ws = fake(0x4000);
    EXPECT(q8_norm_rope_decode_step(o, k, 512, 0, k, 256, k, 256, c, c, sl, 8, sl, 100, w, w, w, 12, 100, 1e-6f, 2, 4, 2, 128,
                                    16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_norm_rope_decode_step(o, k, 512, 0, k, 256, k, 256, c, c, sl, 8, sl, 100, nullptr, w, w, 64, 100, 1e-6f, 2, 4, 2,
                                    128, 16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_NULL);
    EXPECT(q8_norm_rope_decode_step(o, k, 384, 0, k, 192, k, 192, c, c, sl, 8, sl, 100, w, w, w, 32, 100, 1e-6f, 2, 4, 2, 96,
                                    16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_UNSUPPORTED);
    EXPECT(q8_norm_rope_decode_step(o, k, 512, 100, k, 256, k, 256, c, c, sl, 8, sl, 100, w, w, w, 64, 100, 1e-6f, 2, 4, 2,
                                    128, 16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_norm_rope_decode_step(o, k, 0xFFFFFFFFu, 0x7FFFFFFFu, k, 256, k, 256, c, c, sl, 8, sl, 100, w, w, w, 64, 100,
                                    1e-6f, 2, 4, 2, 128, 16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_norm_rope_decode_step(o, k, 512, 0, k, 256, k, 256, reinterpret_cast<uint32_t*>(fake(0x3004)), c, sl, 8, sl,
                                    100, w, w, w, 64, 100, 1e-6f, 2, 4, 2, 128, 16, 64, 0.1f, ws, 1u << 30,
                                    nullptr) == Q8_ERR_UNSUPPORTED);
    EXPECT(q8_norm_rope_decode_step(o, k, 512, 0, k, 256, k, 256, c, c, sl, 8, sl, 100, w, w, w, 64, 100, 1e-6f, 2, 4, 2, 128,
                                    48, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_UNSUPPORTED);
    EXPECT(q8_norm_rope_decode_step(o, k, 512, 0, k, 256, k, 256, c, c, sl, 8, sl, 100, w, w, w, 64, 100, 1e-6f, 2, 4, 2, 128,
                                    16, 64, 0.1f, ws, 16, nullptr) == Q8_ERR_WORKSPACE);
    // a supported shape reaches the launch (no kernel in this build: a HIP error)
    EXPECT(q8_norm_rope_decode_step(o, k, 512, 0, k, 256, k, 256, c, c, sl, 8, sl, 100, w, w, w, 64, 100, 1e-6f, 2, 4, 2, 128,
                                    16, 64, 0.1f, ws, 1u << 30, nullptr) == Q8_ERR_HIP);
    // block selection
    EXPECT(q8_index_select(k, 100, sl, 4, 0, 8, c, 1000, c, nullptr, 0, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_index_select(k, 100, sl, 4, 64, 15, c, 1000, c, nullptr, 0, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_index_select(k, 100, sl, 4, 64, 8, c, 1000, c, c, 3, nullptr) == Q8_ERR_SHAPE);
    EXPECT(q8_index_select(k, 20000, sl, 4, 64, 8, c, 1000, c, nullptr, 0, nullptr) == Q8_ERR_UNSUPPORTED);
    EXPECT(q8_index_select(k, 0xFFFFFFFFu, sl, 4, 0xFFFFFFFFu, 0xFFFFFFFFu, c, 0xFFFFFFFFu, c, c, 0xFFFFFFFFu,
                           nullptr) == Q8_ERR_SHAPE);
}

int main() {
    workspace_properties();
    decode_validation();
    writer_and_step_validation();
    for (int s = 0; s <= 6; ++s) EXPECT(q8_status_string(static_cast<q8_status>(s)) != nullptr);
    if (failures) {
        fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
