// Decode planning and dispatch: the split plan shared by the workspace query
// and the launch, the choice of split-kernel instantiation, and the number of
// persistent wavefronts the device keeps resident for it.  The kernel itself
// (and what it computes) is in decode_kernel.h.
#include <stdlib.h>

#include <mutex>

#include "decode_split.h"

namespace q8kv {

uint64_t decode_wave_override() {
    // Q8KV_DECODE_WAVES (documented in q8kv.h) forces the persistent wave
    // count; tests use it to move the boundaries between wave ranges.
    if (const char* e = getenv("Q8KV_DECODE_WAVES")) {
        const long v = atol(e);
        if (v >= 1 && v <= (1L << 20)) return static_cast<uint64_t>(v);
    }
    return 0;
}

uint64_t decode_wave_bound() {
    const uint64_t o = decode_wave_override();
    return o ? o : kMaxDecodeWaves;
}

DecodePlan plan_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                       uint32_t head_size, uint32_t block_size, uint32_t max_positions, uint64_t target) {
    DecodePlan p{};
    const uint32_t n_rep = num_kv_heads ? num_heads / num_kv_heads : 1;
    p.group = decode_group(n_rep);
    p.num_groups = (n_rep + p.group - 1) / p.group;
    (void)block_size;
    // The persistent wavefronts are shared evenly by the row groups.
    const uint64_t num_rg = static_cast<uint64_t>(num_kv_heads) * p.num_groups;
    uint64_t per = num_rg ? target / num_rg : 1;
    if (per < 1) per = 1;
    p.waves_per_rg = static_cast<uint32_t>(per);
    p.num_waves = num_rg * per;
    p.recs_per_rg = static_cast<uint64_t>(p.waves_per_rg) + (num_seqs ? num_seqs - 1 : 0);
    // Workspace: one arrival counter per (row group, sequence), then the
    // partial records.  A sequence of at most one chunk always lies in a
    // single wave's range, so then no workspace is needed at all.
    // A record holds the padded head size (code words per row rounded up to
    // 16, 32, 48 or 64) for every query head of the group.  The need grows
    // with the wave count, so a workspace sized for the bound serves every
    // launch below it.
    const uint32_t hs4 = head_size / 4;
    const uint32_t hs4p = hs4 <= 16 ? 16 : hs4 <= 32 ? 32 : hs4 <= 48 ? 48 : 64;
    const uint64_t slots = num_rg * p.recs_per_rg * p.group;
    p.counters_offset = 0;
    p.acc_offset = (num_rg * num_seqs * sizeof(uint32_t) + 255) / 256 * 256;
    p.ml_offset = p.acc_offset + (slots * 4 * hs4p * sizeof(float) + 255) / 256 * 256;
    // (a chunk holds 32 or 64 positions: the smaller bounds when one suffices)
    p.bytes = max_positions > 32u ? p.ml_offset + slots * 2 * sizeof(float) : 0;
    return p;
}

namespace {

// Workgroups of one kernel resident per compute unit (LDS, registers and
// its waves-per-EU bound decide it), and the device's compute units; both
// cached per (kernel, device).
struct Residency {
    const void* fn;
    int device;
    uint32_t waves;     // resident wavefronts on the whole device
    uint32_t per_cu;    // resident workgroups per compute unit
};
std::mutex g_res_mu;
Residency g_res[64];
int g_res_n = 0;

hipError_t resident_waves(const void* fn, uint32_t* waves, uint32_t* per_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_res_mu);
    for (int i = 0; i < g_res_n; ++i)
        if (g_res[i].fn == fn && g_res[i].device == dev) {
            *waves = g_res[i].waves;
            *per_cu = g_res[i].per_cu;
            return hipSuccess;
        }
    int blocks = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kWave * kWavesPerGroup, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (blocks < 1) blocks = 1;
    if (cus < 1) cus = 1;
    const uint64_t w = static_cast<uint64_t>(blocks) * kWavesPerGroup * static_cast<uint64_t>(cus);
    *waves = static_cast<uint32_t>(w < kMaxDecodeWaves ? w : kMaxDecodeWaves);
    *per_cu = static_cast<uint32_t>(blocks);
    if (g_res_n < 64) g_res[g_res_n++] = Residency{fn, dev, *waves, *per_cu};
    return hipSuccess;
}

// Chunks of `ch` positions can be copied as tile runs: block_size nests with
// the chunk and both caches are 16-byte aligned.
bool tiles_ok(const DecodeArgs& a, uint32_t ch) {
    const bool shape_ok = a.block_size % 4 == 0 && (ch % a.block_size == 0 || a.block_size % ch == 0);
    const bool align_ok = reinterpret_cast<uintptr_t>(a.key_cache) % 16 == 0 &&
                          reinterpret_cast<uintptr_t>(a.value_cache) % 16 == 0;
    return shape_ok && align_ok;
}

}  // namespace

bool norm_rope_decode_supported(uint32_t head_size, uint32_t num_heads, uint32_t num_kv_heads, uint32_t block_size,
                                const uint32_t* key_cache, const uint32_t* value_cache) {
    if ((head_size != 64 && head_size != 128 && head_size != 256) || num_kv_heads == 0) return false;
    const uint32_t group = decode_group(num_heads / num_kv_heads);
    if (head_size == 256 && group == 16) return false;    // no instantiation (register pressure)
    DecodeArgs a{};
    a.block_size = block_size;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    return tiles_ok(a, static_cast<uint32_t>(decode_chunk(static_cast<int>(head_size / 4), static_cast<int>(group / 4))));
}

hipError_t launch_decode(const DecodeArgs& a, uint32_t max_positions, hipStream_t stream) {
    const bool vis = a.visible_pos != nullptr;
    const uint32_t hs4 = a.head_size / 4;
    const uint32_t wpt = hs4 + 1;
    // Query heads per kv head: (row, head) pairs in multi-row decode.
    const uint32_t num_pairs = a.num_heads * (a.rows_per_seq > 1 ? a.rows_per_seq : 1u);
    const uint32_t group = decode_group(num_pairs / a.num_kv_heads);
    const uint32_t hs4p = hs4 <= 16 ? 16 : hs4 <= 32 ? 32 : hs4 <= 48 ? 48 : 64;
    const uint32_t ch = static_cast<uint32_t>(decode_chunk(static_cast<int>(hs4p), static_cast<int>(group / 4)));
    SplitConsts c{};
    c.seg_rows = a.block_size < ch ? a.block_size : ch;
    c.tiled_ok = tiles_ok(a, ch);
    c.q_vec_ok = reinterpret_cast<uintptr_t>(a.q) % 16 == 0 && a.q_stride % 4 == 0 && a.q_head_stride % 4 == 0;
    c.seg_u4 = c.seg_rows * wpt / 4;
    if (c.seg_u4 == 0) c.seg_u4 = 1;
    c.seg_magic = static_cast<uint32_t>((0x100000000ull + c.seg_u4 - 1) / c.seg_u4);
    const bool t = c.tiled_ok != 0;
    // Segment layouts need whole tiles per segment: blocks no longer than a chunk.
    const uint32_t seg_whole = a.block_size <= ch ? c.seg_rows : 0u;
    const void* fn;
    if (hs4 <= 16) fn = split_kernel_hs16(vis, t, hs4 == 16, group, seg_whole);
    else if (hs4 <= 32) fn = split_kernel_hs32(vis, t, hs4 == 32, group, seg_whole);
    else if (hs4 <= 48) fn = split_kernel_hs48(vis, t, hs4 == 48, group, seg_whole);
    else fn = split_kernel_hs64(vis, t, hs4 == 64, group, seg_whole);
    if (a.nr_q_weight) {
        // the norm + rotary step exists for the shapes norm_rope_decode_supported accepts
        fn = nullptr;
        if (!vis && t && a.rows_per_seq <= 1) {
            if (hs4 == 16) fn = split_kernel_nr_hs16(group, seg_whole);
            else if (hs4 == 32) fn = split_kernel_nr_hs32(group, seg_whole);
            else if (hs4 == 64) fn = split_kernel_nr_hs64(group, seg_whole);
        }
        if (!fn) return hipErrorInvalidValue;
    }
    // As many persistent wavefronts as the device keeps resident for this
    // kernel, at most the bound the workspace was sized for.
    uint64_t target = decode_wave_override();
    uint32_t per_cu = 1;
    if (!target) {
        uint32_t w = 0;
        const hipError_t e = resident_waves(fn, &w, &per_cu);
        if (e != hipSuccess) return e;
        target = w;
    }
    const DecodePlan p = plan_decode(a.num_seqs, num_pairs, a.num_kv_heads, a.head_size, a.block_size,
                                     max_positions, target);
    c.waves_per_rg = p.waves_per_rg;
    c.num_rg = a.num_kv_heads * p.num_groups;
    c.group = p.group;
    c.num_groups = p.num_groups;
    c.recs_per_rg = static_cast<uint32_t>(p.recs_per_rg);     // the call's shapes were checked to fit
    // Two resident workgroups per CU with the whole grid resident: the second
    // half of the grid is each CU's second workgroup (smaller shares).
    c.young_from = per_cu == 2 && !decode_wave_override() ? p.waves_per_rg / 2 : p.waves_per_rg;
    // XCD-aware numbering (a permutation of the workgroups within each half
    // of the grid, so that the second-workgroup waves stay the second half),
    // for two resident workgroups per CU.  Measured: Llama-shaped step
    // 63.75 -> 63.46 us; with one workgroup per CU it gave no gain (the
    // 32K-token decode was once 4% slower), so those launches keep the plain
    // numbering.
    const uint64_t groups = (p.num_waves + kWavesPerGroup - 1) / kWavesPerGroup;
    c.xcd_span = 0;
    if (!decode_wave_override() && per_cu == 2 && groups % (2 * kXcds) == 0)
        c.xcd_span = static_cast<uint32_t>(groups / 2);
    DecodeArgs ka = a;
    if (p.bytes) {
        char* ws = static_cast<char*>(a.workspace);
        ka.counters = reinterpret_cast<uint32_t*>(ws + p.counters_offset);
        ka.part_acc = reinterpret_cast<float*>(ws + p.acc_offset);
        ka.part_ml = reinterpret_cast<float*>(ws + p.ml_offset);
    }
    // With no block table or no blocks every sequence attends nothing
    // (positions are capped by the table); the kernel then only writes zeros.
    uint32_t nbm1 = a.num_blocks ? a.num_blocks - 1 : 0;
    void* args[] = {&ka, &c, &nbm1};
    const dim3 grid(static_cast<uint32_t>((p.num_waves + kWavesPerGroup - 1) / kWavesPerGroup));
    const hipError_t e = hipLaunchKernel(fn, grid, dim3(kWave * kWavesPerGroup), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace q8kv
