// Decode planning and dispatch: the split plan shared by the workspace query
// and the launch, and the choice of split-kernel instantiation.  The kernel
// itself (and what it computes) is in decode_kernel.h.
#include <stdlib.h>

#include "decode_split.h"

namespace q8kv {

DecodePlan plan_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                       uint32_t head_size, uint32_t block_size, uint32_t max_positions) {
    DecodePlan p{};
    const uint32_t n_rep = num_kv_heads ? num_heads / num_kv_heads : 1;
    p.group = n_rep > 4 ? 8 : 4;
    p.num_groups = (n_rep + p.group - 1) / p.group;
    (void)block_size;
    // Persistent wavefronts: 4 per compute unit of an MI355X (256 CUs),
    // shared evenly by the row groups.
    uint64_t target = kDecodeWaves;
    if (const char* e = getenv("Q8KV_DECODE_WAVES")) {
        const long v = atol(e);
        if (v >= 1 && v <= (1L << 20)) target = static_cast<uint64_t>(v);
    }
    const uint64_t num_rg = static_cast<uint64_t>(num_kv_heads) * p.num_groups;
    uint64_t per = num_rg ? target / num_rg : 1;
    if (per < 1) per = 1;
    p.waves_per_rg = static_cast<uint32_t>(per);
    p.num_waves = num_rg * per;
    p.recs_per_rg = p.waves_per_rg + (num_seqs ? num_seqs - 1 : 0);
    // Workspace: one arrival counter per (row group, sequence), then the
    // partial records.  A sequence of at most one chunk always lies in a
    // single wave's range, so then no workspace is needed at all.
    // A record holds the padded head size (code words per row rounded up to
    // 16, 32, 48 or 64) for every query head of the group.
    const uint32_t hs4 = head_size / 4;
    const uint32_t hs4p = hs4 <= 16 ? 16 : hs4 <= 32 ? 32 : hs4 <= 48 ? 48 : 64;
    const uint64_t slots = num_rg * p.recs_per_rg * p.group;
    p.counters_offset = 0;
    p.acc_offset = (num_rg * num_seqs * sizeof(uint32_t) + 255) / 256 * 256;
    p.ml_offset = p.acc_offset + (slots * 4 * hs4p * sizeof(float) + 255) / 256 * 256;
    p.bytes = max_positions > static_cast<uint32_t>(kChunk) ? p.ml_offset + slots * 2 * sizeof(float) : 0;
    return p;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
    const bool vis = a.visible_pos != nullptr;
    const uint32_t hs4 = a.head_size / 4;
    const uint32_t wpt = hs4 + 1;
    SplitConsts c{};
    c.waves_per_rg = p.waves_per_rg;
    c.num_rg = a.num_kv_heads * p.num_groups;
    c.group = p.group;
    c.num_groups = p.num_groups;
    c.recs_per_rg = p.recs_per_rg;
    c.seg_rows = a.block_size < static_cast<uint32_t>(kChunk) ? a.block_size : kChunk;
    const bool shape_ok = a.block_size % 4 == 0 &&
                          (kChunk % a.block_size == 0 || a.block_size % kChunk == 0);
    const bool align_ok = reinterpret_cast<uintptr_t>(a.key_cache) % 16 == 0 &&
                          reinterpret_cast<uintptr_t>(a.value_cache) % 16 == 0;
    c.tiled_ok = shape_ok && align_ok;
    c.q_vec_ok = reinterpret_cast<uintptr_t>(a.q) % 16 == 0 && a.q_stride % 4 == 0;
    c.seg_u4 = c.seg_rows * wpt / 4;
    if (c.seg_u4 == 0) c.seg_u4 = 1;
    c.seg_magic = static_cast<uint32_t>((0x100000000ull + c.seg_u4 - 1) / c.seg_u4);
    // With no block table or no blocks every sequence attends nothing
    // (positions are capped by the table); the kernel then only writes zeros.
    const uint32_t nbm1 = a.num_blocks ? a.num_blocks - 1 : 0;
    {
        const dim3 grid(static_cast<uint32_t>((p.num_waves + kWavesPerGroup - 1) / kWavesPerGroup));
        hipError_t err;
        const bool t = c.tiled_ok != 0;
        if (hs4 <= 16) err = launch_split_hs16(a, c, nbm1, grid, stream, vis, t, hs4 == 16);
        else if (hs4 <= 32) err = launch_split_hs32(a, c, nbm1, grid, stream, vis, t, hs4 == 32);
        else if (hs4 <= 48) err = launch_split_hs48(a, c, nbm1, grid, stream, vis, t, hs4 == 48);
        else err = launch_split_hs64(a, c, nbm1, grid, stream, vis, t, hs4 == 64);
        if (err != hipSuccess) return err;
    }
    return hipGetLastError();
}

}  // namespace q8kv
