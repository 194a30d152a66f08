// Split-kernel launch interface shared by the decode translation units.
#pragma once
#include "q8kv_internal.h"

namespace q8kv {

// Independent wavefronts packed per workgroup (fewer workgroups to dispatch).
constexpr uint32_t kWavesPerGroup = 4;

struct SplitConsts {
    uint32_t waves_per_rg;  // persistent wavefronts per row group (before capping by the chunk count)
    uint32_t num_rg;        // row groups: num_kv_heads * num_groups
    uint32_t group, num_groups;
    uint32_t recs_per_rg;   // partial records per row group: waves_per_rg + num_seqs - 1
    uint32_t seg_u4;        // 16-byte units per tile segment in a chunk
    uint32_t seg_magic;     // ceil(2^32 / seg_u4): u / seg_u4 == mulhi(u, magic) for u < 2^16
    uint32_t seg_rows;      // rows per segment = min(block_size, 64)
    uint32_t tiled_ok;      // segment copies are legal (alignment, block_size shape)
    uint32_t q_vec_ok;      // q rows of every sequence are 16-byte aligned
};

// One translation unit per padded head size (code words per row rounded up
// to 16, 32, 48 or 64); `exact` when head_size / 4 equals that size.
hipError_t launch_split_hs16(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st,
                             bool vis, bool tiled, bool exact);
hipError_t launch_split_hs32(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st,
                             bool vis, bool tiled, bool exact);
hipError_t launch_split_hs48(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st,
                             bool vis, bool tiled, bool exact);
hipError_t launch_split_hs64(const DecodeArgs& a, const SplitConsts& c, uint32_t nbm1, dim3 grid, hipStream_t st,
                             bool vis, bool tiled, bool exact);

}  // namespace q8kv
