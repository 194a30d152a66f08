// Split-kernel launch interface shared by the decode translation units.
#pragma once
#include "q8kv_internal.h"

namespace q8kv {

// Independent wavefronts packed per workgroup (fewer workgroups to dispatch).
constexpr uint32_t kWavesPerGroup = 4;

// Positions per chunk of a split-kernel instantiation: 32 for up to 32 code
// words per row with one set of 4 query heads (two chunks in flight per
// wave fit in a quarter of the CU's LDS, so two workgroups share a CU), else
// 64.  hs4p: code words per row rounded up to 16, 32, 48 or 64; nhs: sets of
// 4 query heads per wavefront.
constexpr int decode_chunk(int hs4p, int nhs) { return hs4p <= 32 && nhs == 1 ? 32 : 64; }

// Query heads (or, in multi-row decode, (row, head) pairs) of one kv head
// handled together by a wavefront, so that each K/V byte is read once for
// them: 4, 8 or 16 (n_rep above 16 takes several groups of 16).
constexpr uint32_t decode_group(uint32_t n_rep) { return n_rep > 8 ? 16u : n_rep > 4 ? 8u : 4u; }

struct SplitConsts {
    uint32_t waves_per_rg;  // persistent wavefronts per row group (before capping by the chunk count)
    uint32_t num_rg;        // row groups: num_kv_heads * num_groups
    uint32_t group, num_groups;
    uint32_t recs_per_rg;   // partial records per row group: waves_per_rg + num_seqs - 1
    uint32_t seg_u4;        // 16-byte units per tile segment in a chunk
    uint32_t seg_magic;     // ceil(2^32 / seg_u4): u / seg_u4 == mulhi(u, magic) for u < 2^16
    uint32_t seg_rows;      // rows per segment = min(block_size, chunk positions)
    uint32_t tiled_ok;      // segment copies are legal (alignment, block_size shape)
    uint32_t q_vec_ok;      // q rows of every sequence are 16-byte aligned
    uint32_t young_from;    // first wave (of a row group) in the grid's second workgroup per CU; >= waves: none
    uint32_t xcd_span;      // XCD-aware workgroup numbering over spans of this many workgroups; 0: none
};

// The split-kernel instantiation for these arguments: one translation unit
// per padded head size (code words per row rounded up to 16, 32, 48 or 64);
// `exact` when head_size / 4 equals that size; seg_rows: the block size when
// a block is a whole tile segment of a chunk (at most the chunk's positions),
// else 0.  Launched with (DecodeArgs, SplitConsts, uint32_t num_blocks_m1).
const void* split_kernel_hs16(bool vis, bool tiled, bool exact, uint32_t group, uint32_t seg_rows);
const void* split_kernel_hs32(bool vis, bool tiled, bool exact, uint32_t group, uint32_t seg_rows);
const void* split_kernel_hs48(bool vis, bool tiled, bool exact, uint32_t group, uint32_t seg_rows);
const void* split_kernel_hs64(bool vis, bool tiled, bool exact, uint32_t group, uint32_t seg_rows);
// The norm + rotary decode step's instantiation (head_size 64, 128 or 256:
// 16, 32 or 64 code words per row; dense positions, tiled chunks) for
// query-head groups of 4, 8 or 16 (not 16 at head_size 256: null).
const void* split_kernel_nr_hs16(uint32_t group, uint32_t seg_rows);
const void* split_kernel_nr_hs32(uint32_t group, uint32_t seg_rows);
const void* split_kernel_nr_hs64(uint32_t group, uint32_t seg_rows);

}  // namespace q8kv
