// Internal declarations shared by the HIP translation units of libq8kv.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q8kv {

constexpr uint32_t kPadSlot = 0xFFFFFFFFu;
constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kChunk = 64;         // decode positions per chunk
constexpr uint32_t kMaxSplit = 1024;   // longest context split (positions) of one work item

struct CacheWriteArgs {
    const float* key;
    const float* value;
    uint32_t* key_cache;
    uint32_t* value_cache;
    const uint32_t* slot_mapping;
    uint32_t key_stride, value_stride;
    uint32_t num_tokens, num_kv_heads, head_size, block_size, num_blocks;
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);

// Split plan shared by the workspace query and the decode call.
struct DecodePlan {
    uint32_t split_tokens;   // positions per split, a multiple of kChunk
    uint32_t num_splits;     // splits of the longest possible position list
    uint32_t group;          // query heads handled together per kv head (4 or 8)
    uint32_t num_groups;     // ceil(n_rep / group)
    size_t ml_offset, acc_offset, bytes;
};

DecodePlan plan_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                       uint32_t head_size, uint32_t block_size, uint32_t max_positions);

struct DecodeArgs {
    float* out;
    const float* q;
    const uint32_t* key_cache;
    const uint32_t* value_cache;
    const uint32_t* block_tables;
    const uint32_t* context_lens;
    const uint32_t* visible_pos;
    const uint32_t* num_visible;
    float* part_ml;          // [S, H, num_splits, 2]: running max (log2 units), sum
    float* part_acc;         // [S, H, num_splits, head_size]: unnormalized output
    uint32_t q_stride, max_num_blocks_per_seq, max_context_len, vis_stride;
    uint32_t num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks;
    float scale_log2;        // softmax scale * log2(e)
};

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream);

}  // namespace q8kv
