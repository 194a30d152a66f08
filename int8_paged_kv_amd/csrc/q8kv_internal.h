// Internal declarations shared by the HIP translation units of libq8kv.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q8kv {

constexpr uint32_t kPadSlot = 0xFFFFFFFFu;
constexpr int kWave = 64;          // CDNA wavefront width
// Bound on the persistent decode wavefronts (8 per CU of a 256-CU MI355X);
// a launch takes as many as the device keeps resident for its kernel, up to
// this bound, which also sizes the workspace.
constexpr uint32_t kMaxDecodeWaves = 2048;
constexpr uint32_t kXcds = 8;       // MI355X: accelerator complex dies, each with its own L2
// Cache writers: from this many (token, kv head) pairs on, each wave takes
// kWritePairsPerWave consecutive pairs with all their loads in flight.
constexpr uint64_t kWriteBatchMinPairs = 32768;
constexpr int kWritePairsPerWave = 4;
// Largest one-dimensional grid (workgroups) a launch may ask for.
constexpr uint64_t kMaxGridBlocks = 0x7FFFFFFFull;
// Workgroups of a q8_cache_write launch: one per four (token, kv head) pairs
// in small writes, one per 16 tokens of a kv head in batched ones.
inline uint64_t cache_write_blocks(uint32_t num_tokens, uint32_t num_kv_heads) {
    const uint64_t pairs = static_cast<uint64_t>(num_tokens) * num_kv_heads;
    if (pairs >= kWriteBatchMinPairs) return (static_cast<uint64_t>(num_tokens) + 15) / 16 * num_kv_heads;
    return (pairs + 3) / 4;
}

struct CacheWriteArgs {
    const float* key;
    const float* value;
    uint32_t* key_cache;
    uint32_t* value_cache;
    const uint32_t* slot_mapping;
    uint32_t key_stride, value_stride;
    uint32_t num_tokens, num_kv_heads, head_size, block_size, num_blocks;
    uint32_t* bounds_flags;  // Q8_DEBUG_BOUNDS builds: device flag word of failed content checks
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);

// ---- per-head RMSNorm + partial rotary embedding (q rows; fused into the K write) ----

struct NormRopeArgs {
    float* out;                  // [num_rows, num_heads, head_size] rows of out_stride floats
    const float* x;              // head h of row t at x[t*x_stride + h*head_stride]
    const uint32_t* positions;   // [num_rows]
    const float* weight;         // [head_size] norm weight
    const float* table;          // [num_positions, rot] rotary cos | sin
    uint32_t x_stride, head_stride, out_stride;
    uint32_t num_rows, num_heads, head_size, rot, num_positions;
    float eps;
    bool params_vec4;            // weight and table 16-byte aligned (rot % 8 == 0 keeps table rows so)
};

struct NormRopeCacheWriteArgs {
    const float* key;
    const float* value;
    uint32_t* key_cache;
    uint32_t* value_cache;
    const uint32_t* slot_mapping;
    const uint32_t* positions;   // [num_tokens]; may be read for pad tokens, never used for them
    const float* weight;         // [head_size] K norm weight
    const float* table;          // [num_positions, rot]
    uint32_t key_stride, value_stride;
    uint32_t num_tokens, num_kv_heads, head_size, block_size, num_blocks, rot, num_positions;
    float eps;
    bool params_vec4;            // weight and table 16-byte aligned
};

// ---- block selection into a visible list ----

constexpr uint32_t kSelectMaxBlocks = 16384;   // scores per row held in LDS

struct IndexSelectArgs {
    const float* scores;         // row r's block j at scores[r*score_stride + j]
    const uint32_t* row_lens;    // [num_rows] t_len
    uint32_t* visible_pos;       // row r's list at visible_pos[r*vis_stride]
    uint32_t* num_visible;       // [num_rows]
    uint32_t* visible_mask;      // row r's block bits at visible_mask[r*mask_stride], or null
    uint32_t score_stride, num_rows, ratio, k, vis_stride, mask_stride;
};

hipError_t launch_index_select(const IndexSelectArgs& a, hipStream_t stream);

hipError_t launch_rope_table(float* table, uint32_t num_positions, uint32_t rot, double theta, hipStream_t stream);
hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t stream);
hipError_t launch_norm_rope_cache_write(const NormRopeCacheWriteArgs& a, hipStream_t stream);
// q rows and the K/V write in one launch (two for a bulk write)
hipError_t launch_norm_rope_qk_cache_write(const NormRopeArgs& q, const NormRopeCacheWriteArgs& k, hipStream_t stream);

// Decode plan shared by the workspace query and the decode call.  For each
// row group (kv head, group of query heads sharing it) waves_per_rg
// persistent wavefronts split the batch's chunks (32 or 64 positions) by
// cost; a sequence covered by more than one wavefront leaves one partial
// record per wavefront.
struct DecodePlan {
    uint32_t group;          // query heads handled together per kv head (4, 8 or 16)
    uint32_t num_groups;     // ceil(n_rep / group)
    uint32_t waves_per_rg;   // persistent wavefronts per row group
    uint64_t recs_per_rg;    // partial record slots per row group: waves_per_rg + num_seqs - 1 (64-bit: no wrap)
    uint64_t num_waves;      // grid: row groups * waves_per_rg
    size_t counters_offset, ml_offset, acc_offset, bytes;
};

// target: persistent wavefronts to spread over the row groups.
DecodePlan plan_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                       uint32_t head_size, uint32_t block_size, uint32_t max_positions, uint64_t target);
// The wave count a workspace must be sized for (kMaxDecodeWaves, or the
// Q8KV_DECODE_WAVES override), and the override alone (0 when unset).
uint64_t decode_wave_bound();
uint64_t decode_wave_override();

struct DecodeArgs {
    float* out;
    const float* q;
    const uint32_t* key_cache;
    const uint32_t* value_cache;
    const uint32_t* block_tables;
    const uint32_t* context_lens;
    const uint32_t* visible_pos;
    const uint32_t* num_visible;
    void* workspace;         // caller workspace, sized for decode_wave_bound() waves (null when none is needed)
    // Set at launch from the plan, inside the workspace:
    uint32_t* counters;      // [row group, seq]: arrivals of a sequence's waves; zero between calls
    float* part_ml;          // [row group, record, head in group, 2]: running max (log2 units), sum
    float* part_acc;         // [row group, record, head in group, head_size]: unnormalized output
    uint32_t q_stride, max_num_blocks_per_seq, max_context_len, vis_stride;
    uint32_t q_head_stride;  // head h of a q row at h * q_head_stride (head_size unless the caller interleaves heads)
    uint32_t num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks;
    float scale_log2;        // softmax scale * log2(e)
    // Decode step (new_key non-null): sequence s's new K and V vectors
    // (element d of kv head h at new_key[s*new_key_stride + h*head_size + d]),
    // appended to the caches at position context_lens[s]-1 before it is attended.
    const float* new_key;
    const float* new_value;
    uint32_t new_key_stride, new_value_stride;
    uint32_t new_vec4;       // the new rows are 16-byte aligned with strides that keep them so
    uint32_t* key_cache_w;   // key_cache / value_cache, written by the append
    uint32_t* value_cache_w;
    // Decode step with the per-head RMSNorm + partial rotary step (nr_q_weight
    // non-null): sequence s's q rows and new K row are normalized and rotated
    // at position context_lens[s] - 1 before use (norm_rope_ops.h).
    const float* nr_q_weight;    // [head_size]
    const float* nr_k_weight;    // [head_size]
    const float* nr_table;       // [nr_num_positions, nr_rot]: cos | sin per position
    uint32_t nr_rot, nr_num_positions;
    float nr_eps;
    uint32_t nr_params_vec4;     // weights and table 16-byte aligned
    // Multi-row decode (> 1): num_seqs counts rows; row v is row v % rows_per_seq
    // of sequence v / rows_per_seq (its block-table row), and attends the first
    // context_lens[seq] - rows_per_seq + (v % rows_per_seq) + 1 positions.
    uint32_t rows_per_seq;
    uint32_t* bounds_flags;  // Q8_DEBUG_BOUNDS builds: device flag word of failed content checks
};

// max_positions: max_context_len in dense mode, vis_stride with visible lists.
hipError_t launch_decode(const DecodeArgs& a, uint32_t max_positions, hipStream_t stream);
// Whether the decode step with the norm + rotary step (dense, one row per
// sequence) has a kernel for these shapes: head_size 64, 128 or 256 (at 256,
// at most 8 query heads per kv head), caches 16-byte aligned and block_size
// nesting with the chunk.
bool norm_rope_decode_supported(uint32_t head_size, uint32_t num_heads, uint32_t num_kv_heads, uint32_t block_size,
                                const uint32_t* key_cache, const uint32_t* value_cache);

// ---- full-width paged-cache baselines: cache [num_blocks, num_kv_heads, block_size, head_size] ----
// of f32 elements (elem_bytes 4) or bfloat16 ones (elem_bytes 2).

constexpr uint32_t kBaselineDecodeWaves = 2048;   // persistent waves: 8 per CU (2 workgroups of 4)

struct BaselineWriteArgs {
    const float* key;
    const float* value;
    void* key_cache;
    void* value_cache;
    const uint32_t* slot_mapping;
    uint32_t key_stride, value_stride;
    uint32_t num_tokens, num_kv_heads, head_size, block_size, num_blocks;
    uint32_t elem_bytes;     // 4: f32 copies; 2: bfloat16, rounded to nearest, ties to even
};

hipError_t launch_baseline_write(const BaselineWriteArgs& a, hipStream_t stream);

// Row groups are (kv head, group of `group` query heads); each has
// waves_per_rg persistent waves over its chunk list and recs_per_rg partial
// record slots.
struct BaselineDecodePlan {
    uint32_t group, num_groups, waves_per_rg;
    uint64_t recs_per_rg;    // 64-bit: no wrap for extreme sequence counts
    uint64_t num_waves;
    size_t counters_offset, ml_offset, acc_offset, bytes;
};

BaselineDecodePlan plan_baseline_decode(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                                        uint32_t head_size);

struct BaselineDecodeArgs {
    float* out;
    const float* q;
    const void* key_cache;   // elem_bytes-wide elements
    const void* value_cache;
    const uint32_t* block_tables;
    const uint32_t* context_lens;
    uint32_t* counters;      // [row group, seq]: arrivals of a sequence's waves; zero between calls
    float* part_ml;          // [row group, record, head in group, 2]: running max (log2 units), sum
    float* part_acc;         // [row group, record, head in group, head_size]: unnormalized output
    uint32_t q_stride, max_num_blocks_per_seq, max_context_len;
    uint32_t num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks;
    uint32_t group, num_groups, waves_per_rg, recs_per_rg;
    uint32_t elem_bytes;     // 4 (f32) or 2 (bfloat16)
    float inv_block_size;    // 1 / block_size in binary32
    float scale_log2;        // softmax scale * log2(e)
};

hipError_t launch_baseline_decode(const BaselineDecodeArgs& a, const BaselineDecodePlan& p, hipStream_t stream);

}  // namespace q8kv
