// C ABI of libq8kv.so: argument validation, split planning, kernel launches.
// Declarations and the contract of every entry point are in include/q8kv.h.
#include "q8kv.h"
#include "q8kv_internal.h"

#include <cmath>
#include <mutex>

namespace {

thread_local int g_last_hip_error = 0;

q8_status hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int>(e);
    return Q8_ERR_HIP;
}

}  // namespace

// ---- content checks of the Q8_DEBUG_BOUNDS build ----
// One device word per GPU collects the bits of failed checks (bounds.h);
// kernels receive its address, looked up once per device.
static __device__ __align__(4) uint32_t bounds_word;

namespace {

constexpr int kMaxBoundsDevices = 64;
std::mutex g_bounds_mu;
uint32_t* g_bounds_ptr[kMaxBoundsDevices];

// Address of the current device's flag word (debug builds), else null.
uint32_t* bounds_flags_ptr() {
#ifdef Q8_DEBUG_BOUNDS
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxBoundsDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_bounds_mu);
    if (!g_bounds_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(bounds_word)) != hipSuccess) return nullptr;
        g_bounds_ptr[dev] = static_cast<uint32_t*>(p);
    }
    return g_bounds_ptr[dev];
#else
    return nullptr;
#endif
}

bool head_size_ok(uint32_t hs) { return hs != 0 && hs % 4 == 0 && hs <= Q8_MAX_HEAD_SIZE; }
// Shape rules of the norm + rotary step.
bool rope_shape_ok(uint32_t head_size, uint32_t rot, uint32_t num_positions, float eps) {
    return head_size_ok(head_size) && rot % 8 == 0 && rot <= head_size && eps >= 0.0f && std::isfinite(eps) &&
           (rot == 0 || num_positions > 0);
}

}  // namespace

extern "C" {

q8_status q8_cache_write(const float* key, uint32_t key_stride,
                         const float* value, uint32_t value_stride,
                         uint32_t* key_cache, uint32_t* value_cache,
                         const uint32_t* slot_mapping, uint32_t num_tokens,
                         uint32_t num_kv_heads, uint32_t head_size,
                         uint32_t block_size, uint32_t num_blocks, void* stream) {
    if (!head_size_ok(head_size) || block_size == 0 || num_kv_heads == 0) return Q8_ERR_SHAPE;
    const uint64_t row = static_cast<uint64_t>(num_kv_heads) * head_size;
    if (key_stride < row || value_stride < row) return Q8_ERR_SHAPE;
    if (num_tokens == 0) return Q8_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping) return Q8_ERR_NULL;
    if (num_blocks == 0) return Q8_ERR_SHAPE;
    if (q8kv::cache_write_blocks(num_tokens, num_kv_heads) > q8kv::kMaxGridBlocks) return Q8_ERR_SHAPE;
    q8kv::CacheWriteArgs a{};
    a.key = key;
    a.value = value;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.slot_mapping = slot_mapping;
    a.key_stride = key_stride;
    a.value_stride = value_stride;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.head_size = head_size;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.bounds_flags = bounds_flags_ptr();
    const hipError_t e = q8kv::launch_cache_write(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

size_t q8_paged_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_heads,
                                       uint32_t num_kv_heads, uint32_t head_size,
                                       uint32_t block_size, uint32_t max_positions) {
    if (num_kv_heads == 0 || num_heads % num_kv_heads != 0) return 0;
    return q8kv::plan_decode(num_seqs, num_heads, num_kv_heads, head_size, block_size,
                             max_positions, q8kv::decode_wave_bound()).bytes;
}

}  // extern "C"

// ---- scratch of the decode entry point that allocates nothing ----
// A fixed device array holds that entry point's partial records and arrival
// counters.  Each GPU the library runs on has its own copy at its own
// address, found once per device with hipGetSymbolAddress; host code uses
// only that address, never the array's name.  All calls on one GPU share it.
namespace {
constexpr size_t kScratchBytes = Q8_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

__global__ void zero_scratch_kernel(uint4* p, size_t n) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];   // device address of `scratch`, per device, once set up

// The scratch address on the current device.  The first call on a device
// looks the address up and clears the whole array (the arrival counters must
// start at zero; every completed decode leaves them at zero again) with a
// fill kernel on the caller's stream, ordered before the caller's decode.
q8_status scratch_of_current_device(void** out, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return Q8_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
        hipLaunchKernelGGL(zero_scratch_kernel, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(ptr),
                           kScratchBytes / sizeof(uint4));
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return Q8_OK;
}

}  // namespace

namespace {

struct AppendArgs {
    const float* key;
    const float* value;
    uint32_t key_stride, value_stride;
    uint32_t* key_cache;
    uint32_t* value_cache;
};

// The norm + rotary step's parameters of a decode step that applies it.
struct NormRopeStepArgs {
    const float* q_weight;
    const float* k_weight;
    const float* table;
    uint32_t rot, num_positions;
    float eps;
};

q8_status decode_common(float* out, const float* q, uint32_t q_stride,
                        const uint32_t* key_cache, const uint32_t* value_cache,
                        const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                        const uint32_t* context_lens, uint32_t max_context_len,
                        const uint32_t* visible_pos, const uint32_t* num_visible,
                        uint32_t vis_stride,
                        uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                        uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                        float scale, void* workspace, size_t workspace_bytes,
                        void* stream, const AppendArgs* app, uint32_t rows_per_seq,
                        bool static_scratch = false, const NormRopeStepArgs* nr = nullptr,
                        uint32_t q_head_stride = 0) {
    if (!head_size_ok(head_size) || block_size == 0 || num_heads == 0 || num_kv_heads == 0 ||
        num_heads % num_kv_heads != 0)
        return Q8_ERR_SHAPE;
    // head h of a q row at h * q_head_stride (0: packed heads, head_size apart)
    if (q_head_stride == 0) q_head_stride = head_size;
    if (q_head_stride < head_size) return Q8_ERR_SHAPE;
    if (static_cast<uint64_t>(q_stride) < static_cast<uint64_t>(num_heads - 1) * q_head_stride + head_size)
        return Q8_ERR_SHAPE;
    const bool vis = visible_pos != nullptr;
    if (vis && vis_stride == 0) return Q8_ERR_SHAPE;
    if (app) {
        const uint64_t row = static_cast<uint64_t>(num_kv_heads) * head_size;
        if (app->key_stride < row || app->value_stride < row) return Q8_ERR_SHAPE;
    }
    if (rows_per_seq == 0 || (rows_per_seq > 1 && vis)) return Q8_ERR_SHAPE;
    if (static_cast<uint64_t>(num_seqs) * rows_per_seq > 0xFFFFFFFFull) return Q8_ERR_UNSUPPORTED;
    // Multi-row decode: a sequence's rows are query heads of its kv heads' groups
    // (num_heads * rows_per_seq (row, head) pairs), so they share the K/V reads.
    const uint64_t num_pairs = static_cast<uint64_t>(num_heads) * rows_per_seq;
    if (num_pairs > 0xFFFFFFFFull) return Q8_ERR_UNSUPPORTED;
    if (num_seqs == 0) return Q8_OK;
    if (!out || !q || !key_cache || !value_cache || !block_tables) return Q8_ERR_NULL;
    if (vis ? !num_visible : !context_lens) return Q8_ERR_NULL;
    if (app && (!app->key || !app->value)) return Q8_ERR_NULL;
    if (nr && !q8kv::norm_rope_decode_supported(head_size, num_heads, num_kv_heads, block_size, key_cache, value_cache))
        return Q8_ERR_UNSUPPORTED;
    const uint32_t max_pos = vis ? vis_stride : max_context_len;
    if (max_pos > 0 && (max_num_blocks_per_seq == 0 || num_blocks == 0)) return Q8_ERR_SHAPE;
    if (!std::isfinite(scale)) return Q8_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return Q8_ERR_UNSUPPORTED;   // rows are written as 16-byte stores
    // Grid limits: one wavefront per workgroup in 1-D grids.
    // Workspace need at the wave bound; a launch uses at most that many waves.
    const q8kv::DecodePlan p = q8kv::plan_decode(num_seqs, static_cast<uint32_t>(num_pairs), num_kv_heads, head_size,
                                                 block_size, max_pos, q8kv::decode_wave_bound());
    if (p.num_waves > 0x7FFFFFFFull || static_cast<uint64_t>(num_seqs) * num_pairs > 0x7FFFFFFFull ||
        p.recs_per_rg > 0x7FFFFFFFull)
        return Q8_ERR_UNSUPPORTED;
    if (p.bytes > 0 && static_scratch) {
        // The library's own scratch array instead of a caller workspace.
        if (p.bytes > kScratchBytes) return Q8_ERR_WORKSPACE;
        const q8_status st = scratch_of_current_device(&workspace, static_cast<hipStream_t>(stream));
        if (st != Q8_OK) return st;
        workspace_bytes = kScratchBytes;
    }
    if (p.bytes > 0) {
        if (!workspace || workspace_bytes < p.bytes) return Q8_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return Q8_ERR_WORKSPACE;
    }
    q8kv::DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.visible_pos = visible_pos;
    a.num_visible = num_visible;
    a.workspace = p.bytes ? workspace : nullptr;
    a.q_stride = q_stride;
    a.q_head_stride = q_head_stride;
    a.max_num_blocks_per_seq = max_num_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.vis_stride = vis_stride;
    a.num_seqs = num_seqs;
    a.rows_per_seq = rows_per_seq;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_size = head_size;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.bounds_flags = bounds_flags_ptr();
    if (app) {
        a.new_key = app->key;
        a.new_value = app->value;
        a.new_key_stride = app->key_stride;
        a.new_value_stride = app->value_stride;
        a.new_vec4 = reinterpret_cast<uintptr_t>(app->key) % 16 == 0 && reinterpret_cast<uintptr_t>(app->value) % 16 == 0 &&
                     app->key_stride % 4 == 0 && app->value_stride % 4 == 0 && head_size % 4 == 0;
        a.key_cache_w = app->key_cache;
        a.value_cache_w = app->value_cache;
    }
    if (nr) {
        a.nr_q_weight = nr->q_weight;
        a.nr_k_weight = nr->k_weight;
        a.nr_table = nr->table;
        a.nr_rot = nr->rot;
        a.nr_num_positions = nr->num_positions;
        a.nr_eps = nr->eps;
        a.nr_params_vec4 = reinterpret_cast<uintptr_t>(nr->q_weight) % 16 == 0 &&
                           reinterpret_cast<uintptr_t>(nr->k_weight) % 16 == 0 &&
                           reinterpret_cast<uintptr_t>(nr->table) % 16 == 0;
    }
    const hipError_t e = q8kv::launch_decode(a, max_pos, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

}  // namespace

extern "C" {

q8_status q8_paged_decode(float* out, const float* q, uint32_t q_stride,
                          const uint32_t* key_cache, const uint32_t* value_cache,
                          const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                          const uint32_t* context_lens, uint32_t max_context_len,
                          const uint32_t* visible_pos, const uint32_t* num_visible,
                          uint32_t vis_stride,
                          uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                          uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                          float scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return decode_common(out, q, q_stride, key_cache, value_cache, block_tables, max_num_blocks_per_seq,
                         context_lens, max_context_len, visible_pos, num_visible, vis_stride, num_seqs,
                         num_heads, num_kv_heads, head_size, block_size, num_blocks, scale, workspace,
                         workspace_bytes, stream, nullptr, 1);
}

q8_status q8_paged_decode_noalloc(float* out, const float* q, uint32_t q_stride,
                                  const uint32_t* key_cache, const uint32_t* value_cache,
                                  const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                                  const uint32_t* context_lens, uint32_t max_context_len,
                                  const uint32_t* visible_pos, const uint32_t* num_visible,
                                  uint32_t vis_stride,
                                  uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                                  uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                                  float scale, void* stream) {
    return decode_common(out, q, q_stride, key_cache, value_cache, block_tables, max_num_blocks_per_seq,
                         context_lens, max_context_len, visible_pos, num_visible, vis_stride, num_seqs,
                         num_heads, num_kv_heads, head_size, block_size, num_blocks, scale, nullptr, 0, stream,
                         nullptr, 1, true);
}

q8_status q8_paged_decode_rows(float* out, const float* q, uint32_t q_stride,
                               const uint32_t* key_cache, const uint32_t* value_cache,
                               const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                               const uint32_t* context_lens, uint32_t max_context_len, uint32_t rows_per_seq,
                               uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                               uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return decode_common(out, q, q_stride, key_cache, value_cache, block_tables, max_num_blocks_per_seq,
                         context_lens, max_context_len, nullptr, nullptr, 0, num_seqs, num_heads, num_kv_heads,
                         head_size, block_size, num_blocks, scale, workspace, workspace_bytes, stream, nullptr,
                         rows_per_seq);
}

q8_status q8_decode_step(float* out, const float* q, uint32_t q_stride,
                         const float* key, uint32_t key_stride,
                         const float* value, uint32_t value_stride,
                         uint32_t* key_cache, uint32_t* value_cache,
                         const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                         const uint32_t* context_lens, uint32_t max_context_len,
                         uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                         uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                         float scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
    const AppendArgs app{key, value, key_stride, value_stride, key_cache, value_cache};
    return decode_common(out, q, q_stride, key_cache, value_cache, block_tables, max_num_blocks_per_seq,
                         context_lens, max_context_len, nullptr, nullptr, 0, num_seqs, num_heads,
                         num_kv_heads, head_size, block_size, num_blocks, scale, workspace, workspace_bytes,
                         stream, &app, 1);
}

q8_status q8_norm_rope_decode_step(float* out, const float* q, uint32_t q_stride, uint32_t q_head_stride,
                                   const float* key, uint32_t key_stride,
                                   const float* value, uint32_t value_stride,
                                   uint32_t* key_cache, uint32_t* value_cache,
                                   const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                                   const uint32_t* context_lens, uint32_t max_context_len,
                                   const float* q_weight, const float* k_weight, const float* table,
                                   uint32_t rot, uint32_t num_positions, float eps,
                                   uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                                   uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                                   float scale, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (!rope_shape_ok(head_size, rot, num_positions, eps)) return Q8_ERR_SHAPE;
    if (num_seqs > 0 && (!q_weight || !k_weight || (rot > 0 && !table))) return Q8_ERR_NULL;
    const AppendArgs app{key, value, key_stride, value_stride, key_cache, value_cache};
    const NormRopeStepArgs nr{q_weight, k_weight, table, rot, num_positions, eps};
    return decode_common(out, q, q_stride, key_cache, value_cache, block_tables, max_num_blocks_per_seq,
                         context_lens, max_context_len, nullptr, nullptr, 0, num_seqs, num_heads,
                         num_kv_heads, head_size, block_size, num_blocks, scale, workspace, workspace_bytes,
                         stream, &app, 1, false, &nr, q_head_stride);
}

}  // extern "C"

namespace {

// Writers and decodes of the full-width baseline caches: elem_bytes 4 (f32)
// or 2 (bfloat16).
q8_status baseline_write(const float* key, uint32_t key_stride, const float* value, uint32_t value_stride,
                         void* key_cache, void* value_cache, const uint32_t* slot_mapping, uint32_t num_tokens,
                         uint32_t num_kv_heads, uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                         uint32_t elem_bytes, void* stream) {
    if (!head_size_ok(head_size) || block_size == 0 || num_kv_heads == 0 || num_blocks == 0) return Q8_ERR_SHAPE;
    const uint64_t row = static_cast<uint64_t>(num_kv_heads) * head_size;
    if (key_stride < row || value_stride < row) return Q8_ERR_SHAPE;
    if (num_tokens == 0) return Q8_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping) return Q8_ERR_NULL;
    // one thread per 16-byte unit of a (token, kv head) row, 256 per workgroup
    const uint32_t epl = 16 / elem_bytes;
    if ((static_cast<uint64_t>(num_tokens) * num_kv_heads * (head_size / epl) + 255) / 256 > q8kv::kMaxGridBlocks)
        return Q8_ERR_SHAPE;
    if (head_size % epl != 0) return Q8_ERR_UNSUPPORTED;      // bfloat16 rows are written in units of 8
    if (reinterpret_cast<uintptr_t>(key_cache) % 16 != 0 || reinterpret_cast<uintptr_t>(value_cache) % 16 != 0)
        return Q8_ERR_UNSUPPORTED;
    q8kv::BaselineWriteArgs a{};
    a.key = key;
    a.value = value;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.slot_mapping = slot_mapping;
    a.key_stride = key_stride;
    a.value_stride = value_stride;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.head_size = head_size;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.elem_bytes = elem_bytes;
    const hipError_t e = q8kv::launch_baseline_write(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

size_t baseline_workspace_bytes(uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads, uint32_t head_size) {
    if (num_kv_heads == 0 || num_heads == 0 || num_heads % num_kv_heads != 0) return 0;
    return q8kv::plan_baseline_decode(num_seqs, num_heads, num_kv_heads, head_size).bytes;
}

q8_status baseline_decode(float* out, const float* q, uint32_t q_stride, const void* key_cache,
                          const void* value_cache, const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                          const uint32_t* context_lens, uint32_t max_context_len, uint32_t num_seqs,
                          uint32_t num_heads, uint32_t num_kv_heads, uint32_t head_size, uint32_t block_size,
                          uint32_t num_blocks, float scale, void* workspace, size_t workspace_bytes,
                          uint32_t elem_bytes, void* stream) {
    if (!head_size_ok(head_size) || block_size == 0 || num_heads == 0 || num_kv_heads == 0 ||
        num_heads % num_kv_heads != 0)
        return Q8_ERR_SHAPE;
    if (static_cast<uint64_t>(q_stride) < static_cast<uint64_t>(num_heads) * head_size) return Q8_ERR_SHAPE;
    if (!std::isfinite(scale)) return Q8_ERR_SHAPE;
    if (max_context_len > 0 && (max_num_blocks_per_seq == 0 || num_blocks == 0)) return Q8_ERR_SHAPE;
    if (head_size != 16 && head_size != 32 && head_size != 64 && head_size != 128 && head_size != 256)
        return Q8_ERR_UNSUPPORTED;
    if (max_context_len >= 0x80000000u || q_stride % 4 != 0) return Q8_ERR_UNSUPPORTED;
    if (num_seqs == 0) return Q8_OK;
    if (!out || !q || !key_cache || !value_cache || !block_tables || !context_lens) return Q8_ERR_NULL;
    for (const void* p : {static_cast<const void*>(out), static_cast<const void*>(q), key_cache, value_cache})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return Q8_ERR_UNSUPPORTED;
    const q8kv::BaselineDecodePlan p = q8kv::plan_baseline_decode(num_seqs, num_heads, num_kv_heads, head_size);
    if (p.num_waves > 0x7FFFFFFFull || p.recs_per_rg > 0x7FFFFFFFull) return Q8_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < p.bytes || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return Q8_ERR_WORKSPACE;
    q8kv::BaselineDecodeArgs a{};
    a.out = out;
    a.q = q;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    char* ws = static_cast<char*>(workspace);
    a.counters = reinterpret_cast<uint32_t*>(ws + p.counters_offset);
    a.part_acc = reinterpret_cast<float*>(ws + p.acc_offset);
    a.part_ml = reinterpret_cast<float*>(ws + p.ml_offset);
    a.q_stride = q_stride;
    a.max_num_blocks_per_seq = max_num_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_size = head_size;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.group = p.group;
    a.num_groups = p.num_groups;
    a.waves_per_rg = p.waves_per_rg;
    a.recs_per_rg = static_cast<uint32_t>(p.recs_per_rg);
    a.elem_bytes = elem_bytes;
    a.inv_block_size = 1.0f / static_cast<float>(block_size);
    a.scale_log2 = scale * 1.4426950408889634f;
    const hipError_t e = q8kv::launch_baseline_decode(a, p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

}  // namespace

extern "C" {

q8_status q8_f32_cache_write(const float* key, uint32_t key_stride,
                             const float* value, uint32_t value_stride,
                             float* key_cache, float* value_cache,
                             const uint32_t* slot_mapping, uint32_t num_tokens,
                             uint32_t num_kv_heads, uint32_t head_size,
                             uint32_t block_size, uint32_t num_blocks, void* stream) {
    return baseline_write(key, key_stride, value, value_stride, key_cache, value_cache, slot_mapping, num_tokens,
                          num_kv_heads, head_size, block_size, num_blocks, 4, stream);
}

size_t q8_f32_paged_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_heads,
                                           uint32_t num_kv_heads, uint32_t head_size) {
    return baseline_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size);
}

q8_status q8_f32_paged_decode(float* out, const float* q, uint32_t q_stride,
                              const float* key_cache, const float* value_cache,
                              const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                              const uint32_t* context_lens, uint32_t max_context_len,
                              uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                              uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                              float scale, void* workspace, size_t workspace_bytes,
                              void* stream) {
    return baseline_decode(out, q, q_stride, key_cache, value_cache, block_tables, max_num_blocks_per_seq,
                           context_lens, max_context_len, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                           num_blocks, scale, workspace, workspace_bytes, 4, stream);
}

q8_status q8_bf16_cache_write(const float* key, uint32_t key_stride,
                              const float* value, uint32_t value_stride,
                              uint16_t* key_cache, uint16_t* value_cache,
                              const uint32_t* slot_mapping, uint32_t num_tokens,
                              uint32_t num_kv_heads, uint32_t head_size,
                              uint32_t block_size, uint32_t num_blocks, void* stream) {
    return baseline_write(key, key_stride, value, value_stride, key_cache, value_cache, slot_mapping, num_tokens,
                          num_kv_heads, head_size, block_size, num_blocks, 2, stream);
}

size_t q8_bf16_paged_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_heads,
                                            uint32_t num_kv_heads, uint32_t head_size) {
    return baseline_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size);
}

q8_status q8_bf16_paged_decode(float* out, const float* q, uint32_t q_stride,
                               const uint16_t* key_cache, const uint16_t* value_cache,
                               const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                               const uint32_t* context_lens, uint32_t max_context_len,
                               uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                               uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return baseline_decode(out, q, q_stride, key_cache, value_cache, block_tables, max_num_blocks_per_seq,
                           context_lens, max_context_len, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                           num_blocks, scale, workspace, workspace_bytes, 2, stream);
}

q8_status q8_rope_table(float* table, uint32_t num_positions, uint32_t rot, float theta, void* stream) {
    if (rot % 2 != 0 || !(theta > 0.0f) || !std::isfinite(theta)) return Q8_ERR_SHAPE;
    if (rot == 0 || num_positions == 0) return Q8_OK;
    if (!table) return Q8_ERR_NULL;
    // one thread per (position, pair), 256 per workgroup
    if ((static_cast<uint64_t>(num_positions) * (rot / 2) + 255) / 256 > q8kv::kMaxGridBlocks) return Q8_ERR_UNSUPPORTED;
    const hipError_t e = q8kv::launch_rope_table(table, num_positions, rot, static_cast<double>(theta),
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// Validation and argument block of q8_norm_rope; *empty when nothing is to be done.
q8_status norm_rope_args(q8kv::NormRopeArgs& a, bool* empty, float* out, uint32_t out_stride, const float* x,
                         uint32_t x_stride, uint32_t head_stride, uint32_t num_rows, uint32_t num_heads,
                         uint32_t head_size, const uint32_t* positions, const float* weight, const float* table,
                         uint32_t rot, uint32_t num_positions, float eps) {
    *empty = true;
    if (!rope_shape_ok(head_size, rot, num_positions, eps) || head_stride < head_size) return Q8_ERR_SHAPE;
    if (num_heads > 0) {
        const uint64_t span = static_cast<uint64_t>(num_heads - 1) * head_stride + head_size;
        if (x_stride < span || out_stride < static_cast<uint64_t>(num_heads) * head_size) return Q8_ERR_SHAPE;
    }
    if (num_rows == 0 || num_heads == 0) return Q8_OK;
    if (!out || !x || !weight || (rot > 0 && (!table || !positions))) return Q8_ERR_NULL;
    // at most one (row, head) unit per wave, four waves per workgroup
    if (static_cast<uint64_t>(num_rows) * num_heads > q8kv::kMaxGridBlocks * 4) return Q8_ERR_UNSUPPORTED;
    a.out = out;
    a.x = x;
    a.positions = positions;
    a.weight = weight;
    a.table = table;
    a.x_stride = x_stride;
    a.head_stride = head_stride;
    a.out_stride = out_stride;
    a.num_rows = num_rows;
    a.num_heads = num_heads;
    a.head_size = head_size;
    a.rot = rot;
    a.num_positions = num_positions;
    a.eps = eps;
    a.params_vec4 = reinterpret_cast<uintptr_t>(weight) % 16 == 0 && reinterpret_cast<uintptr_t>(table) % 16 == 0;
    *empty = false;
    return Q8_OK;
}

// Validation and argument block of q8_norm_rope_cache_write.
q8_status norm_rope_write_args(q8kv::NormRopeCacheWriteArgs& a, bool* empty, const float* key, uint32_t key_stride,
                               const float* value, uint32_t value_stride, uint32_t* key_cache,
                               uint32_t* value_cache, const uint32_t* slot_mapping, const uint32_t* positions,
                               const float* weight, const float* table, uint32_t rot, uint32_t num_positions,
                               float eps, uint32_t num_tokens, uint32_t num_kv_heads, uint32_t head_size,
                               uint32_t block_size, uint32_t num_blocks) {
    *empty = true;
    if (!rope_shape_ok(head_size, rot, num_positions, eps) || block_size == 0 || num_kv_heads == 0)
        return Q8_ERR_SHAPE;
    const uint64_t row = static_cast<uint64_t>(num_kv_heads) * head_size;
    if (key_stride < row || value_stride < row) return Q8_ERR_SHAPE;
    if (num_tokens == 0) return Q8_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping || !weight ||
        (rot > 0 && (!table || !positions)))
        return Q8_ERR_NULL;
    if (num_blocks == 0) return Q8_ERR_SHAPE;
    // at most one (token, kv head) pair per wave, four waves per workgroup
    if (static_cast<uint64_t>(num_tokens) * num_kv_heads > q8kv::kMaxGridBlocks * 4) return Q8_ERR_UNSUPPORTED;
    a.key = key;
    a.value = value;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.slot_mapping = slot_mapping;
    a.positions = positions;
    a.weight = weight;
    a.table = table;
    a.key_stride = key_stride;
    a.value_stride = value_stride;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.head_size = head_size;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.rot = rot;
    a.num_positions = num_positions;
    a.eps = eps;
    a.params_vec4 = reinterpret_cast<uintptr_t>(weight) % 16 == 0 && reinterpret_cast<uintptr_t>(table) % 16 == 0;
    *empty = false;
    return Q8_OK;
}

}  // namespace

extern "C" {

q8_status q8_norm_rope(float* out, uint32_t out_stride, const float* x, uint32_t x_stride,
                       uint32_t head_stride, uint32_t num_rows, uint32_t num_heads, uint32_t head_size,
                       const uint32_t* positions, const float* weight, const float* table,
                       uint32_t rot, uint32_t num_positions, float eps, void* stream) {
    q8kv::NormRopeArgs a{};
    bool empty;
    const q8_status st = norm_rope_args(a, &empty, out, out_stride, x, x_stride, head_stride, num_rows, num_heads,
                                        head_size, positions, weight, table, rot, num_positions, eps);
    if (st != Q8_OK || empty) return st;
    const hipError_t e = q8kv::launch_norm_rope(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

q8_status q8_norm_rope_cache_write(const float* key, uint32_t key_stride,
                                   const float* value, uint32_t value_stride,
                                   uint32_t* key_cache, uint32_t* value_cache,
                                   const uint32_t* slot_mapping, const uint32_t* positions,
                                   const float* weight, const float* table, uint32_t rot,
                                   uint32_t num_positions, float eps, uint32_t num_tokens,
                                   uint32_t num_kv_heads, uint32_t head_size,
                                   uint32_t block_size, uint32_t num_blocks, void* stream) {
    q8kv::NormRopeCacheWriteArgs a{};
    bool empty;
    const q8_status st = norm_rope_write_args(a, &empty, key, key_stride, value, value_stride, key_cache, value_cache,
                                              slot_mapping, positions, weight, table, rot, num_positions, eps,
                                              num_tokens, num_kv_heads, head_size, block_size, num_blocks);
    if (st != Q8_OK || empty) return st;
    const hipError_t e = q8kv::launch_norm_rope_cache_write(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

q8_status q8_norm_rope_qk_cache_write(float* q_out, uint32_t q_out_stride, const float* q, uint32_t q_stride,
                                      uint32_t q_head_stride, uint32_t num_q_rows, uint32_t num_heads,
                                      const uint32_t* q_positions, const float* q_weight,
                                      const float* key, uint32_t key_stride, const float* value,
                                      uint32_t value_stride, uint32_t* key_cache, uint32_t* value_cache,
                                      const uint32_t* slot_mapping, const uint32_t* positions,
                                      const float* k_weight, const float* table, uint32_t rot,
                                      uint32_t num_positions, float eps, uint32_t num_tokens,
                                      uint32_t num_kv_heads, uint32_t head_size, uint32_t block_size,
                                      uint32_t num_blocks, void* stream) {
    q8kv::NormRopeArgs qa{};
    q8kv::NormRopeCacheWriteArgs ka{};
    bool q_empty, k_empty;
    q8_status st = norm_rope_args(qa, &q_empty, q_out, q_out_stride, q, q_stride, q_head_stride, num_q_rows, num_heads,
                                  head_size, q_positions, q_weight, table, rot, num_positions, eps);
    if (st != Q8_OK) return st;
    st = norm_rope_write_args(ka, &k_empty, key, key_stride, value, value_stride, key_cache, value_cache, slot_mapping,
                              positions, k_weight, table, rot, num_positions, eps, num_tokens, num_kv_heads,
                              head_size, block_size, num_blocks);
    if (st != Q8_OK || (q_empty && k_empty)) return st;
    const hipError_t e = q8kv::launch_norm_rope_qk_cache_write(qa, ka, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

q8_status q8_index_select(const float* scores, uint32_t score_stride, const uint32_t* row_lens,
                          uint32_t num_rows, uint32_t ratio, uint32_t k, uint32_t* visible_pos,
                          uint32_t vis_stride, uint32_t* num_visible, uint32_t* visible_mask,
                          uint32_t mask_stride, void* stream) {
    if (ratio == 0 || (static_cast<uint64_t>(k) + 1) * ratio > vis_stride) return Q8_ERR_SHAPE;
    // a bit for each block a row can touch: score_stride complete ones and a trailing one
    if (visible_mask && static_cast<uint64_t>(mask_stride) * 32 < static_cast<uint64_t>(score_stride) + 1)
        return Q8_ERR_SHAPE;
    if (score_stride > q8kv::kSelectMaxBlocks) return Q8_ERR_UNSUPPORTED;
    if (num_rows == 0) return Q8_OK;
    if (!scores || !row_lens || !visible_pos || !num_visible) return Q8_ERR_NULL;
    if (num_rows > 0x7FFFFFFFu) return Q8_ERR_UNSUPPORTED;
    q8kv::IndexSelectArgs a{};
    a.scores = scores;
    a.row_lens = row_lens;
    a.visible_pos = visible_pos;
    a.num_visible = num_visible;
    a.score_stride = score_stride;
    a.num_rows = num_rows;
    a.ratio = ratio;
    a.k = k;
    a.vis_stride = vis_stride;
    a.visible_mask = visible_mask;
    a.mask_stride = visible_mask ? mask_stride : 0;
    const hipError_t e = q8kv::launch_index_select(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_last_hip_error(void) { return g_last_hip_error; }

q8_status q8_bounds_flags(uint32_t* flags, int clear) {
    if (!flags) return Q8_ERR_NULL;
    *flags = 0;
#ifdef Q8_DEBUG_BOUNDS
    uint32_t* p = bounds_flags_ptr();
    if (!p) return hip_fail(hipErrorInvalidSymbol);
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(flags, p, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess && clear) e = hipMemset(p, 0, sizeof(uint32_t));
    return e == hipSuccess ? Q8_OK : hip_fail(e);
#else
    (void)clear;
    return Q8_ERR_UNSUPPORTED;
#endif
}

const char* q8_status_string(q8_status status) {
    switch (status) {
        case Q8_OK: return "Q8_OK";
        case Q8_ERR_NULL: return "Q8_ERR_NULL";
        case Q8_ERR_SHAPE: return "Q8_ERR_SHAPE";
        case Q8_ERR_WORKSPACE: return "Q8_ERR_WORKSPACE";
        case Q8_ERR_HIP: return "Q8_ERR_HIP";
        case Q8_ERR_UNSUPPORTED: return "Q8_ERR_UNSUPPORTED";
    }
    return "Q8_UNKNOWN";
}

}  // extern "C"
