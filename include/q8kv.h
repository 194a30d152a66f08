/*
 * q8kv.h -- C ABI of libq8kv.so: int8 paged KV cache write and single-query
 * paged decode attention on AMD MI355X (gfx950).
 *
 * Cache format (the "paged_attn_q8.comp" and "reshape_and_cache_q8.comp"
 * pages, header comment "Quantized cache (K and V), u32 buffer"):
 *   a u32 buffer [num_blocks, num_kv_heads, block_size, words_per_token],
 *   words_per_token = head_size/4 + 1.  One token's vector for one kv head is
 *   head_size/4 code words, each holding four signed int8 codes with element
 *   4w+l in byte l (little-endian lane), followed by one word holding the bits
 *   of the f32 per-token scale.  K and V use two separate buffers of this shape.
 *   A value dequantizes as code * scale.
 *
 * Conventions for every entry point:
 *   - Array pointers are DEVICE pointers owned by the caller.  The library
 *     keeps no per-call state and allocates no memory (the one exception to
 *     the first: q8_paged_decode_noalloc's scratch array, below).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work; they never synchronize.  They are reentrant.
 *   - Shapes are validated on the host before anything is enqueued; on any
 *     non-OK return nothing has been enqueued.
 *   - The CONTENTS of device arrays are a caller contract and are not checked
 *     (as in the pages' shaders): slots below num_blocks*block_size or the pad
 *     value, distinct non-pad slots within one write, block ids below
 *     num_blocks, block-table rows holding valid ids for every block a
 *     sequence uses, finite inputs.  Breaking it is undefined behaviour.
 *   - head_size must be a multiple of 4 and at most 256 (the pages' maximum).
 *   - Two environment variables, meant for tests, force the number of
 *     persistent wavefronts the decodes split the batch over (otherwise:
 *     as many as the device keeps resident for the kernel, at most 2048 for
 *     the int8 decodes, and 2048 for the f32 and bf16 decodes):
 *     Q8KV_DECODE_WAVES (int8 decodes and the decode step) and
 *     Q8KV_F32_DECODE_WAVES (the f32 and bf16 decodes),
 *     each an integer from 1 to 2^20, read by every call.  The workspace
 *     query reads the same variable, so a workspace sized under one setting
 *     must be used under it.  Results do not depend on the setting beyond
 *     f32 rounding.
 */
#ifndef Q8KV_H
#define Q8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* slot_mapping value meaning "skip this token" (the writer page's PAD_SLOT). */
#define Q8_PAD_SLOT 0xFFFFFFFFu
#define Q8_MAX_HEAD_SIZE 256u

typedef enum {
    Q8_OK = 0,
    Q8_ERR_NULL = 1,         /* a required pointer is NULL */
    Q8_ERR_SHAPE = 2,        /* sizes or strides violate the limits listed per call */
    Q8_ERR_WORKSPACE = 3,    /* workspace too small or not 16-byte aligned */
    Q8_ERR_HIP = 4,          /* a HIP launch failed; see q8_last_hip_error() */
    Q8_ERR_UNSUPPORTED = 5   /* a valid combination the library does not handle */
} q8_status;

/*
 * q8_cache_write -- quantize the new K and V vectors of num_tokens tokens and
 * pack them into the paged caches ("reshape_and_cache_q8.comp" page, main():
 * per (token, kv head), amax = max|x|, inv = amax > 0 ? 127/amax : 0, code =
 * clamp(round(x*inv), -127, 127), scale word = bits(amax > 0 ? amax/127 : 1.0);
 * K and V are both written by the one call).
 *
 *   key, value   f32 device arrays: element d of kv head h of token t is at
 *                key[t*key_stride + h*head_size + d] (resp. value_stride).
 *   key_cache,   u32 device caches [num_blocks, num_kv_heads, block_size,
 *   value_cache  head_size/4 + 1], written at row (slot/block_size, h,
 *                slot%block_size) for every non-pad slot.
 *   slot_mapping u32 [num_tokens]; Q8_PAD_SLOT skips the token: nothing is
 *                read or written for it (as on the page, its key/value rows
 *                are not touched).
 *
 * Rounding: every step is one IEEE binary32 operation with round-to-nearest,
 * and the round() of the page is round-half-even.  The output is bit-exact.
 * Errors: Q8_ERR_NULL for a NULL array with num_tokens > 0; Q8_ERR_SHAPE when
 * head_size is 0, not a multiple of 4 or above 256, when block_size or
 * num_kv_heads is 0, when a stride is below num_kv_heads*head_size, or when
 * the launch would need more than 2^31 - 1 workgroups (one per 16 tokens of a
 * kv head once num_tokens*num_kv_heads reaches 32768, one per four (token,
 * kv head) pairs below).  num_tokens == 0 returns Q8_OK and enqueues nothing.
 */
q8_status q8_cache_write(const float* key, uint32_t key_stride,
                         const float* value, uint32_t value_stride,
                         uint32_t* key_cache, uint32_t* value_cache,
                         const uint32_t* slot_mapping, uint32_t num_tokens,
                         uint32_t num_kv_heads, uint32_t head_size,
                         uint32_t block_size, uint32_t num_blocks, void* stream);

/*
 * q8_paged_decode_workspace_bytes -- bytes of device workspace q8_paged_decode
 * needs for these sizes: softmax partials (running max, sum and unnormalized
 * output row per query head) of sequences whose positions are split over
 * several wavefronts, plus one arrival counter per (kv head group, sequence);
 * the split-context decode with a combine step follows the "attention.rs"
 * page.  max_positions is max_context_len in dense mode and vis_stride in
 * visible-list mode.  Returns 0 when no workspace is needed (every sequence
 * has at most 32 positions).  Pure host arithmetic; needs no GPU.
 */
size_t q8_paged_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_heads,
                                       uint32_t num_kv_heads, uint32_t head_size,
                                       uint32_t block_size, uint32_t max_positions);

/*
 * q8_paged_decode -- single-query decode attention over the int8 paged cache
 * ("paged_attn_q8.comp" page: output = softmax(scale * Q.K^T) . V with K and
 * V dequantized on read, kv head = h / (num_heads/num_kv_heads), token t at
 * block_tables[s*max_num_blocks_per_seq + t/block_size], offset
 * t % block_size, context length clamped to max_context_len).
 *
 *   out           f32 [num_seqs, num_heads, head_size], dense, 16-byte aligned.
 *   q             f32; element d of head h of seq s at q[s*q_stride + h*head_size + d].
 *   key_cache,    u32 caches in the format above.
 *   value_cache
 *   block_tables  u32 [num_seqs, max_num_blocks_per_seq].
 *   context_lens  u32 [num_seqs]; seq s attends positions
 *                 0 .. min(context_lens[s], max_context_len) - 1.
 *   visible_pos,  optional visible-list mode (the "attention.rs" page's
 *   num_visible,  selective decode over the row's visible token list): when
 *   vis_stride    visible_pos != NULL, seq s attends exactly the positions
 *                 visible_pos[s*vis_stride + i], i < num_visible[s]
 *                 (num_visible[s] <= vis_stride; positions ascending and
 *                 distinct: 64 listed positions from a multiple of 64 to 63
 *                 above it are read as one tile run);
 *                 context_lens and max_context_len are then unused.
 *   scale         f32 softmax scale applied to q.k.
 *   workspace     device memory of at least q8_paged_decode_workspace_bytes()
 *                 bytes, 16-byte aligned, ZERO-FILLED before its first use
 *                 (e.g. hipMemset once after allocation).  Each completed
 *                 call leaves its counters at zero again, so the same
 *                 workspace serves any later call without clearing; after a
 *                 failed or aborted launch, zero it again.  Concurrent calls
 *                 need distinct workspaces.
 *
 * An empty position set gives a zero output row.  Accuracy: each output is
 * within 1e-4 + 1e-4*|exact| of the exact attention over the dequantized cache
 * for the documented workloads (f32 arithmetic throughout).
 * Errors: Q8_ERR_NULL for a NULL required pointer; Q8_ERR_SHAPE when
 * head_size is 0, not a multiple of 4 or above 256, block_size, num_heads or
 * num_kv_heads is 0, num_heads % num_kv_heads != 0, q_stride <
 * num_heads*head_size, max_num_blocks_per_seq is 0 while positions are
 * possible, or vis_stride is 0 in visible-list mode; Q8_ERR_WORKSPACE when the
 * workspace is too small or misaligned; Q8_ERR_UNSUPPORTED when out is not
 * 16-byte aligned.  num_seqs == 0 enqueues nothing.
 */
q8_status q8_paged_decode(float* out, const float* q, uint32_t q_stride,
                          const uint32_t* key_cache, const uint32_t* value_cache,
                          const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                          const uint32_t* context_lens, uint32_t max_context_len,
                          const uint32_t* visible_pos, const uint32_t* num_visible,
                          uint32_t vis_stride,
                          uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                          uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                          float scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * q8_paged_decode_noalloc -- q8_paged_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The partial records
 * and arrival counters live in a fixed device array of
 * Q8_NOALLOC_SCRATCH_BYTES inside the library; each GPU the library runs on
 * holds its own copy until the process ends.  The call allocates nothing:
 * the first call on a device looks up the array's address
 * (hipGetSymbolAddress) and clears it with a fill kernel on `stream`.
 *
 *   All arguments mean what they mean for q8_paged_decode (dense or
 *   visible-list mode); the results are the same as those of q8_paged_decode
 *   with its own workspace.
 *
 * Every call on one GPU shares that GPU's array, and each call leaves it ready
 * for the next: calls on one GPU must not overlap (the same stream, or
 * streams ordered by the caller); overlapping calls race on the array and
 * give undefined results.  After a failed or aborted launch the array's
 * counters may be left nonzero and later results are undefined.
 * Errors: those of q8_paged_decode, except that Q8_ERR_WORKSPACE means these
 * sizes need more than Q8_NOALLOC_SCRATCH_BYTES of scratch
 * (q8_paged_decode_workspace_bytes gives the need); Q8_ERR_HIP when the
 * array's address cannot be found; Q8_ERR_UNSUPPORTED on a device ordinal
 * of 64 or more.
 */
#define Q8_NOALLOC_SCRATCH_BYTES (32u << 20)
q8_status q8_paged_decode_noalloc(float* out, const float* q, uint32_t q_stride,
                                  const uint32_t* key_cache, const uint32_t* value_cache,
                                  const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                                  const uint32_t* context_lens, uint32_t max_context_len,
                                  const uint32_t* visible_pos, const uint32_t* num_visible,
                                  uint32_t vis_stride,
                                  uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                                  uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                                  float scale, void* stream);

/*
 * q8_decode_step -- one decode step in a single launch: every sequence's new K
 * and V vector is quantized and packed into the caches at the sequence's last
 * position, and the batch attends over the caches including it.  The result
 * (cache words and outputs) is that of q8_cache_write of token s at the slot
 * of position context_lens[s]-1 of sequence s (its block_tables entry, offset
 * position % block_size), followed by q8_paged_decode in dense mode; the
 * packing is the "reshape_and_cache_q8.comp" page's, the attention the
 * "paged_attn_q8.comp" page's.  One launch instead of two: the wavefront that
 * attends the last chunk of a sequence quantizes the new rows itself, uses them
 * in place of the rows the cache still held, and writes them to the caches.
 *
 *   key, value    f32 new vectors: element d of kv head h of sequence s at
 *                 key[s*key_stride + h*head_size + d] (resp. value_stride).
 *   key_cache,    u32 caches, read and written.
 *   value_cache
 *   the rest      as q8_paged_decode in dense mode (visible lists are not
 *                 supported here), including the workspace
 *                 (q8_paged_decode_workspace_bytes with max_positions =
 *                 max_context_len).
 *
 * Contract on the contents (not checked): the new position's slot is attended
 * by no other sequence of the call.  A sequence is appended to only when
 * 1 <= context_lens[s] <= max_context_len and its table covers position
 * context_lens[s]-1; otherwise nothing is written for it and it attends the
 * cache as it is.  Errors: those of q8_paged_decode in dense mode, plus
 * Q8_ERR_NULL for a NULL key or value and Q8_ERR_SHAPE for a stride below
 * num_kv_heads*head_size.
 */
q8_status q8_decode_step(float* out, const float* q, uint32_t q_stride,
                         const float* key, uint32_t key_stride,
                         const float* value, uint32_t value_stride,
                         uint32_t* key_cache, uint32_t* value_cache,
                         const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                         const uint32_t* context_lens, uint32_t max_context_len,
                         uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                         uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                         float scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * q8_paged_decode_rows -- multi-row causal decode: rows_per_seq (nb) query
 * rows per sequence at its last nb positions, as in chunked prefill or
 * speculative verification ("attention.rs" page, attention_b: row b of the nb
 * rows starting at base_pos attends its causal prefix of base_pos + b + 1
 * positions, with the "paged_attn_q8.comp" page's attention over it).  Here
 * base_pos = context_lens[s] - nb: row b of sequence s attends positions
 * 0 .. context_lens[s] - nb + b, clamped to max_context_len (a row whose
 * prefix is empty gets a zero row).  The rows of a sequence share its
 * block_tables row and its K/V reads: they are processed as extra query
 * heads of each kv head, each with its own causal limit.
 *
 *   out           f32 [num_seqs * nb, num_heads, head_size], dense, 16-byte
 *                 aligned; row b of sequence s at index s*nb + b.
 *   q             f32; element d of head h of row b of sequence s at
 *                 q[(s*nb + b)*q_stride + h*head_size + d].
 *   workspace     q8_paged_decode_workspace_bytes(num_seqs, num_heads * nb,
 *                 num_kv_heads, head_size, block_size, max_context_len).
 *   the rest      as q8_paged_decode in dense mode.
 *
 * nb == 1 is q8_paged_decode.  Errors: those of q8_paged_decode in dense mode,
 * plus Q8_ERR_SHAPE for nb == 0.
 */
q8_status q8_paged_decode_rows(float* out, const float* q, uint32_t q_stride,
                               const uint32_t* key_cache, const uint32_t* value_cache,
                               const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                               const uint32_t* context_lens, uint32_t max_context_len, uint32_t rows_per_seq,
                               uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                               uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * f32 paged-cache baseline.  The "paged_attn_q8.comp" page's header says the
 * int8 decode keeps the math and workgroup structure of an f32 paged decode
 * whose cache holds 4 bytes per element, and the "reshape_and_cache_q8.comp"
 * page's header says its pad-slot rule mirrors the f32 writer.  The pages do
 * not print the f32 layout; here it is the int8 layout with one f32 per
 * element: an f32 buffer [num_blocks, num_kv_heads, block_size, head_size]
 * for K and one for V.  These calls exist so that the int8 cache can be
 * measured against the f32 one on the same batch.
 *
 * q8_f32_cache_write -- copy the new K and V vectors of num_tokens tokens
 * into the f32 paged caches at their slots (block slot / block_size, offset
 * slot % block_size); a slot equal to Q8_PAD_SLOT skips the token.
 *
 *   key, value   f32 device arrays, as for q8_cache_write.
 *   key_cache,   f32 device caches in the layout above, 16-byte aligned.
 *   value_cache
 *   slot_mapping u32 [num_tokens].
 *
 * Errors: Q8_ERR_NULL for a NULL pointer when num_tokens > 0; Q8_ERR_SHAPE
 * when head_size is 0, not a multiple of 4 or above 256, block_size,
 * num_kv_heads or num_blocks is 0, a stride is below num_kv_heads *
 * head_size, or the launch would need more than 2^31 - 1 workgroups (one
 * thread per 16 bytes of the new rows, 256 per workgroup);
 * Q8_ERR_UNSUPPORTED when a cache is not 16-byte aligned.  num_tokens == 0
 * enqueues nothing.
 */
q8_status q8_f32_cache_write(const float* key, uint32_t key_stride,
                             const float* value, uint32_t value_stride,
                             float* key_cache, float* value_cache,
                             const uint32_t* slot_mapping, uint32_t num_tokens,
                             uint32_t num_kv_heads, uint32_t head_size,
                             uint32_t block_size, uint32_t num_blocks, void* stream);

/* Workspace bytes q8_f32_paged_decode needs for these sizes (0 when the
 * head counts are inconsistent). */
size_t q8_f32_paged_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_heads,
                                           uint32_t num_kv_heads, uint32_t head_size);

/*
 * q8_f32_paged_decode -- single-query decode over the f32 paged caches: for
 * each (seq s, head h), out = softmax(scale * q . K^T) . V over positions
 * 0 .. min(context_lens[s], max_context_len) - 1 of kv head
 * h / (num_heads / num_kv_heads), position t at block_tables[s][t /
 * block_size], offset t % block_size (the "paged_attn_q8.comp" page's math
 * with the f32 elements it replaces).
 *
 *   out           f32 [num_seqs, num_heads, head_size], dense, 16-byte aligned.
 *   q             f32, 16-byte aligned, q_stride a multiple of 4; element d
 *                 of head h of seq s at q[s*q_stride + h*head_size + d].
 *   key_cache,    f32 caches in the layout above, 16-byte aligned.
 *   value_cache
 *   block_tables, context_lens, max_context_len, scale: as q8_paged_decode.
 *   workspace     q8_f32_paged_decode_workspace_bytes() bytes, 16-byte
 *                 aligned, ZERO-FILLED before its first use; each completed
 *                 call leaves it ready for the next (as for q8_paged_decode).
 *
 * An empty position set gives a zero output row.  Errors: Q8_ERR_NULL for a
 * NULL required pointer; Q8_ERR_SHAPE when head_size is not a multiple of 4
 * or above 256, block_size, num_heads or num_kv_heads is 0, num_heads %
 * num_kv_heads != 0, q_stride < num_heads*head_size, or
 * max_num_blocks_per_seq or num_blocks is 0 while positions are possible;
 * Q8_ERR_WORKSPACE when the workspace is too small or misaligned;
 * Q8_ERR_UNSUPPORTED when head_size is not 16, 32, 64, 128 or 256, a pointer
 * above is not 16-byte aligned, q_stride is not a multiple of 4, or
 * max_context_len >= 2^31.  num_seqs == 0 enqueues nothing.
 */
q8_status q8_f32_paged_decode(float* out, const float* q, uint32_t q_stride,
                              const float* key_cache, const float* value_cache,
                              const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                              const uint32_t* context_lens, uint32_t max_context_len,
                              uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                              uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                              float scale, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * bfloat16 paged-cache baseline (not on the pages: the half-width cache most
 * serving stacks keep, so the int8 cache can be measured against it too).
 * Layout as the f32 baseline with 2-byte elements: a u16 buffer
 * [num_blocks, num_kv_heads, block_size, head_size] for K and one for V, each
 * element the bfloat16 encoding (the upper 16 bits of a binary32).
 *
 * q8_bf16_cache_write -- q8_f32_cache_write with every element rounded to the
 * nearest bfloat16, ties to the even encoding (inputs finite).  Errors: those
 * of q8_f32_cache_write, plus Q8_ERR_UNSUPPORTED when head_size is not a
 * multiple of 8 (rows are written in 16-byte units of 8 elements).
 *
 * q8_bf16_paged_decode_workspace_bytes, q8_bf16_paged_decode -- as the f32
 * calls, over the bfloat16 caches (each element widened to f32 exactly); the
 * arguments, workspace rules and errors are the same.
 */
q8_status q8_bf16_cache_write(const float* key, uint32_t key_stride,
                              const float* value, uint32_t value_stride,
                              uint16_t* key_cache, uint16_t* value_cache,
                              const uint32_t* slot_mapping, uint32_t num_tokens,
                              uint32_t num_kv_heads, uint32_t head_size,
                              uint32_t block_size, uint32_t num_blocks, void* stream);
size_t q8_bf16_paged_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_heads,
                                            uint32_t num_kv_heads, uint32_t head_size);
q8_status q8_bf16_paged_decode(float* out, const float* q, uint32_t q_stride,
                               const uint16_t* key_cache, const uint16_t* value_cache,
                               const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                               const uint32_t* context_lens, uint32_t max_context_len,
                               uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                               uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Per-head RMSNorm + partial rotary embedding.  The "attention.rs" page
 * normalizes q and k per head with a learned weight (rms eps) and rotates
 * the first rot = head_dim * partial_rotary_factor elements at the row's
 * position (rope theta) before the q8 append (its q/k norm-and-rope
 * dispatches); the kernel body is not printed.  Computed here, per head
 * vector x of head_size elements at position pos:
 *   r   = 1 / sqrt(mean_d x_d^2 + eps)          (binary64, rounded to f32)
 *   n_d = (x_d * r) * w_d                        (binary32 products)
 *   for i < rot/2, a = n_i, b = n_{i+rot/2}, c/s = table[pos][i], table[pos][rot/2 + i]:
 *     y_i = a*c - b*s,   y_{i+rot/2} = b*c + a*s (binary32, never fused)
 *   y_d = n_d for d >= rot.
 * rot must be 0 or a multiple of 8 not above head_size.  Inputs must be
 * finite; a zero vector with eps == 0 is outside the contract.
 *
 * q8_rope_table -- fill the rotary table: table[p*rot + i] =
 * cos(p * theta^(-2i/rot)) and table[p*rot + rot/2 + i] = sin(p *
 * theta^(-2i/rot)) for p < num_positions, i < rot/2, each evaluated in
 * binary64 and rounded to f32.  table: caller-owned device f32 array of
 * num_positions*rot elements.  Q8_ERR_SHAPE when rot is odd or theta is not
 * positive and finite; Q8_ERR_NULL for a NULL table with rot*num_positions > 0.
 */
q8_status q8_rope_table(float* table, uint32_t num_positions, uint32_t rot, float theta, void* stream);

/*
 * q8_norm_rope -- the step above on rows of heads (the q side): head h of row
 * t is read at x[t*x_stride + h*head_stride + d] and written to
 * out[t*out_stride + h*head_size + d], at position positions[t].
 *   weight     device f32 [head_size], shared by the heads.
 *   table      device f32 [num_positions, rot] from q8_rope_table (unused and
 *              may be NULL when rot == 0, as may positions).
 * positions[t] < num_positions is a caller contract (out-of-range values are
 * clamped, not reported).  out must not overlap x unless out == x with
 * matching strides (in place).  Errors: Q8_ERR_NULL; Q8_ERR_SHAPE when
 * head_size is not a multiple of 4 or above 256, rot is not a multiple of 8
 * or exceeds head_size, head_stride < head_size, x_stride or out_stride is
 * too small for num_heads heads, eps is negative or not finite, or rot > 0
 * with num_positions == 0.  num_rows == 0 enqueues nothing.
 */
q8_status q8_norm_rope(float* out, uint32_t out_stride, const float* x, uint32_t x_stride,
                       uint32_t head_stride, uint32_t num_rows, uint32_t num_heads, uint32_t head_size,
                       const uint32_t* positions, const float* weight, const float* table,
                       uint32_t rot, uint32_t num_positions, float eps, void* stream);

/*
 * q8_norm_rope_cache_write -- q8_cache_write with the step above applied to
 * the K vectors first: for each token whose slot is not Q8_PAD_SLOT, each kv
 * head's K vector becomes its normalized, rotated self at positions[t]
 * (weight: the K norm weight) and is packed as q8_cache_write packs it; V is
 * packed unchanged.  The arguments shared with q8_cache_write mean the same;
 * weight, table, rot, num_positions and eps are as for q8_norm_rope.  Nothing
 * is read or written for a pad token (rows, position).  Errors: those of
 * q8_cache_write plus the shape rules of q8_norm_rope.
 */
q8_status q8_norm_rope_cache_write(const float* key, uint32_t key_stride,
                                   const float* value, uint32_t value_stride,
                                   uint32_t* key_cache, uint32_t* value_cache,
                                   const uint32_t* slot_mapping, const uint32_t* positions,
                                   const float* weight, const float* table, uint32_t rot,
                                   uint32_t num_positions, float eps, uint32_t num_tokens,
                                   uint32_t num_kv_heads, uint32_t head_size,
                                   uint32_t block_size, uint32_t num_blocks, void* stream);

/*
 * q8_norm_rope_qk_cache_write -- q8_norm_rope on query rows and
 * q8_norm_rope_cache_write on the new K/V rows of the same step, in one launch.
 * The "attention.rs" page normalizes and rotates q and k together in one
 * dispatch (its qk_norm_rope_b) ahead of the q8 append; here that dispatch
 * also quantizes and packs K and V into the cache.  The result is exactly that
 * of q8_norm_rope(q_out, q_out_stride, q, q_stride, q_head_stride, num_q_rows,
 * num_heads, head_size, q_positions, q_weight, table, rot, num_positions, eps)
 * followed by q8_norm_rope_cache_write(key, ..., k_weight, table, ...): the
 * arguments mean the same as there, head_size, table, rot, num_positions and
 * eps are shared, and q_weight / k_weight are the q and K norm weights.  q_out
 * must not overlap key, value or the caches (q and q_out may be the same
 * rows).  Writes of at least 32768 (token, kv head) pairs take a second launch
 * (the bulk writer).  Errors: those of the two calls; either side may be empty
 * (num_q_rows or num_heads 0, num_tokens 0).
 */
q8_status q8_norm_rope_qk_cache_write(float* q_out, uint32_t q_out_stride, const float* q, uint32_t q_stride,
                                      uint32_t q_head_stride, uint32_t num_q_rows, uint32_t num_heads,
                                      const uint32_t* q_positions, const float* q_weight,
                                      const float* key, uint32_t key_stride, const float* value,
                                      uint32_t value_stride, uint32_t* key_cache, uint32_t* value_cache,
                                      const uint32_t* slot_mapping, const uint32_t* positions,
                                      const float* k_weight, const float* table, uint32_t rot,
                                      uint32_t num_positions, float eps, uint32_t num_tokens,
                                      uint32_t num_kv_heads, uint32_t head_size, uint32_t block_size,
                                      uint32_t num_blocks, void* stream);

/*
 * q8_norm_rope_decode_step -- q8_decode_step with the per-head RMSNorm +
 * partial rotary step above applied to the query rows and to the new K rows,
 * in the same single launch.  The "attention.rs" page normalizes and rotates q
 * and k ahead of the q8 append and the decode (its qk_norm_rope_b dispatch),
 * and its decode reads q heads 2*head_dim apart (q and the output gate
 * interleaved per head); here the wavefront that stages a sequence's q rows
 * normalizes and rotates them, and the one that appends its new K row does
 * the same to it before quantizing.  The result (outputs and cache words) is
 * exactly that of
 *   q8_norm_rope(q', .., q, q_stride, q_head_stride, .., positions, q_weight, table, rot, num_positions, eps)
 *   q8_norm_rope_cache_write(key, .., value, .., slots, positions, k_weight, ...)
 *   q8_paged_decode(out, q', ...)                       (dense mode)
 * with positions[s] = context_lens[s] - 1 and slots[s] the slot of that
 * position (its block_tables entry, offset position % block_size), for the
 * sequences q8_decode_step appends to (the others are not written, and their
 * q rows are still rotated at context_lens[s] - 1).  q itself is not written.
 *
 *   q             f32 query rows before the step: head h of sequence s at
 *                 q[s*q_stride + h*q_head_stride + d].
 *   q_head_stride elements between the heads of a row: head_size for packed
 *                 heads (0 means the same), 2*head_size for the q/gate
 *                 interleave; at least head_size, and q_stride at least
 *                 (num_heads-1)*q_head_stride + head_size.
 *   q_weight,     device f32 [head_size]: the q and K norm weights.
 *   k_weight
 *   table, rot,   as for q8_norm_rope (table unused and may be NULL when
 *   num_positions, rot == 0); a position past the table is clamped to its
 *   eps           last row, as there.
 *   the rest      as q8_decode_step, including the workspace.
 *
 * Errors: those of q8_decode_step; Q8_ERR_SHAPE under the shape rules of
 * q8_norm_rope or for a q_head_stride below head_size; Q8_ERR_NULL for a NULL
 * weight, or a NULL table with rot > 0 (num_seqs > 0); Q8_ERR_UNSUPPORTED
 * unless head_size is 64, 128 or 256, both caches are 16-byte aligned and
 * block_size is a multiple of 4 that divides, or is a multiple of, the
 * positions per chunk (32 for head_size <= 128 with num_heads / num_kv_heads
 * <= 4, else 64).  Other shapes take q8_norm_rope_qk_cache_write followed by
 * q8_paged_decode.
 */
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
                                   void* stream);

/*
 * q8_index_select -- block selection into a visible list.  The
 * "attention.rs" page's per-row decode gives row r t_len = row_lens[r]
 * positions and blocks = t_len / ratio complete blocks; with k = kblk
 * (budget / ratio) a row is selective when blocks > k and then attends
 * k*ratio + (t_len - blocks*ratio) positions, else all t_len, from a list
 * the indexer's select pass builds out of block scores (vis_stride = budget
 * + ratio apart).  The select kernel is not printed; computed here: the k
 * complete blocks of highest score (ties to the lower block index), their
 * positions ascending, then the trailing incomplete block's positions; with
 * blocks <= k, every position 0 .. t_len-1.  The lists feed q8_paged_decode's
 * visible-position mode directly.  The pass also emits the per-row block
 * bitmask the page sizes as ceil(max_blocks/32) words; its meaning is not
 * printed either: bit j (word j/32, bit j%32) is set exactly when the list
 * holds a position of block j.
 *   scores        device f32; row r's block j at scores[r*score_stride + j],
 *                 finite, read for j < blocks only.
 *   row_lens      device u32 [num_rows]: t_len per row; t_len / ratio <=
 *                 score_stride is a caller contract (clamped, not reported).
 *   visible_pos   device u32; row r's list at visible_pos[r*vis_stride + i],
 *                 i < num_visible[r]; entries past it are left untouched.
 *   num_visible   device u32 [num_rows].
 *   visible_mask  device u32 or NULL (no mask); row r's bits at
 *                 visible_mask[r*mask_stride + w], all mask_stride words
 *                 written (0 where no block is touched).
 *   mask_stride   words per mask row, >= ceil((score_stride + 1) / 32): a bit
 *                 for every complete block and the trailing one.  Ignored
 *                 when visible_mask is NULL.
 * Errors: Q8_ERR_NULL; Q8_ERR_SHAPE when ratio == 0, (k + 1)*ratio >
 * vis_stride (the longest list must fit) or the mask rows are too narrow;
 * Q8_ERR_UNSUPPORTED when score_stride > 16384.  num_rows == 0 enqueues
 * nothing.
 */
q8_status q8_index_select(const float* scores, uint32_t score_stride, const uint32_t* row_lens,
                          uint32_t num_rows, uint32_t ratio, uint32_t k, uint32_t* visible_pos,
                          uint32_t vis_stride, uint32_t* num_visible, uint32_t* visible_mask,
                          uint32_t mask_stride, void* stream);

/* hipError_t code behind the calling thread's last Q8_ERR_HIP (0 if none). */
int q8_last_hip_error(void);

/*
 * Content checks (libq8kv_debug.so, the library built with Q8_DEBUG_BOUNDS).
 * The release library trusts the contents of the device arrays as the
 * pages' shaders do; the debug build also checks them on the device and
 * records every failed check as a bit of a flag word per GPU, while still
 * computing as the release build does (reads clamped into the cache, writes
 * past it skipped):
 *   Q8_BOUNDS_SLOT     q8_cache_write: a slot past num_blocks*block_size that
 *                      is not Q8_PAD_SLOT (nothing is written for it)
 *   Q8_BOUNDS_BLOCK    decode / decode step: a block id at or past num_blocks
 *                      for an attended position or the appended row
 *   Q8_BOUNDS_TABLE    decode: positions of a sequence past its block-table
 *                      row (context_lens beyond max_num_blocks_per_seq*block_size,
 *                      or a visible position whose block is past the row)
 *   Q8_BOUNDS_VISIBLE  visible lists: num_visible past vis_stride, or listed
 *                      positions of a chunk not ascending and distinct
 * q8_bounds_flags -- wait for the device (hipDeviceSynchronize), store the
 * current device's flag word in *flags and, when clear != 0, reset it.  In the
 * release library it stores 0 and returns Q8_ERR_UNSUPPORTED.  Q8_ERR_NULL for
 * a NULL flags pointer; Q8_ERR_HIP when the device calls fail.
 */
#define Q8_BOUNDS_SLOT 1u
#define Q8_BOUNDS_BLOCK 2u
#define Q8_BOUNDS_TABLE 4u
#define Q8_BOUNDS_VISIBLE 8u
q8_status q8_bounds_flags(uint32_t* flags, int clear);

/* Static, human-readable name of a status code. */
const char* q8_status_string(q8_status status);

#ifdef __cplusplus
}
#endif

#endif /* Q8KV_H */
