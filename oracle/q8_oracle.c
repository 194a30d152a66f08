/*
 * q8_oracle.c -- plain, slow CPU oracle for the int8 paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  The HIP library never calls it, and the
 * two share no code, headers, tables or helpers.
 *
 * What it computes, and the passage each part follows:
 *
 *   Cache format ("paged_attn_q8.comp" and "reshape_and_cache_q8.comp" pages,
 *   header comments on the quantized cache): a u32 buffer laid out
 *   [num_blocks, num_kv_heads, block_size, words_per_token] with
 *   words_per_token = head_size/4 + 1.  A token's vector for one kv head is
 *   head_size/4 code words, four int8 codes per word with element 4w+l in byte
 *   l (little-endian lane), followed by one word holding the f32 scale's bits.
 *
 *   Quantize + pack ("reshape_and_cache_q8.comp" page, main(), its KEY block
 *   and the VALUE block that repeats it for V).  Binary32,
 *   one IEEE operation per step, as the page's shader states them:
 *     amax = max_d |x_d| (starting from 0)
 *     inv  = amax > 0 ? 127/amax : 0
 *     code = clamp(round(x_d * inv), -127, 127), ties to even (the page leaves
 *            the tie rule to the implementation; ties go to even here)
 *     scale word = bits(amax > 0 ? amax/127 : 1.0)
 *   A slot equal to 0xFFFFFFFF is a pad: nothing is read or written.
 *
 *   Decode ("paged_attn_q8.comp" page, main(): output = softmax(scale*Q.K^T).V
 *   with K and V dequantized on read as code * token_scale).  This oracle writes
 *   out the plain definition in binary64, not the page's three-pass structure:
 *     L     = min(context_lens[s], max_context_len)   (or a visible list)
 *     kvh   = h / (num_heads / num_kv_heads)
 *     k_hat = code * kscale, v_hat = code * vscale    (exact in binary64)
 *     z_t   = scale * sum_d q_d * k_hat_{t,d}
 *     o_d   = sum_t exp(z_t - max z) v_hat_{t,d} / sum_t exp(z_t - max z)
 *   rounded once to f32.  An empty position set gives a zero row (the page's
 *   1/(exp_sum + 1e-6) with exp_sum = 0 multiplies a zero accumulator).  For a
 *   non-empty set the page's 1e-6 is dropped: exp_sum >= 1 there, so it moves
 *   the result by at most 1e-6 relative, below the parity tolerance.
 *
 *   Visible-list decode (the "attention.rs" page, the selective branch of the
 *   per-row split decode that binds the row's visible token list): the row
 *   attends exactly the listed logical positions; context_lens is unused.
 *
 *   f32 cache baseline (the "paged_attn_q8.comp" page's header: the int8 decode
 *   keeps the math and structure of the f32 decode, whose cache holds 4 bytes
 *   per element; the "reshape_and_cache_q8.comp" page's header: pad slots are
 *   skipped as in the f32 writer).  The pages do not print the f32 layout; it
 *   is read as the quantized layout with each token vector stored as head_size
 *   f32 values: [num_blocks, num_kv_heads, block_size, head_size] f32.  The
 *   writer copies rows; the decode is the definition above with
 *   k_hat, v_hat the stored f32 values (exact in binary64).
 *
 *   bf16 cache baseline (not on the pages: the half-width cache most serving
 *   stacks keep, measured beside the f32 one).  The same layout with each
 *   element stored as bfloat16, the upper half of a binary32 encoding: the
 *   writer rounds each f32 input to the nearest bfloat16 value, ties to the
 *   one with an even last significand bit (IEEE 754 round-to-nearest-even at
 *   8 significand bits); the decode is the definition above with k_hat, v_hat
 *   the stored bfloat16 values (exact in binary64).
 *
 *   Norm + rotary step ahead of the cache write (the "attention.rs" page: the
 *   q/k norm-and-rope dispatches before the q8 append, with a learned per-head
 *   norm weight, rot = head_dim * partial_rotary_factor rotated elements, the
 *   model's rope theta and rms eps, and row b at position base_pos + b).  The
 *   page does not print the kernel body; the reading taken is the usual
 *   per-head RMSNorm followed by a rotate-half rotary embedding of the first
 *   rot elements:
 *     r     = 1 / sqrt(mean_d x_d^2 + eps)
 *     n_d   = x_d * r * w_d
 *     for i < rot/2, with a = n_i, b = n_{i+rot/2}, phi = pos * theta^(-2i/rot):
 *       y_i = a cos(phi) - b sin(phi),   y_{i+rot/2} = b cos(phi) + a sin(phi)
 *     y_d = n_d for d >= rot.
 *   The result feeds the quantizer, whose codes are decided in binary32, so
 *   the rounding points are fixed: mean_d x_d^2 + eps, the square root and the
 *   reciprocal in binary64, r rounded to binary32; x*r and then *w, each one
 *   binary32 product; cos and sin in binary64, rounded to binary32 (a table
 *   per position); each rotated element as binary32 products and one binary32
 *   sum.  q8o_norm_rope_row_f64 is the same definition in binary64 throughout
 *   (angles straight from theta), the reference the pins check against.
 *
 *   Block selection into a visible list (the "attention.rs" page: each row b
 *   of a step has t_len = base_pos + b + 1 positions and blocks = t_len /
 *   ratio complete blocks; with kblk = budget / ratio, a row is selective when
 *   blocks > kblk and then attends kblk*ratio + (t_len - blocks*ratio)
 *   positions, else all t_len; the indexer's select pass turns block scores
 *   into that list, vis_stride = budget + ratio apart).  The select kernel is
 *   not printed; the reading taken: the kblk complete blocks of highest score
 *   (ties to the lower block index), their positions in ascending order, then
 *   the trailing incomplete block's positions.  When blocks <= kblk every
 *   complete block is taken, which is the dense list 0 .. t_len-1.  The pass
 *   also emits a per-row bitmask of ceil(max_blocks/32) words (max_blocks =
 *   max_t/ratio + 1, so the trailing block has a bit); its meaning is not
 *   printed either: bit j (word j/32, bit j%32) is set exactly when the list
 *   holds a position of block j.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fopenmp -fPIC
 * -shared.  On x86-64 (SSE, FLT_EVAL_METHOD == 0) every float operation above
 * rounds to binary32 once.  OpenMP only spreads independent (seq, head) units
 * over threads; each unit's arithmetic is sequential, so the result does not
 * depend on the thread count.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define Q8O_PAD_SLOT 0xFFFFFFFFu

enum {
    Q8O_OK = 0,
    Q8O_ERR_SHAPE = 1,   /* head_size not a positive multiple of 4, etc. */
    Q8O_ERR_RANGE = 2,   /* an index read from an input array is out of range */
    Q8O_ERR_INPUT = 3,   /* non-finite input, or 0 < amax < 2^-100 (outside the contract) */
    Q8O_ERR_NOMEM = 4
};

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* A bfloat16 value read as binary32 (its 16 bits are the upper half). */
float q8o_bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

/*
 * The bfloat16 nearest to finite x, ties to even: bfloat16 keeps a binary32
 * value's sign, exponent and top 7 fraction bits, so the candidates are the
 * truncation t (x's upper 16 bits) and the next value away from zero, t + 1.
 * The dropped 16 bits r decide: below half an ulp (0x8000) keep t, above it
 * take t + 1, exactly half keep whichever of the two has an even last bit.
 * (t + 1 past the largest finite magnitude is infinity, as rounding gives.)
 */
uint16_t q8o_f32_to_bf16(float x)
{
    const uint32_t u = f32_to_bits(x);
    const uint32_t t = u >> 16, r = u & 0xFFFFu;
    if (r < 0x8000u) return (uint16_t)t;
    if (r > 0x8000u) return (uint16_t)(t + 1u);
    return (uint16_t)((t & 1u) ? t + 1u : t);
}

/* One token vector x[0..head_size) -> head_size/4 code words + 1 scale word. */
int q8o_quantize_row(const float* x, uint32_t head_size, uint32_t* row)
{
    if (head_size == 0 || head_size % 4 != 0) return Q8O_ERR_SHAPE;
    float amax = 0.0f;
    for (uint32_t d = 0; d < head_size; ++d) {
        if (!isfinite(x[d])) return Q8O_ERR_INPUT;
        float a = fabsf(x[d]);
        if (a > amax) amax = a;
    }
    if (amax > 0.0f && amax < 0x1p-100f) return Q8O_ERR_INPUT;
    float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    for (uint32_t w = 0; w < head_size / 4; ++w) {
        uint32_t word = 0;
        for (uint32_t l = 0; l < 4; ++l) {
            float p = x[4 * w + l] * inv;      /* one f32 multiply */
            float r = nearbyintf(p);           /* default mode: nearest, ties to even */
            if (r < -127.0f) r = -127.0f;
            if (r > 127.0f) r = 127.0f;
            int8_t c = (int8_t)(int)r;
            word |= (uint32_t)(uint8_t)c << (8u * l);
        }
        row[w] = word;
    }
    row[head_size / 4] = f32_to_bits(amax > 0.0f ? amax / 127.0f : 1.0f);
    return Q8O_OK;
}

/* Signed code of element d of a packed row: byte d%4 of word d/4, sign-extended. */
static int code_at(const uint32_t* row, uint32_t d)
{
    uint32_t byte = (row[d / 4] >> (8u * (d % 4))) & 0xFFu;
    return (int)(int8_t)(uint8_t)byte;
}

/* Dequantize a packed row to binary64: out[d] = code_d * scale (exact). */
void q8o_dequantize_row(const uint32_t* row, uint32_t head_size, double* out)
{
    double scale = (double)bits_to_f32(row[head_size / 4]);
    for (uint32_t d = 0; d < head_size; ++d) out[d] = (double)code_at(row, d) * scale;
}

/* Word offset of (slot, kv head) in a cache laid out [blocks, kv heads, block_size, wpt]. */
static uint64_t row_offset(uint64_t block, uint64_t off, uint64_t kvh,
                           uint64_t num_kv_heads, uint64_t block_size, uint64_t wpt)
{
    return ((block * num_kv_heads + kvh) * block_size + off) * wpt;
}

int q8o_cache_write(const float* key, uint32_t key_stride,
                    const float* value, uint32_t value_stride,
                    uint32_t* key_cache, uint32_t* value_cache,
                    const uint32_t* slot_mapping, uint32_t num_tokens,
                    uint32_t num_kv_heads, uint32_t head_size,
                    uint32_t block_size, uint32_t num_blocks)
{
    if (head_size == 0 || head_size % 4 != 0 || block_size == 0 || num_kv_heads == 0)
        return Q8O_ERR_SHAPE;
    if ((uint64_t)key_stride < (uint64_t)num_kv_heads * head_size ||
        (uint64_t)value_stride < (uint64_t)num_kv_heads * head_size)
        return Q8O_ERR_SHAPE;
    uint32_t wpt = head_size / 4 + 1;
    for (uint32_t t = 0; t < num_tokens; ++t) {
        uint32_t slot = slot_mapping[t];
        if (slot == Q8O_PAD_SLOT) continue;
        uint64_t block = slot / block_size, off = slot % block_size;
        if (block >= num_blocks) return Q8O_ERR_RANGE;
        for (uint32_t h = 0; h < num_kv_heads; ++h) {
            uint64_t dst = row_offset(block, off, h, num_kv_heads, block_size, wpt);
            int rc = q8o_quantize_row(key + (uint64_t)t * key_stride + (uint64_t)h * head_size,
                                      head_size, key_cache + dst);
            if (rc != Q8O_OK) return rc;
            rc = q8o_quantize_row(value + (uint64_t)t * value_stride + (uint64_t)h * head_size,
                                  head_size, value_cache + dst);
            if (rc != Q8O_OK) return rc;
        }
    }
    return Q8O_OK;
}

typedef struct {
    const float* q; uint32_t q_stride;
    const uint32_t* key_cache; const uint32_t* value_cache;
    const float* key_cache_f32; const float* value_cache_f32;   /* f32 baseline when non-NULL */
    const uint16_t* key_cache_bf16; const uint16_t* value_cache_bf16;   /* bf16 baseline when non-NULL */
    const uint32_t* block_tables; uint32_t max_num_blocks_per_seq;
    const uint32_t* context_lens; uint32_t max_context_len;
    const uint32_t* visible_pos; const uint32_t* num_visible; uint32_t vis_stride;
    uint32_t num_seqs, num_heads, num_kv_heads, head_size, block_size, num_blocks;
    double scale;
} decode_args;

/* The K (or V) vector of kv head kvh at (physical block, offset), in binary64. */
static void load_row(const decode_args* a, int value, uint32_t phys, uint32_t off, uint32_t kvh,
                     double* out)
{
    const uint32_t hs = a->head_size;
    if (a->key_cache_f32) {
        const float* c = value ? a->value_cache_f32 : a->key_cache_f32;
        const float* row = c + (((uint64_t)phys * a->num_kv_heads + kvh) * a->block_size + off) * hs;
        for (uint32_t d = 0; d < hs; ++d) out[d] = (double)row[d];
    } else if (a->key_cache_bf16) {
        const uint16_t* c = value ? a->value_cache_bf16 : a->key_cache_bf16;
        const uint16_t* row = c + (((uint64_t)phys * a->num_kv_heads + kvh) * a->block_size + off) * hs;
        for (uint32_t d = 0; d < hs; ++d) out[d] = (double)q8o_bf16_to_f32(row[d]);
    } else {
        const uint32_t* c = value ? a->value_cache : a->key_cache;
        q8o_dequantize_row(c + row_offset(phys, off, kvh, a->num_kv_heads, a->block_size, hs / 4 + 1),
                           hs, out);
    }
}

/*
 * One (seq, head) unit.  out_row gets head_size floats; work holds 2*head_size
 * doubles plus one double per attended position.
 */
static int decode_unit(const decode_args* a, uint32_t s, uint32_t h, float* out_row)
{
    const uint32_t hs = a->head_size;
    const uint32_t kvh = h / (a->num_heads / a->num_kv_heads);
    uint32_t n;
    const uint32_t* pos = NULL;
    if (a->visible_pos) {
        n = a->num_visible[s];
        if (n > a->vis_stride) return Q8O_ERR_RANGE;
        pos = a->visible_pos + (uint64_t)s * a->vis_stride;
    } else {
        n = a->context_lens[s];
        if (n > a->max_context_len) n = a->max_context_len;
    }
    if (n == 0) {
        for (uint32_t d = 0; d < hs; ++d) out_row[d] = 0.0f;
        return Q8O_OK;
    }
    double* z = (double*)malloc(sizeof(double) * ((size_t)n + 2u * hs));
    if (!z) return Q8O_ERR_NOMEM;
    double* k_hat = z + n;
    double* o = k_hat + hs;
    const float* qv = a->q + (uint64_t)s * a->q_stride + (uint64_t)h * hs;
    const uint32_t* bt = a->block_tables + (uint64_t)s * a->max_num_blocks_per_seq;

    /* pass over positions: logits z_t = scale * <q, k_hat_t> */
    double zmax = -INFINITY;
    for (uint32_t i = 0; i < n; ++i) {
        uint32_t t = pos ? pos[i] : i;
        uint32_t j = t / a->block_size;
        if (j >= a->max_num_blocks_per_seq) { free(z); return Q8O_ERR_RANGE; }
        uint32_t phys = bt[j];
        if (phys >= a->num_blocks) { free(z); return Q8O_ERR_RANGE; }
        load_row(a, 0, phys, t % a->block_size, kvh, k_hat);
        double dot = 0.0;
        for (uint32_t d = 0; d < hs; ++d) dot += (double)qv[d] * k_hat[d];
        z[i] = a->scale * dot;
        if (!(z[i] > -INFINITY && z[i] < INFINITY)) { free(z); return Q8O_ERR_INPUT; }
        if (z[i] > zmax) zmax = z[i];
    }
    /* weights and weighted sum of dequantized V */
    double denom = 0.0;
    for (uint32_t d = 0; d < hs; ++d) o[d] = 0.0;
    for (uint32_t i = 0; i < n; ++i) {
        uint32_t t = pos ? pos[i] : i;
        uint32_t phys = bt[t / a->block_size];
        double w = exp(z[i] - zmax);
        denom += w;
        load_row(a, 1, phys, t % a->block_size, kvh, k_hat);     /* reuse buffer for v_hat */
        for (uint32_t d = 0; d < hs; ++d) o[d] += w * k_hat[d];
    }
    for (uint32_t d = 0; d < hs; ++d) out_row[d] = (float)(o[d] / denom);
    free(z);
    return Q8O_OK;
}

static int check_decode_shape(const decode_args* a)
{
    if (a->head_size == 0 || a->head_size % 4 != 0 || a->block_size == 0 ||
        a->num_kv_heads == 0 || a->num_heads == 0 || a->num_heads % a->num_kv_heads != 0)
        return Q8O_ERR_SHAPE;
    if ((uint64_t)a->q_stride < (uint64_t)a->num_heads * a->head_size) return Q8O_ERR_SHAPE;
    return Q8O_OK;
}

static int run_units(const decode_args* a, float* out, const uint32_t* units, uint32_t num_units,
                     int nthreads)
{
    int rc = check_decode_shape(a);
    if (rc != Q8O_OK) return rc;
    for (uint32_t i = 0; i < num_units; ++i)
        if (units[2 * i] >= a->num_seqs || units[2 * i + 1] >= a->num_heads) return Q8O_ERR_RANGE;
    int err = Q8O_OK;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < (int64_t)num_units; ++i) {
        int r = decode_unit(a, units[2 * i], units[2 * i + 1], out + (uint64_t)i * a->head_size);
        if (r != Q8O_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
            err = r;
        }
    }
    (void)nthreads;
    return err;
}

/* Every (seq, head) of the batch as a unit list, in row-major output order. */
static uint32_t* all_units(uint32_t num_seqs, uint32_t num_heads, uint64_t* nu)
{
    *nu = (uint64_t)num_seqs * num_heads;
    uint32_t* units = (uint32_t*)malloc(sizeof(uint32_t) * 2 * (*nu ? *nu : 1));
    if (!units) return NULL;
    for (uint64_t i = 0; i < *nu; ++i) {
        units[2 * i] = (uint32_t)(i / num_heads);
        units[2 * i + 1] = (uint32_t)(i % num_heads);
    }
    return units;
}

/*
 * Decode selected (seq, head) units: units[2*i] = seq, units[2*i+1] = head;
 * out receives head_size floats per unit, in unit order.  visible_pos == NULL
 * selects dense mode.  nthreads <= 0 uses the OpenMP default.
 */
int q8o_paged_decode_units(float* out, const uint32_t* units, uint32_t num_units,
                           const float* q, uint32_t q_stride,
                           const uint32_t* key_cache, const uint32_t* value_cache,
                           const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                           const uint32_t* context_lens, uint32_t max_context_len,
                           const uint32_t* visible_pos, const uint32_t* num_visible,
                           uint32_t vis_stride,
                           uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                           uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                           float scale, int nthreads)
{
    decode_args a = { q, q_stride, key_cache, value_cache, NULL, NULL, NULL, NULL, block_tables,
                      max_num_blocks_per_seq, context_lens, max_context_len,
                      visible_pos, num_visible, vis_stride, num_seqs, num_heads,
                      num_kv_heads, head_size, block_size, num_blocks, (double)scale };
    return run_units(&a, out, units, num_units, nthreads);
}

/* Decode every (seq, head): out is [num_seqs, num_heads, head_size] dense f32. */
int q8o_paged_decode(float* out, const float* q, uint32_t q_stride,
                     const uint32_t* key_cache, const uint32_t* value_cache,
                     const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                     const uint32_t* context_lens, uint32_t max_context_len,
                     const uint32_t* visible_pos, const uint32_t* num_visible,
                     uint32_t vis_stride,
                     uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                     uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                     float scale, int nthreads)
{
    uint64_t nu;
    uint32_t* units = all_units(num_seqs, num_heads, &nu);
    if (!units) return Q8O_ERR_NOMEM;
    int rc = q8o_paged_decode_units(out, units, (uint32_t)nu, q, q_stride, key_cache,
                                    value_cache, block_tables, max_num_blocks_per_seq,
                                    context_lens, max_context_len, visible_pos,
                                    num_visible, vis_stride, num_seqs, num_heads,
                                    num_kv_heads, head_size, block_size, num_blocks,
                                    scale, nthreads);
    free(units);
    return rc;
}

/* f32 baseline writer: row t, kv head h is copied to its slot; pads are skipped. */
int q8o_f32_cache_write(const float* key, uint32_t key_stride,
                        const float* value, uint32_t value_stride,
                        float* key_cache, float* value_cache,
                        const uint32_t* slot_mapping, uint32_t num_tokens,
                        uint32_t num_kv_heads, uint32_t head_size,
                        uint32_t block_size, uint32_t num_blocks)
{
    if (head_size == 0 || block_size == 0 || num_kv_heads == 0) return Q8O_ERR_SHAPE;
    if ((uint64_t)key_stride < (uint64_t)num_kv_heads * head_size ||
        (uint64_t)value_stride < (uint64_t)num_kv_heads * head_size)
        return Q8O_ERR_SHAPE;
    for (uint32_t t = 0; t < num_tokens; ++t) {
        uint32_t slot = slot_mapping[t];
        if (slot == Q8O_PAD_SLOT) continue;
        uint64_t block = slot / block_size, off = slot % block_size;
        if (block >= num_blocks) return Q8O_ERR_RANGE;
        for (uint32_t h = 0; h < num_kv_heads; ++h) {
            uint64_t dst = ((block * num_kv_heads + h) * block_size + off) * head_size;
            memcpy(key_cache + dst, key + (uint64_t)t * key_stride + (uint64_t)h * head_size,
                   sizeof(float) * head_size);
            memcpy(value_cache + dst, value + (uint64_t)t * value_stride + (uint64_t)h * head_size,
                   sizeof(float) * head_size);
        }
    }
    return Q8O_OK;
}

/* f32 baseline decode of selected units (dense mode only); as q8o_paged_decode_units. */
int q8o_f32_paged_decode_units(float* out, const uint32_t* units, uint32_t num_units,
                               const float* q, uint32_t q_stride,
                               const float* key_cache, const float* value_cache,
                               const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                               const uint32_t* context_lens, uint32_t max_context_len,
                               uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                               uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                               float scale, int nthreads)
{
    if (!key_cache || !value_cache) return Q8O_ERR_SHAPE;
    decode_args a = { q, q_stride, NULL, NULL, key_cache, value_cache, NULL, NULL, block_tables,
                      max_num_blocks_per_seq, context_lens, max_context_len,
                      NULL, NULL, 0, num_seqs, num_heads,
                      num_kv_heads, head_size, block_size, num_blocks, (double)scale };
    return run_units(&a, out, units, num_units, nthreads);
}

/* f32 baseline decode of every (seq, head): out is [num_seqs, num_heads, head_size]. */
int q8o_f32_paged_decode(float* out, const float* q, uint32_t q_stride,
                         const float* key_cache, const float* value_cache,
                         const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                         const uint32_t* context_lens, uint32_t max_context_len,
                         uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                         uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                         float scale, int nthreads)
{
    uint64_t nu;
    uint32_t* units = all_units(num_seqs, num_heads, &nu);
    if (!units) return Q8O_ERR_NOMEM;
    int rc = q8o_f32_paged_decode_units(out, units, (uint32_t)nu, q, q_stride, key_cache,
                                        value_cache, block_tables, max_num_blocks_per_seq,
                                        context_lens, max_context_len, num_seqs, num_heads,
                                        num_kv_heads, head_size, block_size, num_blocks,
                                        scale, nthreads);
    free(units);
    return rc;
}

/* bf16 baseline writer: each element of row t, kv head h rounded to bfloat16
 * (q8o_f32_to_bf16) at its slot; pads are skipped. */
int q8o_bf16_cache_write(const float* key, uint32_t key_stride,
                         const float* value, uint32_t value_stride,
                         uint16_t* key_cache, uint16_t* value_cache,
                         const uint32_t* slot_mapping, uint32_t num_tokens,
                         uint32_t num_kv_heads, uint32_t head_size,
                         uint32_t block_size, uint32_t num_blocks)
{
    if (head_size == 0 || block_size == 0 || num_kv_heads == 0) return Q8O_ERR_SHAPE;
    if ((uint64_t)key_stride < (uint64_t)num_kv_heads * head_size ||
        (uint64_t)value_stride < (uint64_t)num_kv_heads * head_size)
        return Q8O_ERR_SHAPE;
    for (uint32_t t = 0; t < num_tokens; ++t) {
        uint32_t slot = slot_mapping[t];
        if (slot == Q8O_PAD_SLOT) continue;
        uint64_t block = slot / block_size, off = slot % block_size;
        if (block >= num_blocks) return Q8O_ERR_RANGE;
        for (uint32_t h = 0; h < num_kv_heads; ++h) {
            uint64_t dst = ((block * num_kv_heads + h) * block_size + off) * head_size;
            const float* k = key + (uint64_t)t * key_stride + (uint64_t)h * head_size;
            const float* v = value + (uint64_t)t * value_stride + (uint64_t)h * head_size;
            for (uint32_t d = 0; d < head_size; ++d) {
                key_cache[dst + d] = q8o_f32_to_bf16(k[d]);
                value_cache[dst + d] = q8o_f32_to_bf16(v[d]);
            }
        }
    }
    return Q8O_OK;
}

/* bf16 baseline decode of selected units (dense mode only); as q8o_paged_decode_units. */
int q8o_bf16_paged_decode_units(float* out, const uint32_t* units, uint32_t num_units,
                                const float* q, uint32_t q_stride,
                                const uint16_t* key_cache, const uint16_t* value_cache,
                                const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                                const uint32_t* context_lens, uint32_t max_context_len,
                                uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                                uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                                float scale, int nthreads)
{
    if (!key_cache || !value_cache) return Q8O_ERR_SHAPE;
    decode_args a = { q, q_stride, NULL, NULL, NULL, NULL, key_cache, value_cache, block_tables,
                      max_num_blocks_per_seq, context_lens, max_context_len,
                      NULL, NULL, 0, num_seqs, num_heads,
                      num_kv_heads, head_size, block_size, num_blocks, (double)scale };
    return run_units(&a, out, units, num_units, nthreads);
}

/* bf16 baseline decode of every (seq, head): out is [num_seqs, num_heads, head_size]. */
int q8o_bf16_paged_decode(float* out, const float* q, uint32_t q_stride,
                          const uint16_t* key_cache, const uint16_t* value_cache,
                          const uint32_t* block_tables, uint32_t max_num_blocks_per_seq,
                          const uint32_t* context_lens, uint32_t max_context_len,
                          uint32_t num_seqs, uint32_t num_heads, uint32_t num_kv_heads,
                          uint32_t head_size, uint32_t block_size, uint32_t num_blocks,
                          float scale, int nthreads)
{
    uint64_t nu;
    uint32_t* units = all_units(num_seqs, num_heads, &nu);
    if (!units) return Q8O_ERR_NOMEM;
    int rc = q8o_bf16_paged_decode_units(out, units, (uint32_t)nu, q, q_stride, key_cache,
                                         value_cache, block_tables, max_num_blocks_per_seq,
                                         context_lens, max_context_len, num_seqs, num_heads,
                                         num_kv_heads, head_size, block_size, num_blocks,
                                         scale, nthreads);
    free(units);
    return rc;
}

/* ---------------------------------------------------- norm + rotary ---- */

static int rope_shape_ok(uint32_t head_size, uint32_t rot)
{
    return head_size > 0 && head_size % 4 == 0 && rot % 2 == 0 && rot <= head_size;
}

/* Rotary table, one row of rot floats per position p < num_positions:
 * row[i] = cos(p * theta^(-2i/rot)), row[rot/2 + i] = sin(...), i < rot/2,
 * each evaluated in binary64 and rounded to binary32. */
int q8o_rope_table(float* table, uint32_t num_positions, uint32_t rot, float theta)
{
    if (rot % 2 != 0 || !(theta > 0.0f)) return Q8O_ERR_SHAPE;
    uint32_t half = rot / 2;
    for (uint32_t p = 0; p < num_positions; ++p)
        for (uint32_t i = 0; i < half; ++i) {
            double inv_freq = pow((double)theta, -(2.0 * i) / (double)rot);
            double phi = (double)p * inv_freq;
            table[(uint64_t)p * rot + i] = (float)cos(phi);
            table[(uint64_t)p * rot + half + i] = (float)sin(phi);
        }
    return Q8O_OK;
}

/* One head vector x[0..head_size) at the rounding points stated above; cs is
 * the rotary table row of the vector's position (unused when rot == 0). */
int q8o_norm_rope_row(const float* x, uint32_t head_size, const float* weight, const float* cs,
                      uint32_t rot, float eps, float* y)
{
    if (!rope_shape_ok(head_size, rot)) return Q8O_ERR_SHAPE;
    double ss = 0.0;
    for (uint32_t d = 0; d < head_size; ++d) {
        if (!isfinite(x[d])) return Q8O_ERR_INPUT;
        ss += (double)x[d] * (double)x[d];
    }
    float r = (float)(1.0 / sqrt(ss / (double)head_size + (double)eps));
    for (uint32_t d = 0; d < head_size; ++d) {
        float t = x[d] * r;
        y[d] = t * weight[d];
    }
    uint32_t half = rot / 2;
    for (uint32_t i = 0; i < half; ++i) {
        float a = y[i], b = y[i + half];
        float c = cs[i], sn = cs[half + i];
        float ac = a * c, bs = b * sn, bc = b * c, as = a * sn;
        y[i] = ac - bs;
        y[i + half] = bc + as;
    }
    return Q8O_OK;
}

/* The same definition in binary64, with the angle taken straight from theta. */
int q8o_norm_rope_row_f64(const float* x, uint32_t head_size, const float* weight, uint32_t pos,
                          uint32_t rot, double theta, double eps, double* y)
{
    if (!rope_shape_ok(head_size, rot)) return Q8O_ERR_SHAPE;
    double ss = 0.0;
    for (uint32_t d = 0; d < head_size; ++d) ss += (double)x[d] * (double)x[d];
    double r = 1.0 / sqrt(ss / (double)head_size + eps);
    for (uint32_t d = 0; d < head_size; ++d) y[d] = (double)x[d] * r * (double)weight[d];
    uint32_t half = rot / 2;
    for (uint32_t i = 0; i < half; ++i) {
        double phi = (double)pos * pow(theta, -(2.0 * i) / (double)rot);
        double a = y[i], b = y[i + half];
        y[i] = a * cos(phi) - b * sin(phi);
        y[i + half] = b * cos(phi) + a * sin(phi);
    }
    return Q8O_OK;
}

/* Rows of f32 head vectors: head h of row t at x[t*x_stride + h*head_stride],
 * written to out[t*out_stride + h*head_size]; row t at positions[t]. */
int q8o_norm_rope(float* out, uint32_t out_stride, const float* x, uint32_t x_stride, uint32_t head_stride,
                  uint32_t num_rows, uint32_t num_heads, uint32_t head_size, const uint32_t* positions,
                  const float* weight, const float* table, uint32_t rot, uint32_t num_positions, float eps)
{
    if (!rope_shape_ok(head_size, rot) || head_stride < head_size ||
        (uint64_t)out_stride < (uint64_t)num_heads * head_size)
        return Q8O_ERR_SHAPE;
    for (uint32_t t = 0; t < num_rows; ++t) {
        /* without rotation, positions and table may be NULL and are not read */
        uint32_t p = rot > 0 ? positions[t] : 0;
        if (rot > 0 && p >= num_positions) return Q8O_ERR_RANGE;
        const float* cs = rot > 0 ? table + (uint64_t)p * rot : NULL;
        for (uint32_t h = 0; h < num_heads; ++h) {
            int rc = q8o_norm_rope_row(x + (uint64_t)t * x_stride + (uint64_t)h * head_stride, head_size,
                                       weight, cs, rot, eps,
                                       out + (uint64_t)t * out_stride + (uint64_t)h * head_size);
            if (rc != Q8O_OK) return rc;
        }
    }
    return Q8O_OK;
}

/* Cache write with the norm + rotary step on K: for each non-pad token, each
 * kv head's K vector becomes q8o_norm_rope_row of it (at positions[t]) and is
 * then packed as q8o_cache_write packs it; V is packed unchanged. */
int q8o_norm_rope_cache_write(const float* key, uint32_t key_stride,
                              const float* value, uint32_t value_stride,
                              uint32_t* key_cache, uint32_t* value_cache,
                              const uint32_t* slot_mapping, const uint32_t* positions,
                              const float* weight, const float* table, uint32_t rot,
                              uint32_t num_positions, float eps, uint32_t num_tokens,
                              uint32_t num_kv_heads, uint32_t head_size,
                              uint32_t block_size, uint32_t num_blocks)
{
    if (head_size == 0 || head_size % 4 != 0 || block_size == 0 || num_kv_heads == 0 ||
        !rope_shape_ok(head_size, rot))
        return Q8O_ERR_SHAPE;
    if ((uint64_t)key_stride < (uint64_t)num_kv_heads * head_size ||
        (uint64_t)value_stride < (uint64_t)num_kv_heads * head_size)
        return Q8O_ERR_SHAPE;
    uint32_t wpt = head_size / 4 + 1;
    float* y = (float*)malloc(sizeof(float) * head_size);
    if (!y) return Q8O_ERR_NOMEM;
    int rc = Q8O_OK;
    for (uint32_t t = 0; t < num_tokens && rc == Q8O_OK; ++t) {
        uint32_t slot = slot_mapping[t];
        if (slot == Q8O_PAD_SLOT) continue;
        uint64_t block = slot / block_size, off = slot % block_size;
        uint32_t p = rot > 0 ? positions[t] : 0;    /* not read without rotation */
        if (block >= num_blocks || (rot > 0 && p >= num_positions)) { rc = Q8O_ERR_RANGE; break; }
        for (uint32_t h = 0; h < num_kv_heads && rc == Q8O_OK; ++h) {
            uint64_t dst = row_offset(block, off, h, num_kv_heads, block_size, wpt);
            rc = q8o_norm_rope_row(key + (uint64_t)t * key_stride + (uint64_t)h * head_size, head_size,
                                   weight, rot > 0 ? table + (uint64_t)p * rot : NULL, rot, eps, y);
            if (rc == Q8O_OK) rc = q8o_quantize_row(y, head_size, key_cache + dst);
            if (rc == Q8O_OK)
                rc = q8o_quantize_row(value + (uint64_t)t * value_stride + (uint64_t)h * head_size,
                                      head_size, value_cache + dst);
        }
    }
    free(y);
    return rc;
}

/* ------------------------------------------------------- block select ---- */

/* Row r: scores[r*score_stride + j] for its complete blocks j < row_lens[r] /
 * ratio.  Writes visible_pos[r*vis_stride + i], i < num_visible[r]. */
/* visible_mask may be NULL; otherwise mask_stride words per row, all written. */
int q8o_index_select(const float* scores, uint32_t score_stride, const uint32_t* row_lens,
                     uint32_t num_rows, uint32_t ratio, uint32_t k,
                     uint32_t* visible_pos, uint32_t vis_stride, uint32_t* num_visible,
                     uint32_t* visible_mask, uint32_t mask_stride)
{
    if (ratio == 0) return Q8O_ERR_SHAPE;
    if ((uint64_t)k * ratio + ratio > vis_stride) return Q8O_ERR_SHAPE;   /* the longest list must fit */
    for (uint32_t r = 0; r < num_rows; ++r) {
        uint32_t t_len = row_lens[r];
        uint32_t blocks = t_len / ratio;
        if (blocks > score_stride) return Q8O_ERR_RANGE;
        const float* sc = scores + (uint64_t)r * score_stride;
        for (uint32_t j = 0; j < blocks; ++j)
            if (!isfinite(sc[j])) return Q8O_ERR_INPUT;
        uint32_t n = 0;
        uint32_t* out = visible_pos + (uint64_t)r * vis_stride;
        /* block j is selected when fewer than k blocks come before it in the
         * order (score descending, index ascending) */
        for (uint32_t j = 0; j < blocks; ++j) {
            uint32_t ahead = 0;
            for (uint32_t i = 0; i < blocks && ahead < k; ++i)
                if (sc[i] > sc[j] || (sc[i] == sc[j] && i < j)) ++ahead;
            if (ahead < k)
                for (uint32_t p = 0; p < ratio; ++p) out[n++] = j * ratio + p;
        }
        for (uint32_t p = blocks * ratio; p < t_len; ++p) out[n++] = p;
        num_visible[r] = n;
        if (visible_mask) {
            uint32_t* m = visible_mask + (uint64_t)r * mask_stride;
            memset(m, 0, (size_t)mask_stride * sizeof(uint32_t));
            for (uint32_t e = 0; e < n; ++e) {
                uint32_t b = out[e] / ratio;
                if (b / 32 >= mask_stride) return Q8O_ERR_RANGE;   /* a touched block has no bit */
                m[b / 32] |= 1u << (b % 32);
            }
        }
    }
    return Q8O_OK;
}

int q8o_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
