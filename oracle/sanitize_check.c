/*
 * Memory- and UB-checking driver for the oracle (test infrastructure only).
 *
 * Built by tests/test_oracle_sanitize.py with gcc -fsanitize=address,undefined
 * and run on the host: every oracle entry point is called on small inputs in
 * exactly sized heap buffers (so any read or write past a buffer hits an ASan
 * redzone), on edge shapes -- head size 4 and 12, block size 1 and 5, empty
 * sequences, pad slots, a context clamp, visible lists, zero vectors, tails of
 * the block selection and its bitmask.  It prints "ok" when every call
 * returned success; a sanitizer report aborts the run.
 */
#include "q8_oracle.c"

#include <stdio.h>

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) { rng_state = rng_state * 1664525u + 1013904223u; return rng_state >> 8; }
static float rndf(void) { return (float)rnd() / (float)(1u << 24) * 4.0f - 2.0f; }

static void* xalloc(size_t n) { void* p = malloc(n ? n : 1); if (!p) { fputs("oom\n", stderr); exit(2); } return p; }
static float* frand(size_t n) { float* p = xalloc(n * sizeof(float)); for (size_t i = 0; i < n; ++i) p[i] = rndf(); return p; }

#define CHECK(call) do { int rc_ = (call); if (rc_ != Q8O_OK) { fprintf(stderr, "%s -> %d\n", #call, rc_); return 1; } } while (0)

static int quant_cases(void)
{
    const uint32_t sizes[] = {4, 12, 256};
    for (int i = 0; i < 3; ++i) {
        const uint32_t hs = sizes[i];
        float* x = frand(hs);
        uint32_t* row = xalloc((hs / 4 + 1) * sizeof(uint32_t));
        double* back = xalloc(hs * sizeof(double));
        CHECK(q8o_quantize_row(x, hs, row));
        q8o_dequantize_row(row, hs, back);
        memset(x, 0, hs * sizeof(float));                   /* zero vector: scale 1.0 */
        CHECK(q8o_quantize_row(x, hs, row));
        free(x); free(row); free(back);
    }
    return 0;
}

/* int8, f32 and bf16 caches over the same random rows, decoded densely, clamped and through visible lists */
static int decode_cases(uint32_t bs)
{
    const uint32_t S = 3, H = 6, Hkv = 3, hs = 12, wpt = hs / 4 + 1;
    const uint32_t lens[3] = {0, 7, 15};
    const uint32_t max_nb = (15 + bs - 1) / bs;
    uint32_t nb = 0;
    for (uint32_t s = 0; s < S; ++s) nb += (lens[s] + bs - 1) / bs;
    uint32_t* bt = xalloc((size_t)S * max_nb * sizeof(uint32_t));
    for (uint32_t s = 0, at = 0; s < S; ++s)
        for (uint32_t j = 0; j < max_nb; ++j) bt[s * max_nb + j] = j < (lens[s] + bs - 1) / bs ? at++ : 0;
    const size_t words = (size_t)nb * Hkv * bs * wpt, floats = (size_t)nb * Hkv * bs * hs;
    uint32_t* kc = xalloc(words * 4); uint32_t* vc = xalloc(words * 4);
    float* kf = xalloc(floats * 4); float* vf = xalloc(floats * 4);
    uint16_t* kb = xalloc(floats * 2); uint16_t* vb = xalloc(floats * 2);
    memset(kc, 0, words * 4); memset(vc, 0, words * 4); memset(kf, 0, floats * 4); memset(vf, 0, floats * 4);
    memset(kb, 0, floats * 2); memset(vb, 0, floats * 2);
    for (uint32_t s = 0; s < S; ++s) {
        const uint32_t L = lens[s];
        if (!L) continue;
        float* k = frand((size_t)L * Hkv * hs); float* v = frand((size_t)L * Hkv * hs);
        uint32_t* slots = xalloc(L * sizeof(uint32_t));
        for (uint32_t p = 0; p < L; ++p) slots[p] = bt[s * max_nb + p / bs] * bs + p % bs;
        slots[L - 1] = L > 1 ? slots[L - 1] : slots[0];
        CHECK(q8o_cache_write(k, Hkv * hs, v, Hkv * hs, kc, vc, slots, L, Hkv, hs, bs, nb));
        CHECK(q8o_f32_cache_write(k, Hkv * hs, v, Hkv * hs, kf, vf, slots, L, Hkv, hs, bs, nb));
        CHECK(q8o_bf16_cache_write(k, Hkv * hs, v, Hkv * hs, kb, vb, slots, L, Hkv, hs, bs, nb));
        free(k); free(v); free(slots);
    }
    {   /* a pad token among the writes */
        float* k = frand(2 * Hkv * hs); float* v = frand(2 * Hkv * hs);
        uint32_t slots[2] = {Q8O_PAD_SLOT, 0};
        CHECK(q8o_cache_write(k, Hkv * hs, v, Hkv * hs, kc, vc, slots, 2, Hkv, hs, bs, nb));
        free(k); free(v);
    }
    float* q = frand((size_t)S * H * hs);
    float* out = xalloc((size_t)S * H * hs * 4);
    CHECK(q8o_paged_decode(out, q, H * hs, kc, vc, bt, max_nb, lens, 15, NULL, NULL, 0, S, H, Hkv, hs, bs, nb,
                           0.25f, 1));
    CHECK(q8o_paged_decode(out, q, H * hs, kc, vc, bt, max_nb, lens, 4, NULL, NULL, 0, S, H, Hkv, hs, bs, nb,
                           0.25f, 2));
    CHECK(q8o_f32_paged_decode(out, q, H * hs, kf, vf, bt, max_nb, lens, 15, S, H, Hkv, hs, bs, nb, 0.25f, 1));
    CHECK(q8o_bf16_paged_decode(out, q, H * hs, kb, vb, bt, max_nb, lens, 15, S, H, Hkv, hs, bs, nb, 0.25f, 2));
    {
        const uint32_t vs = 15;
        uint32_t* vis = xalloc((size_t)S * vs * sizeof(uint32_t));
        uint32_t nvis[3];
        for (uint32_t s = 0; s < S; ++s) {
            nvis[s] = 0;
            for (uint32_t p = 0; p < lens[s]; ++p)
                if (p % 3 != 1) vis[s * vs + nvis[s]++] = p;
        }
        CHECK(q8o_paged_decode(out, q, H * hs, kc, vc, bt, max_nb, lens, 0, vis, nvis, vs, S, H, Hkv, hs, bs, nb,
                               0.25f, 1));
        free(vis);
    }
    free(bt); free(kc); free(vc); free(kf); free(vf); free(kb); free(vb); free(q); free(out);
    return 0;
}

static int norm_rope_cases(void)
{
    const uint32_t P = 9, rot = 8, hs = 16, hstride = 20, rows = 2, heads = 3;
    float* table = xalloc((size_t)P * rot * 4);
    CHECK(q8o_rope_table(table, P, rot, 10000.0f));
    float* w = frand(hs);
    const uint32_t xs = (heads - 1) * hstride + hs;
    float* x = frand((size_t)rows * xs);
    float* out = xalloc((size_t)rows * heads * hs * 4);
    uint32_t pos[2] = {0, 8};
    CHECK(q8o_norm_rope(out, heads * hs, x, xs, hstride, rows, heads, hs, pos, w, table, rot, P, 1e-6f));
    CHECK(q8o_norm_rope(out, heads * hs, x, xs, hstride, rows, heads, hs, NULL, w, NULL, 0, 0, 1e-6f));
    {
        const uint32_t T = 4, Hkv = 2, bs = 1, nb = 5, wpt = hs / 4 + 1;
        float* k = frand((size_t)T * Hkv * hs); float* v = frand((size_t)T * Hkv * hs);
        uint32_t* kc = xalloc((size_t)nb * Hkv * bs * wpt * 4); uint32_t* vc = xalloc((size_t)nb * Hkv * bs * wpt * 4);
        uint32_t slots[4] = {4, Q8O_PAD_SLOT, 0, 2}, tpos[4] = {3, 0xFFFFFFFFu, 8, 0};
        CHECK(q8o_norm_rope_cache_write(k, Hkv * hs, v, Hkv * hs, kc, vc, slots, tpos, w, table, rot, P, 1e-6f, T,
                                        Hkv, hs, bs, nb));
        CHECK(q8o_norm_rope_cache_write(k, Hkv * hs, v, Hkv * hs, kc, vc, slots, NULL, w, NULL, 0, 0, 1e-6f, T,
                                        Hkv, hs, bs, nb));          /* no rotation: positions and table unread */
        free(k); free(v); free(kc); free(vc);
    }
    free(table); free(w); free(x); free(out);
    return 0;
}

static int select_cases(void)
{
    const uint32_t R = 4, blocks = 5, ratio = 4, k = 2, vs = (k + 1) * ratio, ms = 1;
    float* sc = xalloc((size_t)R * blocks * 4);
    for (uint32_t i = 0; i < R * blocks; ++i) sc[i] = (float)(rnd() % 3);     /* ties */
    uint32_t lens[4] = {0, 7, 23, 20};
    uint32_t* vis = xalloc((size_t)R * vs * 4);
    uint32_t* nvis = xalloc(R * 4);
    uint32_t* mask = xalloc((size_t)R * ms * 4);
    CHECK(q8o_index_select(sc, blocks, lens, R, ratio, k, vis, vs, nvis, mask, ms));
    CHECK(q8o_index_select(sc, blocks, lens, R, ratio, 0, vis, vs, nvis, NULL, 0));
    free(sc); free(vis); free(nvis); free(mask);
    return 0;
}

int main(void)
{
    if (quant_cases() || decode_cases(5) || decode_cases(1) || norm_rope_cases() || select_cases()) return 1;
    puts("ok");
    return 0;
}
