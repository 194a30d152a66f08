"""Pins for the oracle's f32-cache baseline (CPU only).

The decode page's header says the int8 decode keeps the math of the f32 decode
(softmax(scale * q.K^T) . V over the sequence's first context_len tokens, kv
head h / (num_heads / num_kv_heads), token t at block_tables[s][t / block_size],
offset t % block_size) and differs only in the 4-byte f32 cache elements it
replaces; the writer page says pad slots are skipped as in the f32 writer.  The
f32 layout [num_blocks, num_kv_heads, block_size, head_size] is the reading of
the quantized layout with one f32 per element.

Pins: the writer against numpy indexing of that 4-D layout, the decode against
brute-force f64 attention over the original rows, closed forms (one token,
identical keys), and bit-equality with the int8 decode on rows the quantizer
represents exactly.
"""
import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl
from test_oracle_decode import lossless, softmax_attend


class F32Case:
    """Random f32 paged caches filled through the oracle's f32 writer."""

    def __init__(self, oracle_mod, seed, S, H, Hkv, hs, bs, lens, exact=False, spare_blocks=3):
        g = np.random.default_rng(seed)
        self.S, self.H, self.Hkv, self.hs, self.bs = S, H, Hkv, hs, bs
        self.lens = np.asarray(lens, dtype=np.uint32)
        nbs = [-(-int(L) // bs) for L in self.lens]
        self.max_nb = max(nbs + [1]) + 1
        self.num_blocks = sum(nbs) + spare_blocks
        perm = g.permutation(self.num_blocks).astype(np.uint32)
        self.bt = np.full((S, self.max_nb), self.num_blocks, dtype=np.uint32)   # poison block
        at = 0
        for s, nb in enumerate(nbs):
            self.bt[s, :nb] = perm[at:at + nb]
            at += nb
        self.kc = wl.poison_cache_f32(self.num_blocks + 1, Hkv, bs, hs)
        self.vc = wl.poison_cache_f32(self.num_blocks + 1, Hkv, bs, hs)
        self.K, self.V, self.slots = [], [], []
        for s in range(S):
            L = int(self.lens[s])
            if exact:
                K, V = lossless(g, (L, Hkv, hs)), lossless(g, (L, Hkv, hs))
            else:
                K = g.standard_normal((L, Hkv, hs)).astype(np.float32)
                V = g.standard_normal((L, Hkv, hs)).astype(np.float32)
            pos = np.arange(L)
            slots = (self.bt[s, pos // bs].astype(np.int64) * bs + pos % bs).astype(np.uint32)
            self.K.append(K)
            self.V.append(V)
            self.slots.append(slots)
            if L:
                oracle_mod.f32_cache_write(K, V, self.kc, self.vc, slots, Hkv, hs, bs)
        self.q = g.standard_normal((S, H, hs)).astype(np.float32)
        self.scale = float(np.float32(1.0 / np.sqrt(hs)))

    def decode(self, oracle_mod, **kw):
        return oracle_mod.f32_paged_decode(self.q, self.kc, self.vc, self.bt, self.lens, self.scale,
                                           self.Hkv, self.bs, **kw)

    def reference(self, max_context_len=None):
        n_rep = self.H // self.Hkv
        out = np.zeros((self.S, self.H, self.hs))
        for s in range(self.S):
            L = int(self.lens[s]) if max_context_len is None else min(int(self.lens[s]), max_context_len)
            for h in range(self.H):
                out[s, h] = softmax_attend(self.q[s, h], self.K[s][:L, h // n_rep], self.V[s][:L, h // n_rep],
                                           self.scale)
        return out


def test_writer_places_rows_by_layout(oracle_mod):
    g = np.random.default_rng(5)
    Hkv, hs, bs, nb = 3, 20, 7, 9
    T = 40
    slots = g.permutation(nb * bs)[:T].astype(np.uint32)
    slots[[3, 17, 30]] = wl.PAD_SLOT
    K = g.standard_normal((T, Hkv * hs + 5)).astype(np.float32)     # padded row stride
    V = g.standard_normal((T, Hkv * hs + 5)).astype(np.float32)
    kc = wl.poison_cache_f32(nb, Hkv, bs, hs)
    vc = wl.poison_cache_f32(nb, Hkv, bs, hs)
    oracle_mod.f32_cache_write(K, V, kc, vc, slots, Hkv, hs, bs, key_stride=Hkv * hs + 5,
                               value_stride=Hkv * hs + 5)
    written = np.zeros((nb, Hkv, bs), dtype=bool)
    for t in range(T):
        if slots[t] == wl.PAD_SLOT:
            continue
        b, o = divmod(int(slots[t]), bs)
        for h in range(Hkv):
            assert np.array_equal(kc[b, h, o], K[t, h * hs:(h + 1) * hs])
            assert np.array_equal(vc[b, h, o], V[t, h * hs:(h + 1) * hs])
            written[b, :, o] = True
    # every row no token was written to is still poison
    assert np.all(np.isnan(kc[~written])) and np.all(np.isnan(vc[~written]))


def test_writer_rejects_slot_out_of_range(oracle_mod):
    kc = wl.poison_cache_f32(2, 1, 4, 8)
    vc = wl.poison_cache_f32(2, 1, 4, 8)
    x = np.ones((1, 8), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle_mod.f32_cache_write(x, x, kc, vc, np.array([8], dtype=np.uint32), 1, 8, 4)


@pytest.mark.parametrize("S,H,Hkv,hs,bs,lens", [
    (2, 4, 2, 64, 16, [37, 64]),
    (3, 8, 2, 32, 4, [1, 19, 50]),
    (2, 6, 3, 128, 32, [70, 33]),
    (2, 2, 2, 256, 16, [17, 3]),
    (3, 8, 1, 16, 1, [5, 0, 9]),
])
def test_decode_matches_bruteforce(oracle_mod, S, H, Hkv, hs, bs, lens):
    c = F32Case(oracle_mod, 11, S, H, Hkv, hs, bs, lens)
    got = c.decode(oracle_mod)
    ref = c.reference()
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)


def test_context_clamp(oracle_mod):
    c = F32Case(oracle_mod, 12, 3, 4, 2, 64, 16, [40, 9, 70])
    got = c.decode(oracle_mod, max_context_len=20)
    ref = c.reference(max_context_len=20)
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)
    assert np.all(c.decode(oracle_mod, max_context_len=0) == 0)


def test_one_token_returns_v_row(oracle_mod):
    c = F32Case(oracle_mod, 13, 3, 4, 2, 64, 16, [1, 1, 1])
    got = c.decode(oracle_mod)
    for s in range(c.S):
        for h in range(c.H):
            assert np.array_equal(got[s, h], c.V[s][0, h // 2])


def test_identical_keys_give_mean_of_values(oracle_mod):
    c = F32Case(oracle_mod, 14, 2, 4, 2, 64, 8, [23, 40])
    for s in range(c.S):
        c.K[s][:] = c.K[s][0]
        oracle_mod.f32_cache_write(c.K[s], c.V[s], c.kc, c.vc, c.slots[s], c.Hkv, c.hs, c.bs)
    got = c.decode(oracle_mod)
    for s in range(c.S):
        for h in range(c.H):
            want = c.V[s][:, h // 2].astype(np.float64).mean(axis=0)
            assert np.all(np.abs(got[s, h] - want) <= 2.0 ** -22 * np.abs(want) + 1e-12)


def test_equals_int8_decode_on_exactly_quantized_rows(oracle_mod):
    """Rows c*2^j with max |c| = 127 are stored by the int8 writer without loss,
    so both decodes see the same binary64 values and agree bit for bit."""
    S, H, Hkv, hs, bs, lens = 3, 8, 2, 64, 16, [45, 1, 100]
    c = F32Case(oracle_mod, 15, S, H, Hkv, hs, bs, lens, exact=True)
    kq = wl.poison_cache(c.num_blocks + 1, Hkv, bs, hs)
    vq = wl.poison_cache(c.num_blocks + 1, Hkv, bs, hs)
    for s in range(S):
        if lens[s]:
            oracle_mod.cache_write(c.K[s], c.V[s], kq, vq, c.slots[s], Hkv, hs, bs)
    got_f32 = c.decode(oracle_mod)
    got_q8 = oracle_mod.paged_decode(c.q, kq, vq, c.bt, c.lens, c.scale, Hkv, bs)
    assert np.array_equal(got_f32, got_q8)


def test_units_match_full_decode(oracle_mod):
    c = F32Case(oracle_mod, 16, 3, 4, 2, 32, 8, [30, 0, 17])
    full = c.decode(oracle_mod)
    units = [(2, 3), (0, 0), (1, 2), (0, 3)]
    got = oracle_mod.f32_paged_decode_units(units, c.q, c.kc, c.vc, c.bt, c.lens, c.scale, c.Hkv, c.bs)
    for i, (s, h) in enumerate(units):
        assert np.array_equal(got[i], full[s, h])


def test_reads_no_unwritten_row(oracle_mod):
    """Every unwritten row is NaN, so a read past the context poisons the output."""
    c = F32Case(oracle_mod, 17, 2, 4, 4, 32, 16, [17, 31])
    assert np.all(np.isfinite(c.decode(oracle_mod)))
