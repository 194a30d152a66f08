"""Pins for the oracle's paged decode (CPU only).

The decode page defines the output as softmax(scale * q.K^T) . V over the
sequence's first context_len tokens, with K and V dequantized on read as
code * token_scale, the kv head of query head h being h / (num_heads /
num_kv_heads), and token t found at block_tables[s][t / block_size], offset
t % block_size.  These tests pin the oracle to that definition without using
its code: exact lossless inputs against brute-force f64 attention over the
original vectors, closed forms (one token, identical keys, constant values per
kv head), the unquantized error bound, and invariances (block relabeling,
GQA as duplicated MHA, visible lists, compaction, the context clamp).
"""
import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl


def softmax_attend(q, K, V, scale):
    """Brute-force f64 attention of one query over rows K, V (numpy only)."""
    if K.shape[0] == 0:
        return np.zeros(q.shape[0])
    z = scale * (K.astype(np.float64) @ q.astype(np.float64))
    w = np.exp(z - z.max())
    return (w @ V.astype(np.float64)) / w.sum()


def lossless(g, shape):
    """f32 vectors c*2^j (|c| <= 127, one |c| = 127 per vector): quantized exactly."""
    hs = shape[-1]
    n = int(np.prod(shape[:-1]))
    c = g.integers(-127, 128, size=(n, hs))
    c[np.arange(n), g.integers(0, hs, size=n)] = 127 * g.choice([-1, 1], size=n)
    j = g.integers(-9, 1, size=(n, 1))
    return (c * np.exp2(j)).astype(np.float32).reshape(shape)


class Case:
    """Random paged caches filled through the oracle writer, plus the original f32 rows."""

    def __init__(self, oracle_mod, seed, S, H, Hkv, hs, bs, lens, exact=True, spare_blocks=3):
        g = np.random.default_rng(seed)
        self.S, self.H, self.Hkv, self.hs, self.bs = S, H, Hkv, hs, bs
        self.lens = np.asarray(lens, dtype=np.uint32)
        nbs = [-(-int(L) // bs) for L in self.lens]
        self.max_nb = max(nbs + [1]) + 1
        self.num_blocks = sum(nbs) + spare_blocks
        perm = g.permutation(self.num_blocks).astype(np.uint32)
        self.bt = np.full((S, self.max_nb), self.num_blocks, dtype=np.uint32)
        at = 0
        for s, nb in enumerate(nbs):
            self.bt[s, :nb] = perm[at:at + nb]
            at += nb
        self.kc = wl.poison_cache(self.num_blocks + 1, Hkv, bs, hs)
        self.vc = wl.poison_cache(self.num_blocks + 1, Hkv, bs, hs)
        self.K, self.V = [], []
        for s in range(S):
            L = int(self.lens[s])
            if exact:
                K, V = lossless(g, (L, Hkv, hs)), lossless(g, (L, Hkv, hs))
            else:
                K = g.standard_normal((L, Hkv, hs)).astype(np.float32)
                V = g.standard_normal((L, Hkv, hs)).astype(np.float32)
            self.K.append(K)
            self.V.append(V)
            if L:
                pos = np.arange(L)
                slots = (self.bt[s, pos // bs].astype(np.int64) * bs + pos % bs).astype(np.uint32)
                oracle_mod.cache_write(K, V, self.kc, self.vc, slots, Hkv, hs, bs, num_blocks=self.num_blocks + 1)
        self.q = g.standard_normal((S, H, hs)).astype(np.float32)
        self.scale = float(np.float32(1.0 / np.sqrt(hs)))   # the scale argument is binary32

    def decode(self, oracle_mod, **kw):
        args = dict(max_context_len=None, num_blocks=self.num_blocks + 1)
        args.update(kw)
        return oracle_mod.paged_decode(self.q, self.kc, self.vc, self.bt, self.lens, self.scale,
                                       self.Hkv, self.bs, **args)

    def reference(self, K=None, V=None):
        K = self.K if K is None else K
        V = self.V if V is None else V
        n_rep = self.H // self.Hkv
        out = np.zeros((self.S, self.H, self.hs))
        for s in range(self.S):
            for h in range(self.H):
                out[s, h] = softmax_attend(self.q[s, h], K[s][:, h // n_rep], V[s][:, h // n_rep], self.scale)
        return out


@pytest.mark.parametrize("S,H,Hkv,hs,bs,lens", [
    (2, 4, 2, 64, 16, [37, 64]),
    (3, 8, 2, 32, 4, [1, 19, 50]),
    (2, 6, 3, 128, 32, [70, 33]),
    (2, 2, 2, 256, 16, [17, 3]),
])
def test_lossless_matches_bruteforce(oracle_mod, S, H, Hkv, hs, bs, lens):
    c = Case(oracle_mod, 1, S, H, Hkv, hs, bs, lens)
    got = c.decode(oracle_mod)
    ref = c.reference()
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)


def test_unquantized_error_bound(oracle_mod):
    """With eps = max_t scale*sum|q|*kscale_t*(1/2 + 2^-17), every logit moves by at
    most eps, so the softmax weights move by at most e^(2 eps) - 1 in total, and
    each value by at most vscale_t*(1/2 + 2^-17): the output bound follows."""
    c = Case(oracle_mod, 2, 2, 4, 2, 64, 16, [50, 29], exact=False)
    got = c.decode(oracle_mod).astype(np.float64)
    ref = c.reference()
    n_rep = c.H // c.Hkv
    for s in range(c.S):
        L = int(c.lens[s])
        for h in range(c.H):
            kvh = h // n_rep
            ks = np.abs(c.K[s][:, kvh]).max(axis=1) / 127
            vs = np.abs(c.V[s][:, kvh]).max(axis=1) / 127
            eps = c.scale * np.abs(c.q[s, h]).astype(np.float64).sum() * ks.max() * (0.5 + 2.0 ** -17)
            bound = (np.exp(2 * eps) - 1) * np.abs(c.V[s][:L, kvh]).max(axis=0) + vs.max() * (0.5 + 2.0 ** -17)
            assert np.all(np.abs(got[s, h] - ref[s, h]) <= bound + 1e-6)
    # the quantization error is real but far below the bound's scale
    assert np.abs(got - ref).max() > 1e-4


def test_one_token_returns_dequantized_v_exactly(oracle_mod):
    c = Case(oracle_mod, 3, 3, 4, 2, 64, 16, [1, 1, 1], exact=False)
    got = c.decode(oracle_mod)
    for s in range(c.S):
        b = c.bt[s, 0]
        for h in range(c.H):
            row = c.vc[b, h // 2, 0]
            codes = row[:16].copy().view(np.int8).astype(np.float32)
            vs = row[16:17].copy().view(np.float32)[0]
            assert np.array_equal(got[s, h], codes * vs)


def test_identical_keys_give_mean_of_values(oracle_mod):
    c = Case(oracle_mod, 4, 2, 4, 2, 64, 8, [23, 40], exact=False)
    for s in range(c.S):
        c.K[s][:] = c.K[s][0]
    # rebuild the caches with the tied keys
    kc, vc = wl.poison_cache(c.num_blocks + 1, 2, 8, 64), wl.poison_cache(c.num_blocks + 1, 2, 8, 64)
    for s in range(c.S):
        L = int(c.lens[s])
        pos = np.arange(L)
        slots = (c.bt[s, pos // 8].astype(np.int64) * 8 + pos % 8).astype(np.uint32)
        oracle_mod.cache_write(c.K[s], c.V[s], kc, vc, slots, 2, 64, 8)
    c.kc, c.vc = kc, vc
    got = c.decode(oracle_mod)
    for s in range(c.S):
        L = int(c.lens[s])
        for kvh in range(2):
            rows = np.stack([vc[c.bt[s, t // 8], kvh, t % 8] for t in range(L)])
            vhat = rows[:, :16].copy().view(np.int8).astype(np.float64) * rows[:, 16:17].copy().view(np.float32)
            mean = vhat.mean(axis=0)
            for h in (2 * kvh, 2 * kvh + 1):
                assert np.all(np.abs(got[s, h] - mean) <= 2.0 ** -23 * np.abs(mean) + 1e-12)


def test_gqa_mapping_constant_values(oracle_mod):
    """All values of kv head k equal a vector u_k: query head h returns u_{h // n_rep}."""
    c = Case(oracle_mod, 5, 2, 6, 3, 32, 16, [21, 40])
    u = lossless(np.random.default_rng(55), (3, 32))
    for s in range(c.S):
        c.V[s][:] = u[None]
    kc, vc = wl.poison_cache(c.num_blocks + 1, 3, 16, 32), wl.poison_cache(c.num_blocks + 1, 3, 16, 32)
    for s in range(c.S):
        L = int(c.lens[s])
        pos = np.arange(L)
        slots = (c.bt[s, pos // 16].astype(np.int64) * 16 + pos % 16).astype(np.uint32)
        oracle_mod.cache_write(c.K[s], c.V[s], kc, vc, slots, 3, 32, 16)
    c.kc, c.vc = kc, vc
    got = c.decode(oracle_mod)
    for s in range(c.S):
        for h in range(6):
            assert np.array_equal(got[s, h], u[h // 2]), (s, h)


def test_empty_context_gives_zero_row(oracle_mod):
    c = Case(oracle_mod, 6, 3, 4, 2, 64, 16, [0, 5, 0])
    got = c.decode(oracle_mod)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert np.all(np.isfinite(got[1])) and np.any(got[1] != 0)


def test_context_clamp(oracle_mod):
    c = Case(oracle_mod, 7, 2, 4, 2, 64, 16, [40, 70])
    got = c.decode(oracle_mod, max_context_len=33)
    K = [k[:33] for k in c.K]
    V = [v[:33] for v in c.V]
    ref = c.reference(K, V)
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)


def test_block_relabel_invariance(oracle_mod):
    c = Case(oracle_mod, 8, 2, 4, 2, 64, 16, [45, 70])
    base = c.decode(oracle_mod)
    perm = np.random.default_rng(88).permutation(c.num_blocks + 1)   # new id of old block b: perm[b]
    kc2, vc2 = np.empty_like(c.kc), np.empty_like(c.vc)
    kc2[perm] = c.kc
    vc2[perm] = c.vc
    c.kc, c.vc = kc2, vc2
    c.bt = perm[c.bt].astype(np.uint32)
    assert np.array_equal(c.decode(oracle_mod), base)


def test_gqa_equals_duplicated_mha(oracle_mod):
    c = Case(oracle_mod, 9, 2, 8, 2, 64, 16, [30, 52], exact=False)
    base = c.decode(oracle_mod)
    kc = np.repeat(c.kc, 4, axis=1)
    vc = np.repeat(c.vc, 4, axis=1)
    got = oracle_mod.paged_decode(c.q, kc, vc, c.bt, c.lens, c.scale, 8, 16)
    assert np.array_equal(got, base)


def test_visible_list_dense_and_compacted(oracle_mod):
    c = Case(oracle_mod, 10, 2, 4, 2, 64, 16, [60, 90], exact=False)
    dense = c.decode(oracle_mod)
    stride = 100
    vis = np.zeros((2, stride), np.uint32)
    nvis = c.lens.copy()
    for s in range(2):
        vis[s, :c.lens[s]] = np.arange(c.lens[s])
    got = oracle_mod.paged_decode(c.q, c.kc, c.vc, c.bt, np.zeros(2, np.uint32), c.scale, 2, 16,
                                  visible_pos=vis, num_visible=nvis, vis_stride=stride)
    assert np.array_equal(got, dense)
    # a sorted random subset equals dense decode over a cache holding only those rows
    g = np.random.default_rng(101)
    sub = [np.sort(g.choice(int(L), size=int(L) // 3, replace=False)) for L in c.lens]
    vis[:] = 0
    for s in range(2):
        vis[s, :sub[s].size] = sub[s]
    nvis = np.array([x.size for x in sub], np.uint32)
    got = oracle_mod.paged_decode(c.q, c.kc, c.vc, c.bt, c.lens, c.scale, 2, 16,
                                  visible_pos=vis, num_visible=nvis, vis_stride=stride)
    kc, vc = wl.poison_cache(c.num_blocks + 1, 2, 16, 64), wl.poison_cache(c.num_blocks + 1, 2, 16, 64)
    for s in range(2):
        for i, t in enumerate(sub[s]):
            src = (c.bt[s, t // 16], slice(None), t % 16)
            dst = (c.bt[s, i // 16], slice(None), i % 16)
            kc[dst] = c.kc[src]
            vc[dst] = c.vc[src]
    comp = oracle_mod.paged_decode(c.q, kc, vc, c.bt, nvis, c.scale, 2, 16)
    assert np.array_equal(got, comp)


def test_reads_no_unwritten_row(oracle_mod):
    """Rows past the context in a seq's last block hold NaN scale words; the oracle
    reports an error when it reads a non-finite logit, so success means it never read one."""
    c = Case(oracle_mod, 11, 2, 4, 2, 64, 16, [17, 31], exact=False)
    out = c.decode(oracle_mod)
    assert np.all(np.isfinite(out))
    bad = c.lens.copy()
    bad[0] = 20       # reaches unwritten rows
    with pytest.raises(ValueError):
        oracle_mod.paged_decode(c.q, c.kc, c.vc, c.bt, bad, c.scale, 2, 16)


def test_tiny_workload_against_vectorised_reference(oracle_mod):
    """The tiny workload end to end: fill then decode, against a numpy gather of the
    cache through its [blocks, Hkv, bs, wpt] view and an int8 view of the code words."""
    w = wl.tiny()
    kc, vc = w.empty_caches()
    for slots, k, v in w.fill_chunks():
        oracle_mod.cache_write(k, v, kc, vc, slots, w.num_kv_heads, w.head_size, w.block_size)
    q = w.q()
    got = oracle_mod.paged_decode(q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                  w.num_kv_heads, w.block_size)
    hs4 = w.head_size // 4
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        t = np.arange(L)
        blk = w.block_tables[s, t // w.block_size]
        for h in range(w.num_heads):
            kvh = h // (w.num_heads // w.num_kv_heads)
            kr, vr = kc[blk, kvh, t % w.block_size], vc[blk, kvh, t % w.block_size]
            K = kr[:, :hs4].copy().view(np.int8).astype(np.float64) * kr[:, hs4:].copy().view(np.float32)
            V = vr[:, :hs4].copy().view(np.int8).astype(np.float64) * vr[:, hs4:].copy().view(np.float32)
            ref = softmax_attend(q[s, h], K, V, w.scale)
            assert np.all(np.abs(got[s, h] - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)
