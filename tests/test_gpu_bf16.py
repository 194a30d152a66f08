"""GPU parity of the bfloat16 paged-cache baseline against the oracle.

The writer must store, bit for bit, the encodings the oracle's writer stores
(round to nearest, ties to even; pads untouched); the decode must meet
|gpu - oracle| <= 1e-4 + 1e-4*|oracle| on every output with no NaN, over head
sizes, GQA ratios, block sizes on both sides of the chunk length, empty and
clamped sequences, and wave counts that put the boundaries between the
persistent waves' ranges everywhere."""
import os

import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture
def baseline_waves():
    def set_(n):
        os.environ["Q8KV_F32_DECODE_WAVES"] = str(n)
    yield set_
    os.environ.pop("Q8KV_F32_DECODE_WAVES", None)


class Bf16Gpu:
    """Random bf16 paged caches written on the host by the oracle, copied to the device."""

    def __init__(self, oracle, seed, S, H, Hkv, hs, bs, lens, spare_blocks=2, spread=1.0):
        from gpu_util import bf16_dev, f32_dev, u32_dev
        g = np.random.default_rng(seed)
        self.S, self.H, self.Hkv, self.hs, self.bs = S, H, Hkv, hs, bs
        self.lens = np.asarray(lens, dtype=np.uint32)
        nbs = [-(-int(L) // bs) for L in self.lens]
        self.max_nb = max(nbs + [1])
        self.num_blocks = sum(nbs) + spare_blocks
        perm = g.permutation(self.num_blocks).astype(np.uint32)
        self.bt = np.full((S, self.max_nb), self.num_blocks, dtype=np.uint32)   # poison block
        at = 0
        for s, nb in enumerate(nbs):
            self.bt[s, :nb] = perm[at:at + nb]
            at += nb
        self.kc = wl.poison_cache_bf16(self.num_blocks + 1, Hkv, bs, hs)
        self.vc = wl.poison_cache_bf16(self.num_blocks + 1, Hkv, bs, hs)
        for s in range(S):
            L = int(self.lens[s])
            if not L:
                continue
            K = (g.standard_normal((L, Hkv, hs)) * spread).astype(np.float32)
            V = g.standard_normal((L, Hkv, hs)).astype(np.float32)
            pos = np.arange(L)
            slots = (self.bt[s, pos // bs].astype(np.int64) * bs + pos % bs).astype(np.uint32)
            oracle.bf16_cache_write(K, V, self.kc, self.vc, slots, Hkv, hs, bs)
        self.q = g.standard_normal((S, H, hs)).astype(np.float32)
        self.scale = float(np.float32(1.0 / np.sqrt(hs)))
        self.kc_d, self.vc_d = bf16_dev(self.kc), bf16_dev(self.vc)
        self.q_d = f32_dev(self.q)
        self.bt_d = u32_dev(self.bt)
        self.cl_d = u32_dev(self.lens)

    def gpu(self, max_context_len=None, **kw):
        from gpu_util import nan_out
        from int8_paged_kv_amd import q8_bf16_paged_decode
        mcl = int(self.lens.max()) if max_context_len is None else max_context_len
        kw.setdefault("out", nan_out(self.S, self.H, self.hs))
        out = q8_bf16_paged_decode(self.q_d, self.kc_d, self.vc_d, self.bt_d, self.cl_d, self.scale, self.Hkv,
                                   self.bs, max_context_len=mcl, **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle(self, oracle, max_context_len=None):
        return oracle.bf16_paged_decode(self.q, self.kc, self.vc, self.bt, self.lens, self.scale, self.Hkv,
                                        self.bs, max_context_len=max_context_len)


@pytest.mark.parametrize("hs,Hkv,T,pad", [(128, 8, 300, 0), (64, 2, 77, 12), (256, 1, 40, 4), (24, 3, 33, 0),
                                          (16, 4, 5, 0), (8, 2, 19, 0)])
def test_writer_bit_exact(oracle_mod, hs, Hkv, T, pad):
    from gpu_util import bf16_dev, bf16_host, f32_dev, u32_dev
    from int8_paged_kv_amd import q8_bf16_cache_write
    g = np.random.default_rng(hs + T)
    bs, nb = 16, (T + 15) // 16 + 3
    slots = g.permutation(nb * bs)[:T].astype(np.uint32)
    slots[g.random(T) < 0.1] = wl.PAD_SLOT
    K = (g.standard_normal((T, Hkv * hs + pad)) * 50).astype(np.float32)
    V = g.standard_normal((T, Hkv * hs + pad)).astype(np.float32)
    # exact ties between two bfloat16 neighbours, both parities, and values
    # that overflow to infinity, so the rounding rule itself is exercised
    K[0, :8] = (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x3FFF8000, 0x7F7FFFFF,
                          0x00018000, 0x80000000], np.uint32)).view(np.float32)
    kh = wl.poison_cache_bf16(nb, Hkv, bs, hs)
    vh = wl.poison_cache_bf16(nb, Hkv, bs, hs)
    kd, vd = bf16_dev(kh), bf16_dev(vh)
    Kd, Vd = f32_dev(K), f32_dev(V)
    q8_bf16_cache_write(Kd[:, :Hkv * hs] if pad else Kd, Vd[:, :Hkv * hs] if pad else Vd, kd, vd, u32_dev(slots),
                        Hkv, hs, bs)
    oracle_mod.bf16_cache_write(K, V, kh, vh, slots, Hkv, hs, bs, key_stride=Hkv * hs + pad,
                                value_stride=Hkv * hs + pad)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(kd), kh)
    assert np.array_equal(bf16_host(vd), vh)


def test_writer_accepts_torch_bfloat16(oracle_mod):
    """A torch.bfloat16 cache holds the same encodings as the int16 form."""
    from gpu_util import f32_dev, u32_dev
    from int8_paged_kv_amd import q8_bf16_cache_write
    g = np.random.default_rng(81)
    T, Hkv, hs, bs, nb = 40, 2, 64, 16, 4
    slots = g.permutation(nb * bs)[:T].astype(np.uint32)
    K = g.standard_normal((T, Hkv * hs)).astype(np.float32)
    V = g.standard_normal((T, Hkv * hs)).astype(np.float32)
    kd = torch.zeros((nb, Hkv, bs, hs), dtype=torch.bfloat16, device="cuda:0")
    vd = torch.zeros_like(kd)
    q8_bf16_cache_write(f32_dev(K), f32_dev(V), kd, vd, u32_dev(slots), Hkv, hs, bs)
    kh = np.zeros((nb, Hkv, bs, hs), np.uint16)
    vh = kh.copy()
    oracle_mod.bf16_cache_write(K, V, kh, vh, slots, Hkv, hs, bs)
    torch.cuda.synchronize()
    assert np.array_equal(kd.view(torch.int16).cpu().numpy().view(np.uint16), kh)
    assert np.array_equal(vd.view(torch.int16).cpu().numpy().view(np.uint16), vh)


@pytest.mark.parametrize("S,H,Hkv,hs,bs,lens", [
    (3, 8, 2, 128, 16, [1, 200, 77]),
    (3, 4, 2, 64, 16, [0, 1, 17]),            # empty, one token, partial block
    (2, 4, 2, 64, 16, [0, 0]),                # nothing to attend: zero rows
    (2, 8, 8, 128, 16, [100, 33]),            # MHA (groups of one head)
    (2, 12, 2, 128, 16, [129, 70]),           # n_rep 6: three groups of 2
    (2, 6, 2, 64, 8, [90, 200]),              # n_rep 3: single heads
    (2, 16, 2, 128, 32, [333, 65]),           # n_rep 8: two groups of 4
    (2, 4, 1, 256, 16, [150, 40]),            # head_size 256 (one position per load)
    (3, 8, 2, 32, 16, [500, 3, 64]),          # head_size 32
    (2, 8, 4, 16, 16, [700, 129]),            # head_size 16 (two lanes per position)
    (3, 4, 2, 128, 1, [40, 17, 0]),           # block size 1
    (3, 4, 2, 128, 7, [50, 13, 99]),          # block size below the chunk, not dividing it
    (2, 4, 2, 64, 5, [61, 100]),
    (2, 4, 2, 128, 48, [200, 47]),            # block size above the chunk, not a multiple
    (2, 4, 2, 32, 256, [600, 255]),
    (70, 8, 2, 64, 16, list(range(0, 700, 10))),   # more than 64 sequences
])
def test_decode_shapes(oracle_mod, S, H, Hkv, hs, bs, lens):
    from gpu_util import assert_close
    c = Bf16Gpu(oracle_mod, sum(lens) + hs, S, H, Hkv, hs, bs, lens)
    assert_close(c.gpu(), c.oracle(oracle_mod), "bf16 decode")


def test_decode_peaked_scores(oracle_mod):
    """Keys scaled up so the softmax is dominated by a few positions: the
    running maximum is replaced often inside and across the waves' ranges."""
    from gpu_util import assert_close
    c = Bf16Gpu(oracle_mod, 91, 3, 8, 2, 128, 16, [1500, 64, 777], spread=6.0)
    assert_close(c.gpu(), c.oracle(oracle_mod), "peaked")


@pytest.mark.parametrize("waves", [1, 2, 3, 7, 64, 333, 4096])
def test_decode_wave_counts(oracle_mod, baseline_waves, waves):
    from gpu_util import assert_close
    baseline_waves(waves)
    c = Bf16Gpu(oracle_mod, 31, 5, 8, 2, 128, 16, [900, 0, 37, 2000, 16])
    assert_close(c.gpu(), c.oracle(oracle_mod), "waves=%d" % waves)


def test_context_clamp(oracle_mod):
    from gpu_util import assert_close
    c = Bf16Gpu(oracle_mod, 41, 3, 8, 2, 64, 16, [400, 9, 1000])
    assert_close(c.gpu(max_context_len=130), c.oracle(oracle_mod, max_context_len=130), "clamp")
    assert np.all(c.gpu(max_context_len=0) == 0)


def test_workspace_reuse(oracle_mod, baseline_waves):
    from gpu_util import assert_close
    from int8_paged_kv_amd import q8_bf16_paged_decode_workspace_bytes
    baseline_waves(16)
    c = Bf16Gpu(oracle_mod, 51, 4, 8, 2, 128, 16, [1200, 700, 5, 3000])
    ws = torch.zeros(q8_bf16_paged_decode_workspace_bytes(4, 8, 2, 128), dtype=torch.uint8, device="cuda:0")
    want = c.oracle(oracle_mod)
    for _ in range(3):
        assert_close(c.gpu(workspace=ws), want, "repeat")
    small = Bf16Gpu(oracle_mod, 52, 2, 8, 2, 128, 16, [800, 90])
    assert_close(small.gpu(workspace=ws), small.oracle(oracle_mod), "smaller batch")


def test_matches_int8_decode_on_exactly_quantized_cache(oracle_mod):
    """Rows c*2^j with max |c| = 127 are exact in bfloat16 (8 significant bits)
    and in the int8 cache, so the two HIP decodes attend the same values."""
    from gpu_util import RandomCase, assert_close, bf16_dev
    from int8_paged_kv_amd import q8_bf16_paged_decode
    from test_oracle_decode import lossless
    g = np.random.default_rng(62)
    S, H, Hkv, hs, bs = 3, 8, 2, 128, 16
    c = RandomCase(oracle_mod, 62, S, H, Hkv, hs, bs, [300, 1, 90])
    kb = wl.poison_cache_bf16(c.num_blocks + 1, Hkv, bs, hs)
    vb = wl.poison_cache_bf16(c.num_blocks + 1, Hkv, bs, hs)
    kf = wl.poison_cache_f32(c.num_blocks + 1, Hkv, bs, hs)
    vf = wl.poison_cache_f32(c.num_blocks + 1, Hkv, bs, hs)
    for s in range(S):
        L = int(c.lens[s])
        K, V = lossless(g, (L, Hkv, hs)), lossless(g, (L, Hkv, hs))
        pos = np.arange(L)
        slots = (c.bt[s, pos // bs].astype(np.int64) * bs + pos % bs).astype(np.uint32)
        oracle_mod.cache_write(K, V, c.kc, c.vc, slots, Hkv, hs, bs)
        oracle_mod.bf16_cache_write(K, V, kb, vb, slots, Hkv, hs, bs)
        oracle_mod.f32_cache_write(K, V, kf, vf, slots, Hkv, hs, bs)
    # every stored bfloat16 is the f32 value exactly
    live = ~np.isnan(kf)
    assert np.array_equal(oracle_mod.bf16_to_f32(kb)[live], kf[live])
    c.kc_d.copy_(torch.from_numpy(c.kc.view(np.int32)))
    c.vc_d.copy_(torch.from_numpy(c.vc.view(np.int32)))
    q8 = c.gpu()
    b16 = q8_bf16_paged_decode(c.q_d, bf16_dev(kb), bf16_dev(vb), c.bt_d, c.cl_d, c.scale, Hkv, bs).cpu().numpy()
    want = c.oracle(oracle_mod)
    assert np.array_equal(want, oracle_mod.bf16_paged_decode(c.q, kb, vb, c.bt, c.lens, c.scale, Hkv, bs))
    assert_close(q8, want, "int8")
    assert_close(b16, want, "bf16")


def test_llama_full_size_sampled(oracle_mod):
    """The Llama-3-8B-shaped batch (S=64, H=32, Hkv=8, hs=128, bs=16,
    L ~ U[512, 4096]) in the launch configuration the bench times: the whole
    written cache bit-exact against the oracle's writer, the decode checked on
    sampled (seq, head) outputs."""
    from gpu_util import assert_close, bf16_dev, bf16_host, f32_dev, u32_dev
    from int8_paged_kv_amd import q8_bf16_cache_write, q8_bf16_paged_decode
    w = wl.llama()
    nbt = w.num_blocks + 1
    kh = wl.poison_cache_bf16(nbt, w.num_kv_heads, w.block_size, w.head_size)
    vh = wl.poison_cache_bf16(nbt, w.num_kv_heads, w.block_size, w.head_size)
    kd, vd = bf16_dev(kh), bf16_dev(vh)
    writes = list(w.fill_chunks())
    step = w.step_write()
    if step is not None:
        writes.append(step)
    for slots, k, v in writes:
        q8_bf16_cache_write(f32_dev(k), f32_dev(v), kd, vd, u32_dev(slots), w.num_kv_heads, w.head_size,
                            w.block_size)
        oracle_mod.bf16_cache_write(k, v, kh, vh, slots, w.num_kv_heads, w.head_size, w.block_size)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(kd), kh) and np.array_equal(bf16_host(vd), vh)
    q = w.q()
    out = q8_bf16_paged_decode(f32_dev(q), kd, vd, u32_dev(w.block_tables), u32_dev(w.context_lens), w.scale,
                               w.num_kv_heads, w.block_size, max_context_len=w.max_context_len).cpu().numpy()
    assert np.all(np.isfinite(out))
    g = np.random.default_rng(72)
    units = np.stack([g.integers(0, w.num_seqs, 96), g.integers(0, w.num_heads, 96)], axis=1)
    want = oracle_mod.bf16_paged_decode_units(units, q, kh, vh, w.block_tables, w.context_lens, w.scale,
                                              w.num_kv_heads, w.block_size, max_context_len=w.max_context_len)
    got = np.stack([out[s, h] for s, h in units])
    assert_close(got, want, "llama sampled")
