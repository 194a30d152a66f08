"""GPU parity of q8_cache_write against the oracle: the packed words of the whole
K and V buffers (including every untouched poison row) must be bit-identical."""
import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run_write(oracle, key, value, slots, nb, hkv, hs, bs, key_dev=None, value_dev=None):
    from int8_paged_kv_amd import q8_cache_write
    from gpu_util import u32_dev, f32_dev, u32_host
    kh, vh = wl.poison_cache(nb, hkv, bs, hs), wl.poison_cache(nb, hkv, bs, hs)
    kd, vd = u32_dev(kh), u32_dev(vh)
    q8_cache_write(f32_dev(key) if key_dev is None else key_dev,
                   f32_dev(value) if value_dev is None else value_dev,
                   kd, vd, u32_dev(slots), hkv, hs, bs)
    torch.cuda.synchronize()
    oracle.cache_write(key, value, kh, vh, slots, hkv, hs, bs,
                       key_stride=key.reshape(key.shape[0], -1).shape[1],
                       value_stride=value.reshape(value.shape[0], -1).shape[1])
    return u32_host(kd), u32_host(vd), kh, vh


def assert_words_equal(got, want, what):
    if not np.array_equal(got, want):
        diff = np.argwhere(got != want)
        i = tuple(diff[0])
        raise AssertionError("%s: %d words differ; first at %s: got %#010x want %#010x"
                             % (what, diff.shape[0], i, int(got[i]), int(want[i])))


@pytest.mark.parametrize("hs", [4, 8, 64, 68, 124, 128, 132, 252, 256])
def test_head_sizes_pads_zeros_and_ties(oracle_mod, hs):
    g = np.random.default_rng(1000 + hs)
    T, hkv, bs, nb = 37, 3, 16, 8
    key = g.standard_normal((T, hkv, hs)).astype(np.float32)
    val = (g.standard_normal((T, hkv, hs)) * 10).astype(np.float32)
    key[3, 1] = 0.0                                    # zero vector -> scale 1.0
    val[5, 2] = -0.0
    key[7, 0] = np.round(key[7, 0] * 20) + np.float32(0.5)   # exact ties with amax = 127
    key[7, 0, 0] = 127.0
    val[9] *= np.float32(1e-30)                        # tiny and huge magnitudes
    key[11] *= np.float32(1e30)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    slots[[0, 10, 20]] = wl.PAD_SLOT
    k, v, kh, vh = run_write(oracle_mod, key, val, slots, nb, hkv, hs, bs)
    assert_words_equal(k, kh, "key cache")
    assert_words_equal(v, vh, "value cache")


@pytest.mark.parametrize("extra", [0, 3, 4])
def test_strided_and_misaligned_rows(oracle_mod, extra):
    """Rows with a stride that is not a multiple of 4 floats, and rows starting
    one float past a 16-byte boundary, take the scalar-load path."""
    from gpu_util import f32_dev
    g = np.random.default_rng(77 + extra)
    T, hkv, hs, bs, nb = 29, 2, 128, 8, 8
    stride = hkv * hs + extra
    big = g.standard_normal((T, stride + 1)).astype(np.float32)
    key = np.ascontiguousarray(big[:, 1:1 + stride])
    val = np.ascontiguousarray(big[:, :stride] * 3)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    big_d = f32_dev(big)
    key_d = big_d[:, 1:1 + stride]                      # offset by one float: not 16-byte aligned
    val_d = f32_dev(val)
    k, v, kh, vh = run_write(oracle_mod, key, val, slots, nb, hkv, hs, bs, key_dev=key_d, value_dev=val_d)
    assert_words_equal(k, kh, "key cache")
    assert_words_equal(v, vh, "value cache")


def test_tiny_fill_bitexact(oracle_mod):
    from gpu_util import Filled, u32_host
    f = Filled(wl.tiny(), oracle_mod)
    assert_words_equal(u32_host(f.kc_d), f.kc_h, "key cache")
    assert_words_equal(u32_host(f.vc_d), f.vc_h, "value cache")


def test_mha256_4096_token_write(oracle_mod):
    """The MHA head_size=256 step write: 4096 tokens, 10% pad slots, 0.5% all-zero vectors."""
    w = wl.mha256()
    slots, k, v = wl.mha256_write(w)
    # a cache of just the blocks this write can touch keeps the test small: remap slots
    real = slots != wl.PAD_SLOT
    blocks = np.unique(slots[real] // w.block_size)
    remap = np.full(w.num_blocks, 0, dtype=np.int64)
    remap[blocks] = np.arange(blocks.size)
    s2 = slots.copy()
    s2[real] = (remap[slots[real] // w.block_size] * w.block_size + slots[real] % w.block_size).astype(np.uint32)
    kd, vd, kh, vh = run_write(oracle_mod, k, v, s2, blocks.size + 1, w.num_kv_heads, w.head_size, w.block_size)
    assert_words_equal(kd, kh, "key cache")
    assert_words_equal(vd, vh, "value cache")
    # zero vectors got scale word 1.0 and zero codes
    zk = np.argwhere((np.abs(k).max(axis=2) == 0) & real[:, None])
    t, h = zk[0]
    row = kh[s2[t] // w.block_size, h, s2[t] % w.block_size]
    assert row[-1] == 0x3F800000 and not row[:-1].any()


@pytest.mark.parametrize("T,hkv,hs", [(4103, 8, 128), (2053, 16, 256), (8191, 4, 64)])
def test_large_ragged_writes(oracle_mod, T, hkv, hs):
    """Writes of >= 32768 (token, kv head) pairs take several consecutive pairs
    per wave; pair counts that leave the last wave partly filled, with pads."""
    g = np.random.default_rng(T + hkv)
    bs = 16
    nb = T // bs + 8
    key = g.standard_normal((T, hkv, hs)).astype(np.float32)
    val = g.standard_normal((T, hkv, hs)).astype(np.float32)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    slots[g.choice(T, size=T // 10, replace=False)] = wl.PAD_SLOT
    slots[-1] = wl.PAD_SLOT
    k, v, kh, vh = run_write(oracle_mod, key, val, slots, nb, hkv, hs, bs)
    assert_words_equal(k, kh, "key cache")
    assert_words_equal(v, vh, "value cache")
