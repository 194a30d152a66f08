"""GPU parity of the per-head RMSNorm + partial rotary step against the oracle:
q8_rope_table, q8_norm_rope (q rows) and q8_norm_rope_cache_write (K normed and
rotated, then packed; V packed unchanged).

Both sides compute the step at the same binary32 rounding points, with the sum
of squares and the rotary angles in binary64.  Independent binary64 library
routines (square root, pow, cos, sin) may still round a result to the other
side of a binary32 boundary, very rarely.  So:
* the rotary tables must agree within 2^-24 (an ulp of 1), and exactly in all
  but a small fraction of entries;
* q8_norm_rope outputs must be within 1e-4 + 1e-4|x| of the oracle and within
  a few ulps of the row's magnitude;
* packed V words, untouched slots and the code words of K must be bit-exact,
  except a K code may differ by 1 where the oracle's scaled value x*127/amax
  lies within 1e-4 of a rounding tie, and a K scale word may differ by 2 ulps.
"""
import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev():
    from gpu_util import f32_dev, u32_dev, u32_host
    return f32_dev, u32_dev, u32_host


def gpu_table(P, rot, theta):
    from int8_paged_kv_amd import q8_rope_table
    t = q8_rope_table(P, rot, theta, device="cuda:0")
    torch.cuda.synchronize()
    return t


@pytest.mark.parametrize("P,rot,theta", [(4096, 64, 10000.0), (65536, 32, 1e6), (300, 8, 500.0), (2048, 256, 10000.0)])
def test_rope_table(oracle_mod, P, rot, theta):
    got = gpu_table(P, rot, theta).cpu().numpy()
    want = oracle_mod.rope_table(P, rot, theta)
    # The binary64 angle p * theta^(-2i/rot) carries ~p * 2^-53 rad of library
    # rounding on either side: entries may differ by an ulp of their own
    # (possibly tiny) value, never by more than an ulp of 1.
    assert np.max(np.abs(got.astype(np.float64) - want)) <= 2.0 ** -24
    assert np.count_nonzero(got != want) <= max(2, got.size // 200)


def check_rows_close(got, want):
    from gpu_util import assert_close
    assert_close(got, want, "norm_rope")
    mag = np.max(np.abs(want), axis=-1, keepdims=True)
    assert np.all(np.abs(got.astype(np.float64) - want) <= 4 * 2.0 ** -24 * mag + 1e-37)


@pytest.mark.parametrize("hs,rot,H,head_stride,T", [
    (128, 64, 32, 256, 64),      # q and gate interleaved per head (stride 2*head_dim), 64 rows
    (128, 128, 8, 128, 33),
    (64, 32, 6, 64, 17),
    (256, 64, 4, 256, 9),
    (256, 0, 3, 260, 5),
    (32, 8, 5, 40, 3),
])
def test_norm_rope_rows(oracle_mod, hs, rot, H, head_stride, T):
    from int8_paged_kv_amd import q8_norm_rope
    f32_dev, u32_dev, _ = dev()
    g = np.random.default_rng(hs * 7 + rot + H)
    P = 8192
    row = (H - 1) * head_stride + hs + 4
    x = (g.standard_normal((T, row)) * g.uniform(0.1, 20, (T, 1))).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    pos = g.integers(0, P, T).astype(np.uint32)
    tab_h = oracle_mod.rope_table(P, rot, 10000.0) if rot else None
    tab_d = gpu_table(P, rot, 10000.0) if rot else None
    out = q8_norm_rope(f32_dev(x), u32_dev(pos) if rot else None, f32_dev(w), tab_d, rot, 1e-6, H, hs,
                       head_stride=head_stride)
    torch.cuda.synchronize()
    want = oracle_mod.norm_rope(x, pos, w, tab_h, rot, 1e-6, H, hs, x_stride=row, head_stride=head_stride)
    check_rows_close(out.cpu().numpy(), want)


def test_norm_rope_unaligned_rows_and_in_place(oracle_mod):
    from int8_paged_kv_amd import q8_norm_rope
    f32_dev, u32_dev, _ = dev()
    g = np.random.default_rng(5)
    T, H, hs, rot, P = 11, 4, 128, 64, 1000
    base = g.standard_normal(T * H * hs + 1).astype(np.float32)
    xd = f32_dev(base)[1:].view(T, H * hs)                 # rows 4 bytes off 16-byte alignment
    w = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    pos = g.integers(0, P, T).astype(np.uint32)
    tab_d = gpu_table(P, rot, 10000.0)
    out = q8_norm_rope(xd, u32_dev(pos), f32_dev(w), tab_d, rot, 1e-6, H, hs)
    want = oracle_mod.norm_rope(base[1:].reshape(T, H * hs), pos, w, oracle_mod.rope_table(P, rot, 10000.0), rot,
                                1e-6, H, hs)
    torch.cuda.synchronize()
    check_rows_close(out.cpu().numpy(), want)
    xa = f32_dev(base[1:].reshape(T, H, hs).copy())       # in place: out is x
    q8_norm_rope(xa.view(T, H * hs), u32_dev(pos), f32_dev(w), tab_d, rot, 1e-6, H, hs, out=xa)
    torch.cuda.synchronize()
    check_rows_close(xa.cpu().numpy(), want)


def compare_k_rows(oracle_mod, got, want, key, slots, pos, w, tab, rot, hkv, hs, bs):
    """K words: exact, except code +-1 at near-ties of the oracle's scaled value and scale +-2 ulps."""
    hs4 = hs // 4
    diff = got != want
    if not diff.any():
        return 0
    blocks, heads, offs = np.nonzero(diff.any(axis=-1))
    slot_of = {int(s): t for t, s in enumerate(slots) if s != wl.PAD_SLOT}
    allowed = 0
    for b, h, o in zip(blocks, heads, offs):
        t = slot_of.get(int(b) * bs + int(o))
        assert t is not None, "a word changed outside the written slots"
        y = oracle_mod.norm_rope_row(key[t, h], w, tab[pos[t]] if rot else None, rot, 1e-6)
        amax = np.float32(np.max(np.abs(y)))
        inv = np.float32(127.0) / amax
        scaled = (y * inv).astype(np.float64)
        near = np.abs(np.abs(scaled - np.floor(scaled)) - 0.5) < 1e-4
        gw, ww = got[b, h, o], want[b, h, o]
        gc = gw[:hs4].view(np.int8).astype(np.int32)
        wc = ww[:hs4].view(np.int8).astype(np.int32)
        dc = gc != wc
        assert np.all(np.abs(gc - wc) <= 1) and np.all(near[dc]), "code differs away from a rounding tie"
        assert abs(int(gw[hs4]) - int(ww[hs4])) <= 2, "scale word differs by more than 2 ulps"
        allowed += 1
    return allowed


@pytest.mark.parametrize("hs,rot,hkv,theta,stride_pad", [
    (128, 64, 8, 10000.0, 0),
    (128, 128, 2, 1e6, 8),
    (64, 32, 3, 10000.0, 4),
    (64, 0, 2, 10000.0, 0),
    (256, 64, 2, 10000.0, 0),
    (256, 256, 1, 1e6, 12),
    (32, 8, 4, 10000.0, 0),
])
def test_norm_rope_cache_write(oracle_mod, hs, rot, hkv, theta, stride_pad):
    from int8_paged_kv_amd import q8_norm_rope_cache_write
    f32_dev, u32_dev, u32_host = dev()
    g = np.random.default_rng(hs + rot + hkv)
    T, bs, nb, P = 53, 16, 12, 4096
    stride = hkv * hs + stride_pad
    key = (g.standard_normal((T, stride)) * g.uniform(0.05, 30, (T, 1))).astype(np.float32)
    val = g.standard_normal((T, stride)).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    slots[[0, 9, 30]] = wl.PAD_SLOT
    pos = g.integers(0, P, T).astype(np.uint32)
    pos[9] = 0xFFFFFFFF                                   # a pad token's position is not used
    kh, vh = wl.poison_cache(nb, hkv, bs, hs), wl.poison_cache(nb, hkv, bs, hs)
    kd, vd = u32_dev(kh), u32_dev(vh)
    tab_d = gpu_table(P, rot, theta) if rot else None
    q8_norm_rope_cache_write(f32_dev(key), f32_dev(val), kd, vd, u32_dev(slots), u32_dev(pos) if rot else None,
                             f32_dev(w), tab_d, rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
    tab_h = oracle_mod.rope_table(P, rot, theta) if rot else None
    oracle_mod.norm_rope_cache_write(key, val, kh, vh, slots, np.where(slots == wl.PAD_SLOT, 0, pos), w, tab_h, rot,
                                     1e-6, hkv, hs, bs, key_stride=stride, value_stride=stride)
    assert np.array_equal(u32_host(vd), vh)
    k3 = key.reshape(T, -1)[:, :hkv * hs].reshape(T, hkv, hs)
    n = compare_k_rows(oracle_mod, u32_host(kd), kh, k3, slots, pos, w, tab_h, rot, hkv, hs, bs)
    assert n <= 2


def test_norm_rope_cache_write_bulk_llama_shape(oracle_mod):
    """16384 tokens of the Llama-shaped cache (8 kv heads, head_size 128, rot 64)
    at scattered slots and positions, the bulk write the bench times."""
    from int8_paged_kv_amd import q8_norm_rope_cache_write
    f32_dev, u32_dev, u32_host = dev()
    g = np.random.default_rng(77)
    T, hkv, hs, bs, rot, P = 16384, 8, 128, 16, 64, 32768
    nb = T // bs + 64
    key = g.standard_normal((T, hkv, hs)).astype(np.float32)
    val = g.standard_normal((T, hkv, hs)).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    pos = g.integers(0, P, T).astype(np.uint32)
    kh, vh = wl.poison_cache(nb, hkv, bs, hs), wl.poison_cache(nb, hkv, bs, hs)
    kd, vd = u32_dev(kh), u32_dev(vh)
    tab_d = gpu_table(P, rot, 10000.0)
    q8_norm_rope_cache_write(f32_dev(key), f32_dev(val), kd, vd, u32_dev(slots), u32_dev(pos), f32_dev(w), tab_d,
                             rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    oracle_mod.norm_rope_cache_write(key, val, kh, vh, slots, pos, w, tab_h, rot, 1e-6, hkv, hs, bs)
    assert np.array_equal(u32_host(vd), vh)
    n = compare_k_rows(oracle_mod, u32_host(kd), kh, key, slots, pos, w, tab_h, rot, hkv, hs, bs)
    assert n <= max(4, T * hkv // 10000)


def test_norm_rope_then_decode_matches_oracle(oracle_mod):
    """The attention step with the norm + rotary step on both sides: q rows and
    the new K rows through it, written and attended; the decode output against
    the oracle's decode over the oracle's caches."""
    from int8_paged_kv_amd import q8_norm_rope, q8_norm_rope_cache_write, q8_paged_decode
    from gpu_util import assert_close
    f32_dev, u32_dev, u32_host = dev()
    w_ = wl.tiny()
    g = np.random.default_rng(8)
    hs, hkv, H, bs, rot = w_.head_size, w_.num_kv_heads, w_.num_heads, w_.block_size, 32
    P = 256
    tab_d, tab_h = gpu_table(P, rot, 10000.0), oracle_mod.rope_table(P, rot, 10000.0)
    kn = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    qn = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    kh, vh = w_.empty_caches()
    kd, vd = u32_dev(kh), u32_dev(vh)
    for slots, k, v in w_.fill_chunks():
        # positions of the fill: slot -> (sequence, logical position)
        pos = np.zeros(slots.shape[0], np.uint32)
        for t, s in enumerate(slots):
            b, o = divmod(int(s), bs)
            seq, j = np.argwhere(w_.block_tables == b)[0]
            pos[t] = j * bs + o
        q8_norm_rope_cache_write(f32_dev(k), f32_dev(v), kd, vd, u32_dev(slots), u32_dev(pos), f32_dev(kn), tab_d,
                                 rot, 1e-6, hkv, hs, bs)
        oracle_mod.norm_rope_cache_write(k, v, kh, vh, slots, pos, kn, tab_h, rot, 1e-6, hkv, hs, bs)
    q = w_.q()
    qpos = (np.asarray(w_.context_lens) - 1).astype(np.uint32)
    qd = q8_norm_rope(f32_dev(q.reshape(q.shape[0], -1)), u32_dev(qpos), f32_dev(qn), tab_d, rot, 1e-6, H, hs)
    qh = oracle_mod.norm_rope(q.reshape(q.shape[0], -1), qpos, qn, tab_h, rot, 1e-6, H, hs)
    out = q8_paged_decode(qd, kd, vd, u32_dev(w_.block_tables), u32_dev(w_.context_lens), w_.scale, hkv, bs,
                          max_context_len=w_.max_context_len)
    torch.cuda.synchronize()
    # the caches the decode read agree with the oracle's
    assert np.array_equal(u32_host(vd), vh) and np.array_equal(u32_host(kd), kh)
    ref = oracle_mod.paged_decode(qh, kh, vh, w_.block_tables, w_.context_lens, w_.scale, hkv, bs)
    assert_close(out.cpu().numpy(), ref, "decode after norm + rotary")


@pytest.mark.parametrize("T,hkv,hs,rot", [
    (4103, 8, 128, 64),      # four heads of a token per wave
    (2053, 16, 256, 128),    # two heads of a token per wave, head size above 128
    (16411, 2, 64, 32),      # two heads of a token per wave
    (10939, 3, 128, 64),     # pairs straddle tokens; the last wave holds one pair
    (10923, 3, 256, 128),    # the same above head size 128
])
def test_norm_rope_cache_write_large_ragged(oracle_mod, T, hkv, hs, rot):
    """>= 32768 pairs (several consecutive pairs per wave), a partly filled last
    wave or workgroup, pads among them."""
    from int8_paged_kv_amd import q8_norm_rope_cache_write
    f32_dev, u32_dev, u32_host = dev()
    g = np.random.default_rng(T)
    bs, P = 16, 8192
    nb = T // bs + 8
    key = g.standard_normal((T, hkv, hs)).astype(np.float32)
    val = g.standard_normal((T, hkv, hs)).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    slots[g.choice(T, size=T // 10, replace=False)] = wl.PAD_SLOT
    slots[-1] = wl.PAD_SLOT
    pos = g.integers(0, P, T).astype(np.uint32)
    kh, vh = wl.poison_cache(nb, hkv, bs, hs), wl.poison_cache(nb, hkv, bs, hs)
    kd, vd = u32_dev(kh), u32_dev(vh)
    tab_d = gpu_table(P, rot, 10000.0)
    q8_norm_rope_cache_write(f32_dev(key), f32_dev(val), kd, vd, u32_dev(slots), u32_dev(pos), f32_dev(w), tab_d,
                             rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    oracle_mod.norm_rope_cache_write(key, val, kh, vh, slots, pos, w, tab_h, rot, 1e-6, hkv, hs, bs)
    assert np.array_equal(u32_host(vd), vh)
    n = compare_k_rows(oracle_mod, u32_host(kd), kh, key, slots, pos, w, tab_h, rot, hkv, hs, bs)
    assert n <= 4


def test_norm_rope_cache_write_unaligned_weight_and_rows(oracle_mod):
    """Weight and K/V rows 4 bytes off 16-byte alignment (element loads)."""
    from int8_paged_kv_amd import q8_norm_rope_cache_write
    f32_dev, u32_dev, u32_host = dev()
    g = np.random.default_rng(21)
    T, hkv, hs, bs, nb, rot, P = 29, 2, 128, 16, 8, 64, 512
    wx = (1.0 + 0.1 * g.standard_normal(hs + 1)).astype(np.float32)
    kx = g.standard_normal(T * hkv * hs + 1).astype(np.float32)
    vx = g.standard_normal(T * hkv * hs + 1).astype(np.float32)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    pos = g.integers(0, P, T).astype(np.uint32)
    kh, vh = wl.poison_cache(nb, hkv, bs, hs), wl.poison_cache(nb, hkv, bs, hs)
    kd, vd = u32_dev(kh), u32_dev(vh)
    tab_d = gpu_table(P, rot, 10000.0)
    q8_norm_rope_cache_write(f32_dev(kx)[1:].view(T, hkv * hs), f32_dev(vx)[1:].view(T, hkv * hs), kd, vd,
                             u32_dev(slots), u32_dev(pos), f32_dev(wx)[1:], tab_d, rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    key, val, w = kx[1:].reshape(T, hkv, hs), vx[1:].reshape(T, hkv, hs), wx[1:]
    oracle_mod.norm_rope_cache_write(key, val, kh, vh, slots, pos, w, tab_h, rot, 1e-6, hkv, hs, bs)
    assert np.array_equal(u32_host(vd), vh)
    assert compare_k_rows(oracle_mod, u32_host(kd), kh, key, slots, pos, w, tab_h, rot, hkv, hs, bs) <= 2


@pytest.mark.parametrize("Tq,H,T,hkv,hs,rot", [
    (64, 32, 64, 8, 128, 64),        # the decode step's shape: 64 sequences, one new token each
    (5, 4, 7, 2, 256, 128),          # head size above 128
    (0, 4, 9, 2, 64, 32),            # no q rows: the write alone
    (6, 3, 0, 2, 64, 32),            # no new tokens: the q rows alone
    (3, 8, 4200, 8, 128, 64),        # a bulk write: q rows, then the batched writer
])
def test_norm_rope_qk_cache_write(oracle_mod, Tq, H, T, hkv, hs, rot):
    """q rows and the K/V write in one launch: bit-identical to q8_norm_rope
    followed by q8_norm_rope_cache_write, and against the oracle."""
    from int8_paged_kv_amd import q8_norm_rope, q8_norm_rope_cache_write, q8_norm_rope_qk_cache_write
    f32_dev, u32_dev, u32_host = dev()
    g = np.random.default_rng(Tq * 31 + T + hs)
    bs, P = 16, 8192
    nb = T // bs + 4
    q = (g.standard_normal((Tq, H * hs)) * 3).astype(np.float32)
    qpos = g.integers(0, P, Tq).astype(np.uint32)
    key = (g.standard_normal((T, hkv * hs)) * g.uniform(0.05, 30, (T, 1))).astype(np.float32)
    val = g.standard_normal((T, hkv * hs)).astype(np.float32)
    qw = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    kw = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    if T > 3:
        slots[[1, T // 2]] = wl.PAD_SLOT
    kpos = g.integers(0, P, T).astype(np.uint32)
    tab_d = gpu_table(P, rot, 10000.0)
    kh, vh = wl.poison_cache(nb, hkv, bs, hs), wl.poison_cache(nb, hkv, bs, hs)
    kd1, vd1 = u32_dev(kh), u32_dev(vh)
    qo1 = q8_norm_rope_qk_cache_write(f32_dev(q), u32_dev(qpos), f32_dev(qw), H, f32_dev(key), f32_dev(val), kd1, vd1,
                                      u32_dev(slots), u32_dev(kpos), f32_dev(kw), tab_d, rot, 1e-6, hkv, hs, bs)
    kd2, vd2 = u32_dev(kh), u32_dev(vh)
    qo2 = q8_norm_rope(f32_dev(q), u32_dev(qpos), f32_dev(qw), tab_d, rot, 1e-6, H, hs)
    q8_norm_rope_cache_write(f32_dev(key), f32_dev(val), kd2, vd2, u32_dev(slots), u32_dev(kpos), f32_dev(kw), tab_d,
                             rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
    q1, q2 = qo1.cpu().numpy(), qo2.cpu().numpy()
    assert np.array_equal(q1.view(np.uint32), q2.view(np.uint32)), "q rows differ from the separate call"
    assert np.array_equal(u32_host(kd1), u32_host(kd2)) and np.array_equal(u32_host(vd1), u32_host(vd2)), \
        "caches differ from the separate call"
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    if Tq:
        check_rows_close(q1, oracle_mod.norm_rope(q, qpos, qw, tab_h, rot, 1e-6, H, hs))
    oracle_mod.norm_rope_cache_write(key, val, kh, vh, slots, kpos, kw, tab_h, rot, 1e-6, hkv, hs, bs)
    assert np.array_equal(u32_host(vd1), vh)
    n = compare_k_rows(oracle_mod, u32_host(kd1), kh, key.reshape(T, hkv, hs), slots, kpos, kw, tab_h, rot, hkv, hs,
                       bs)
    assert n <= max(2, T * hkv // 10000)
