"""GPU parity of the per-head RMSNorm + partial rotary step against the oracle:
q8_rope_table, q8_norm_rope (q rows) and q8_norm_rope_cache_write (K normed and
rotated, then packed; V packed unchanged).

Both sides compute the step at the same binary32 rounding points, with the sum
of squares and the rotary angles in binary64.

* The rotary table each side builds (binary64 pow, cos and sin of independent
  libraries, each within an ulp or two) is compared entry by entry with a
  bound derived from that: an ulp of the entry's own binary32 value plus the
  angle's binary64 rounding, p * 2^-49 at position p, plus 2^-50.
* Everything downstream is given the oracle's table (copied to the device), so
  the only difference left is the order of the binary64 sum of squares (a
  lane tree on the GPU, sequential in the oracle).  That can move r =
  1/sqrt(mean + eps) across a binary32 rounding boundary only when the exact
  r lies within about 2^-45 of it; rows whose r lies within 2^-40 of one are
  found exactly (math.fsum) and are the only rows allowed to differ: q values
  by 4 ulps of the row's magnitude, K codes by 1 where the oracle's scaled
  value x*127/amax is within 1e-4 of a rounding tie, K scale words by 2 ulps.
  Every other row, and every V word and untouched slot, is bit-exact.
"""
import math

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
    # Each side forms phi = p * theta^(-2i/rot) in binary64 (pow within 2 ulps,
    # one rounding of the product: |dphi| <= p * 3 * 2^-52 <= p * 2^-49, as
    # theta^(-2i/rot) <= 1), then cos/sin (within an ulp, 2^-53 for values up to
    # 1, on either side: 2^-52 together) rounded once to binary32 (half an ulp of
    # the entry on either side).
    pos = np.arange(P, dtype=np.float64)[:, None]
    bound = np.spacing(np.abs(want)).astype(np.float64) + pos * 2.0 ** -49 + 2.0 ** -50
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    worst = np.unravel_index(np.argmax(diff - bound), diff.shape)
    assert np.all(diff <= bound), "entry %s: got %r want %r" % (worst, got[worst], want[worst])


def r_near_boundary(x, eps, margin=2.0 ** -40):
    """Whether r = 1/sqrt(mean(x^2) + eps) (exact sum of squares, math.fsum)
    lies within `margin` (relative) of a binary32 rounding boundary, where a
    different binary64 summation order could round it the other way."""
    x = np.asarray(x, dtype=np.float64)
    ss = math.fsum(float(v) * float(v) for v in x)
    r = 1.0 / math.sqrt(ss / x.size + float(eps))
    r32 = np.float32(r)
    lo = (float(np.nextafter(r32, np.float32(0))) + float(r32)) / 2
    hi = (float(np.nextafter(r32, np.float32(np.inf))) + float(r32)) / 2
    return min(abs(r - lo), abs(r - hi)) <= margin * r


def check_rows_exact(got, want, x_heads, eps):
    """q rows computed from the same table: bit-exact, except whole head
    vectors whose r is near a binary32 boundary (see the module docstring),
    which stay within 4 ulps of the vector's magnitude.  x_heads: the input
    head vectors, shaped like got."""
    from gpu_util import assert_close
    assert_close(got, want, "norm_rope")
    same = np.all(got.view(np.uint32) == want.view(np.uint32), axis=-1)
    for idx in zip(*np.nonzero(~same)):
        assert r_near_boundary(x_heads[idx], eps), "head vector %s differs away from a boundary of r" % (idx,)
        mag = np.max(np.abs(want[idx]))
        assert np.all(np.abs(got[idx].astype(np.float64) - want[idx]) <= 4 * 2.0 ** -24 * mag)
    return int(np.count_nonzero(~same))


def heads_of(x, T, H, hs, x_stride, head_stride):
    """[T, H, hs] view of head h of row t at x.flat[t*x_stride + h*head_stride]."""
    flat = np.ascontiguousarray(x).reshape(-1)
    return np.stack([np.stack([flat[t * x_stride + h * head_stride: t * x_stride + h * head_stride + hs]
                               for h in range(H)]) for t in range(T)]) if T else np.zeros((0, H, hs), np.float32)


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
    tab_d = f32_dev(tab_h) if rot else None                  # the oracle's table on both sides
    out = q8_norm_rope(f32_dev(x), u32_dev(pos) if rot else None, f32_dev(w), tab_d, rot, 1e-6, H, hs,
                       head_stride=head_stride)
    torch.cuda.synchronize()
    want = oracle_mod.norm_rope(x, pos, w, tab_h, rot, 1e-6, H, hs, x_stride=row, head_stride=head_stride)
    check_rows_exact(out.cpu().numpy(), want, heads_of(x, T, H, hs, row, head_stride), 1e-6)


def test_norm_rope_unaligned_rows_and_in_place(oracle_mod):
    from int8_paged_kv_amd import q8_norm_rope
    f32_dev, u32_dev, _ = dev()
    g = np.random.default_rng(5)
    T, H, hs, rot, P = 11, 4, 128, 64, 1000
    base = g.standard_normal(T * H * hs + 1).astype(np.float32)
    xd = f32_dev(base)[1:].view(T, H * hs)                 # rows 4 bytes off 16-byte alignment
    w = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    pos = g.integers(0, P, T).astype(np.uint32)
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    tab_d = f32_dev(tab_h)
    out = q8_norm_rope(xd, u32_dev(pos), f32_dev(w), tab_d, rot, 1e-6, H, hs)
    want = oracle_mod.norm_rope(base[1:].reshape(T, H * hs), pos, w, tab_h, rot, 1e-6, H, hs)
    torch.cuda.synchronize()
    xh = base[1:].reshape(T, H, hs)
    check_rows_exact(out.cpu().numpy(), want, xh, 1e-6)
    xa = f32_dev(base[1:].reshape(T, H, hs).copy())       # in place: out is x
    q8_norm_rope(xa.view(T, H * hs), u32_dev(pos), f32_dev(w), tab_d, rot, 1e-6, H, hs, out=xa)
    torch.cuda.synchronize()
    check_rows_exact(xa.cpu().numpy(), want, xh, 1e-6)


def compare_k_rows(oracle_mod, got, want, key, slots, pos, w, tab, rot, hkv, hs, bs):
    """K words from the same table: exact, except in (token, head) vectors whose
    r is near a binary32 boundary, where a code may differ by 1 at a near-tie
    of the oracle's scaled value and the scale word by 2 ulps."""
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
        assert r_near_boundary(key[t, h], 1e-6), "K row (token %d, head %d) differs away from a boundary of r" % (t, h)
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
    tab_h = oracle_mod.rope_table(P, rot, theta) if rot else None
    tab_d = f32_dev(tab_h) if rot else None
    q8_norm_rope_cache_write(f32_dev(key), f32_dev(val), kd, vd, u32_dev(slots), u32_dev(pos) if rot else None,
                             f32_dev(w), tab_d, rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
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
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    tab_d = f32_dev(tab_h)
    q8_norm_rope_cache_write(f32_dev(key), f32_dev(val), kd, vd, u32_dev(slots), u32_dev(pos), f32_dev(w), tab_d,
                             rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
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
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    tab_d = f32_dev(tab_h)
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
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    tab_d = f32_dev(tab_h)
    q8_norm_rope_cache_write(f32_dev(key), f32_dev(val), kd, vd, u32_dev(slots), u32_dev(pos), f32_dev(w), tab_d,
                             rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
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
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    tab_d = f32_dev(tab_h)
    q8_norm_rope_cache_write(f32_dev(kx)[1:].view(T, hkv * hs), f32_dev(vx)[1:].view(T, hkv * hs), kd, vd,
                             u32_dev(slots), u32_dev(pos), f32_dev(wx)[1:], tab_d, rot, 1e-6, hkv, hs, bs)
    torch.cuda.synchronize()
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
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    tab_d = f32_dev(tab_h)
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
    if Tq:
        check_rows_exact(q1, oracle_mod.norm_rope(q, qpos, qw, tab_h, rot, 1e-6, H, hs), q.reshape(Tq, H, hs), 1e-6)
    oracle_mod.norm_rope_cache_write(key, val, kh, vh, slots, kpos, kw, tab_h, rot, 1e-6, hkv, hs, bs)
    assert np.array_equal(u32_host(vd1), vh)
    n = compare_k_rows(oracle_mod, u32_host(kd1), kh, key.reshape(T, hkv, hs), slots, kpos, kw, tab_h, rot, hkv, hs,
                       bs)
    assert n <= max(2, T * hkv // 10000)
