"""Pins of the oracle's norm + rotary step (CPU only).

The "attention.rs" page normalizes q and k per head (learned weight, rms eps)
and rotates the first rot = head_dim * partial_rotary_factor elements at the
row's position (rope theta) before the q8 append; its kernel body is not
printed.  The reading (per-head RMSNorm, then a rotate-half rotary embedding
with frequencies theta^(-2i/rot)) is pinned here by:

* the rotary table against textbook values (cos 1, sin 1; an exact angle of
  one radian at a chosen frequency), cos^2 + sin^2 = 1 and the double angle;
* the binary64 definition against closed forms: constant vectors, one-hot
  vectors (which fix the pairing and the sign of each term), elements past rot,
  norm and scale invariance, and the relative-position property of rotations;
* the binary32 pipeline (the one the quantizer sees) against the binary64
  definition, element by element;
* the rows-of-heads function's indexing (row, head and output strides, the
  q/gate interleave of head stride 2*head_size, each row's table row) against
  numpy slicing of the same arrays and the binary64 definition at each row's
  position;
* the fused writer against the quantizer applied to the pipeline's rows (also
  with padded key/value row strides), pad slots untouched, and out-of-contract
  shapes and positions rejected.
"""
import math

import numpy as np
import pytest

import oracle
from int8_paged_kv_amd import workloads as wl

COS1 = 0.5403023058681398     # cos(1 rad)
SIN1 = 0.8414709848078965     # sin(1 rad)


def test_table_textbook_values():
    rot, theta = 64, 10000.0
    t = oracle.rope_table(128, rot, theta)
    half = rot // 2
    assert np.array_equal(t[0, :half], np.ones(half, np.float32))
    assert np.array_equal(t[0, half:], np.zeros(half, np.float32))
    # frequency 0 is 1 rad per position
    assert t[1, 0] == np.float32(COS1) and t[1, half] == np.float32(SIN1)
    # frequency 16 of 32 is theta^(-1/2) = 1/100 rad per position: position 100 is one radian
    assert t[100, 16] == np.float32(COS1) and t[100, half + 16] == np.float32(SIN1)
    c, s = t[:, :half].astype(np.float64), t[:, half:].astype(np.float64)
    assert np.max(np.abs(c * c + s * s - 1.0)) < 4 * 2.0 ** -24
    # double angle: cos(2a) = 2 cos^2 a - 1, sin(2a) = 2 sin a cos a
    assert np.max(np.abs(c[2:128:2] - (2 * c[1:64] ** 2 - 1))) < 1e-6
    assert np.max(np.abs(s[2:128:2] - 2 * s[1:64] * c[1:64])) < 1e-6


def test_constant_vector_closed_form():
    hs = 64
    w = np.random.default_rng(1).uniform(0.5, 1.5, hs).astype(np.float32)
    for c in (3.0, -0.25):
        x = np.full(hs, c, np.float32)
        y = oracle.norm_rope_row_f64(x, w, 0, 32, 10000.0, 0.0)
        assert np.allclose(y, math.copysign(1.0, c) * w.astype(np.float64), rtol=1e-15, atol=0)
        eps = 0.5
        y = oracle.norm_rope_row_f64(x, w, 0, 32, 10000.0, eps)
        assert np.allclose(y, c / math.sqrt(c * c + eps) * w.astype(np.float64), rtol=1e-14, atol=0)


@pytest.mark.parametrize("hs,rot", [(64, 32), (128, 64), (128, 128), (256, 64)])
def test_one_hot_fixes_pairing_and_sign(hs, rot):
    half = rot // 2
    w = np.ones(hs, np.float32)
    root = math.sqrt(hs)           # RMSNorm of a one-hot vector (eps = 0)
    e0 = np.zeros(hs, np.float32)
    e0[0] = 1.0
    y = oracle.norm_rope_row_f64(e0, w, 1, rot, 10000.0, 0.0)
    want = np.zeros(hs)
    want[0], want[half] = root * COS1, root * SIN1
    assert np.allclose(y, want, rtol=0, atol=1e-12)
    eh = np.zeros(hs, np.float32)
    eh[half] = 1.0
    y = oracle.norm_rope_row_f64(eh, w, 1, rot, 10000.0, 0.0)
    want = np.zeros(hs)
    want[0], want[half] = -root * SIN1, root * COS1
    assert np.allclose(y, want, rtol=0, atol=1e-12)
    # frequency 1: angle theta^(-2/rot) per position, written as exp(-2 ln(theta) / rot)
    e1 = np.zeros(hs, np.float32)
    e1[1] = 1.0
    phi = 3 * math.exp(-2.0 * math.log(10000.0) / rot)
    y = oracle.norm_rope_row_f64(e1, w, 3, rot, 10000.0, 0.0)
    assert abs(y[1] - root * math.cos(phi)) < 1e-12 and abs(y[1 + half] - root * math.sin(phi)) < 1e-12


def test_unrotated_elements_and_rot_zero():
    g = np.random.default_rng(2)
    hs = 128
    x = g.standard_normal(hs).astype(np.float32)
    w = g.uniform(0.5, 1.5, hs).astype(np.float32)
    n = oracle.norm_rope_row_f64(x, w, 0, 0, 10000.0, 1e-6)          # rot 0: RMSNorm only
    ref = x.astype(np.float64) / math.sqrt(np.mean(x.astype(np.float64) ** 2) + 1e-6) * w
    assert np.allclose(n, ref, rtol=1e-14, atol=0)
    y = oracle.norm_rope_row_f64(x, w, 777, 32, 10000.0, 1e-6)
    assert np.array_equal(y[32:], n[32:])
    assert np.allclose(oracle.norm_rope_row_f64(x, w, 0, 32, 10000.0, 1e-6), n, rtol=1e-15, atol=0)


def test_norm_scale_invariance_and_pair_norms():
    g = np.random.default_rng(3)
    hs, rot = 128, 64
    x = g.standard_normal(hs).astype(np.float32)
    ones = np.ones(hs, np.float32)
    y = oracle.norm_rope_row_f64(x, ones, 41, rot, 10000.0, 0.0)
    assert abs(np.mean(y ** 2) - 1.0) < 1e-12
    y2 = oracle.norm_rope_row_f64((x * np.float32(4.0)), ones, 41, rot, 10000.0, 0.0)
    assert np.allclose(y, y2, rtol=1e-13, atol=1e-15)
    n = oracle.norm_rope_row_f64(x, ones, 0, rot, 10000.0, 0.0)
    half = rot // 2
    assert np.allclose(y[:half] ** 2 + y[half:rot] ** 2, n[:half] ** 2 + n[half:rot] ** 2, rtol=1e-12)


def test_relative_position_property():
    """<R(p) a, R(q) b> over the rotated elements equals <R(p - q) a, b>."""
    g = np.random.default_rng(4)
    hs, rot = 64, 64
    ones = np.ones(hs, np.float32)
    a = g.standard_normal(hs).astype(np.float32)
    b = g.standard_normal(hs).astype(np.float32)
    for p, q in ((10, 3), (500, 499), (1000, 20)):
        lhs = np.dot(oracle.norm_rope_row_f64(a, ones, p, rot, 10000.0, 0.0),
                     oracle.norm_rope_row_f64(b, ones, q, rot, 10000.0, 0.0))
        rhs = np.dot(oracle.norm_rope_row_f64(a, ones, p - q, rot, 10000.0, 0.0),
                     oracle.norm_rope_row_f64(b, ones, 0, rot, 10000.0, 0.0))
        assert abs(lhs - rhs) < 1e-9


@pytest.mark.parametrize("hs,rot,theta", [(64, 32, 10000.0), (128, 64, 1e6), (256, 64, 10000.0), (128, 0, 1.0)])
def test_binary32_pipeline_tracks_definition(hs, rot, theta):
    g = np.random.default_rng(5)
    P = 4096
    tab = oracle.rope_table(P, rot, theta)
    w = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    for _ in range(40):
        x = (g.standard_normal(hs) * g.uniform(0.01, 30)).astype(np.float32)
        p = int(g.integers(0, P))
        y32 = oracle.norm_rope_row(x, w, tab[p] if rot else None, rot, 1e-6)
        y64 = oracle.norm_rope_row_f64(x, w, p, rot, theta, 1e-6)
        # a few binary32 roundings of values of the vector's own magnitude
        assert np.max(np.abs(y32 - y64)) <= 8 * 2.0 ** -24 * np.max(np.abs(y64)) + 1e-30


def test_writer_composes_norm_rope_and_quantizer():
    w_ = wl.tiny()
    g = np.random.default_rng(6)
    T, Hkv, hs, bs = 40, w_.num_kv_heads, w_.head_size, w_.block_size
    rot, P = 32, 512
    tab = oracle.rope_table(P, rot, 10000.0)
    wt = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    k = g.standard_normal((T, Hkv, hs)).astype(np.float32)
    v = g.standard_normal((T, Hkv, hs)).astype(np.float32)
    slots = g.permutation(w_.num_blocks * bs)[:T].astype(np.uint32)
    slots[::7] = oracle.PAD_SLOT
    pos = g.integers(0, P, T).astype(np.uint32)
    kc, vc = w_.empty_caches()
    kc0, vc0 = kc.copy(), vc.copy()
    oracle.norm_rope_cache_write(k, v, kc, vc, slots, pos, wt, tab, rot, 1e-6, Hkv, hs, bs)
    wpt = hs // 4 + 1
    written = np.zeros(kc.shape[:3], dtype=bool)
    for t in range(T):
        if slots[t] == oracle.PAD_SLOT:
            continue
        blk, off = divmod(int(slots[t]), bs)
        for h in range(Hkv):
            y = oracle.norm_rope_row(k[t, h], wt, tab[pos[t]], rot, 1e-6)
            assert np.array_equal(kc[blk, h, off], oracle.quantize_row(y))
            assert np.array_equal(vc[blk, h, off], oracle.quantize_row(v[t, h]))
            written[blk, h, off] = True
    assert np.array_equal(kc[~written], kc0[~written]) and np.array_equal(vc[~written], vc0[~written])
    assert kc.shape[-1] == wpt


@pytest.mark.parametrize("hs,rot,H,head_stride,pad_x,pad_out", [
    (128, 64, 4, 256, 12, 8),       # q and gate interleaved per head: head stride 2*head_size
    (64, 32, 3, 64, 4, 0),
    (32, 8, 5, 40, 0, 4),
    (256, 0, 2, 300, 7, 16),        # no rotation: positions and table unused
])
def test_rows_of_heads_indexing(hs, rot, H, head_stride, pad_x, pad_out):
    """Each output head is the row function of exactly the input slice numpy
    takes at (row * x_stride + head * head_stride), with the table row of that
    row's position, written at (row * out_stride + head * head_size); the
    padding between output rows is left alone.  A swapped stride, a head read
    at head_size instead of head_stride, or a wrong table row fails here."""
    g = np.random.default_rng(hs + rot + H)
    T, P, theta, eps = 9, 700, 10000.0, 1e-6
    xs = (H - 1) * head_stride + hs + pad_x
    os_ = H * hs + pad_out
    x = (g.standard_normal(T * xs) * 2.5).astype(np.float32)
    w = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    pos = g.permutation(P)[:T].astype(np.uint32)            # distinct, shuffled positions
    tab = oracle.rope_table(P, rot, theta) if rot else None
    out = np.full((T, os_), 1234.5, np.float32)
    oracle.norm_rope(x, pos, w, tab, rot, eps, H, hs, x_stride=xs, head_stride=head_stride, out_stride=os_,
                     out=out)
    for t in range(T):
        p = int(pos[t])
        for h in range(H):
            xi = x[t * xs + h * head_stride: t * xs + h * head_stride + hs]
            want = oracle.norm_rope_row(xi, w, tab[p] if rot else None, rot, eps)
            got = out[t, h * hs:(h + 1) * hs]
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (t, h)
            # and the position's angle, taken straight from theta, not from a table row
            y64 = oracle.norm_rope_row_f64(xi, w, p, rot, theta, eps)
            assert np.max(np.abs(got - y64)) <= 8 * 2.0 ** -24 * np.max(np.abs(y64)) + 1e-30, (t, h)
        assert np.all(out[t, H * hs:] == np.float32(1234.5)), "padding between output rows written"


def test_writer_row_strides():
    """The fused writer with key and value rows of different padded strides:
    each non-pad (token, kv head) is the quantizer of the row function of the
    slice at token * stride + head * head_size."""
    g = np.random.default_rng(16)
    T, Hkv, hs, bs, nb, rot, P = 23, 3, 64, 8, 12, 32, 300
    ks, vs = Hkv * hs + 20, Hkv * hs + 4
    key = g.standard_normal(T * ks).astype(np.float32)
    val = g.standard_normal(T * vs).astype(np.float32)
    tab = oracle.rope_table(P, rot, 500.0)
    wt = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    slots[[2, 11]] = oracle.PAD_SLOT
    pos = g.integers(0, P, T).astype(np.uint32)
    kc, vc = wl.poison_cache(nb, Hkv, bs, hs), wl.poison_cache(nb, Hkv, bs, hs)
    kc0, vc0 = kc.copy(), vc.copy()
    oracle.norm_rope_cache_write(key, val, kc, vc, slots, pos, wt, tab, rot, 1e-6, Hkv, hs, bs,
                                 key_stride=ks, value_stride=vs)
    written = np.zeros(kc.shape[:3], dtype=bool)
    for t in range(T):
        if slots[t] == oracle.PAD_SLOT:
            continue
        blk, off = divmod(int(slots[t]), bs)
        for h in range(Hkv):
            kx = key[t * ks + h * hs: t * ks + (h + 1) * hs]
            vx = val[t * vs + h * hs: t * vs + (h + 1) * hs]
            assert np.array_equal(kc[blk, h, off], oracle.quantize_row(oracle.norm_rope_row(kx, wt, tab[pos[t]],
                                                                                            rot, 1e-6)))
            assert np.array_equal(vc[blk, h, off], oracle.quantize_row(vx))
            written[blk, h, off] = True
    assert np.array_equal(kc[~written], kc0[~written]) and np.array_equal(vc[~written], vc0[~written])


def test_out_of_contract_rejected():
    hs = 64
    x = np.ones(hs, np.float32)
    w = np.ones(hs, np.float32)
    with pytest.raises(Exception):
        oracle.norm_rope_row(x, w, np.ones(6, np.float32), 3, 1e-6)          # odd rot
    with pytest.raises(Exception):
        oracle.norm_rope_row(x, w, np.ones(80, np.float32), 80, 1e-6)        # rot > head_size
    tab = oracle.rope_table(8, 16, 10000.0)
    with pytest.raises(Exception):
        oracle.norm_rope(x[None, :], np.array([8], np.uint32), w, tab, 16, 1e-6, 1, hs)   # position past the table
