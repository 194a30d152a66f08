"""Pins of the oracle's bf16 cache baseline (CPU).

* Rounding to bfloat16 (nearest, ties to even) against an independent
  implementation, torch's float32 -> bfloat16 conversion, over random values
  of every magnitude and the edge cases, plus hand-derived encodings:
  exact ties going to the even neighbour, a carry into the exponent, overflow
  to infinity, subnormals and signed zero.
* The writer's layout and pad handling: every stored element is the rounded
  input at [block, kv head, offset, d], pad tokens write nothing.
* The decode: on bfloat16 values it must give exactly the f32-cache decode (the
  definition already pinned for the f32 baseline) of the same values.
"""
import struct

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_of_bits(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u))[0]


@pytest.mark.parametrize("bits,want", [
    (0x3F800000, 0x3F80),    # 1.0
    (0x3F808000, 0x3F80),    # 1 + 2^-8: exactly halfway to 0x3F81, ties to the even 0x3F80
    (0x3F818000, 0x3F82),    # 1 + 3*2^-8: halfway between 0x3F81 and 0x3F82, ties to the even 0x3F82
    (0x3F808001, 0x3F81),    # just above half an ulp: rounds up
    (0x3F807FFF, 0x3F80),    # just below half an ulp: rounds down
    (0xBFC00000, 0xBFC0),    # -1.5, exact
    (0xBF818000, 0xBF82),    # negative tie: magnitude rounds to even
    (0x3FFF8000, 0x4000),    # halfway from the largest significand below 2: carries into the exponent (2.0)
    (0x7F7FFFFF, 0x7F80),    # the largest finite binary32 rounds past the largest bfloat16: infinity
    (0x7F7F7FFF, 0x7F7F),    # the largest bfloat16 itself, from just below half an ulp above it
    (0x00000001, 0x0000),    # the smallest subnormal rounds to +0
    (0x00018000, 0x0002),    # subnormal tie to even
    (0x80000000, 0x8000),    # -0 stays -0
])
def test_bf16_rounding_golden(oracle_mod, bits, want):
    got = int(oracle_mod.f32_to_bf16(np.array([f32_of_bits(bits)], np.float32))[0])
    assert got == want, "0x%08x -> 0x%04x, want 0x%04x" % (bits, got, want)


def test_bf16_rounding_matches_torch(oracle_mod):
    g = np.random.default_rng(3)
    # random bit patterns over every finite exponent, and values near ties
    u = g.integers(0, 0x7F800000, 20000, dtype=np.uint64).astype(np.uint32)
    u |= (g.integers(0, 2, u.size).astype(np.uint32) << 31)
    ties = (g.integers(0, 0x7F7F, 3000).astype(np.uint32) << 16) | np.uint32(0x8000)
    near = ties + g.integers(-2, 3, ties.size).astype(np.int64).astype(np.uint32)
    x = np.concatenate([u, ties, near]).view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(oracle_mod.f32_to_bf16(x), torch_bf16_bits(x))


def test_bf16_to_f32_is_the_upper_half(oracle_mod):
    b = np.array([0x3F80, 0xBFC0, 0x7F80, 0x0001, 0x8000], np.uint16)
    want = np.array([f32_of_bits(int(v) << 16) for v in b], np.float32)
    got = np.array([oracle_mod._load().q8o_bf16_to_f32(int(v)) for v in b], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_bf16_writer_layout_and_pads(oracle_mod):
    g = np.random.default_rng(4)
    T, Hkv, hs, bs, nb = 9, 3, 16, 4, 7
    key = (g.standard_normal((T, Hkv * hs + 5)) * 10).astype(np.float32)       # row stride with padding
    val = g.standard_normal((T, Hkv * hs + 5)).astype(np.float32)
    slots = g.choice(nb * bs, T, replace=False).astype(np.uint32)
    slots[[2, 6]] = oracle_mod.PAD_SLOT
    kc = np.full(nb * Hkv * bs * hs, 0xABCD, np.uint16)
    vc = kc.copy()
    oracle_mod.bf16_cache_write(key, val, kc, vc, slots, Hkv, hs, bs, key_stride=Hkv * hs + 5,
                                value_stride=Hkv * hs + 5)
    kw = np.full((nb, Hkv, bs, hs), 0xABCD, np.uint16)
    vw = kw.copy()
    for t, s in enumerate(slots):
        if s == oracle_mod.PAD_SLOT:
            continue
        for h in range(Hkv):
            kw[s // bs, h, s % bs] = torch_bf16_bits(key[t, h * hs:(h + 1) * hs])
            vw[s // bs, h, s % bs] = torch_bf16_bits(val[t, h * hs:(h + 1) * hs])
    assert np.array_equal(kc, kw.reshape(-1)) and np.array_equal(vc, vw.reshape(-1))


@pytest.mark.parametrize("bs,lens,mcl", [(16, [37, 0, 100], None), (5, [12, 61, 1], 40)])
def test_bf16_decode_is_the_f32_decode_of_the_stored_values(oracle_mod, bs, lens, mcl):
    g = np.random.default_rng(5)
    S, H, Hkv, hs = len(lens), 6, 2, 32
    nbs = [-(-L // bs) for L in lens]
    nb = sum(nbs) + 1
    perm = g.permutation(nb).astype(np.uint32)
    bt = np.zeros((S, max(nbs)), np.uint32)
    at = 0
    for s, n in enumerate(nbs):
        bt[s, :n] = perm[at:at + n]
        at += n
    kb = np.zeros(nb * Hkv * bs * hs, np.uint16)
    vb = kb.copy()
    for s, L in enumerate(lens):
        if not L:
            continue
        k = (g.standard_normal((L, Hkv * hs)) * 3).astype(np.float32)
        v = g.standard_normal((L, Hkv * hs)).astype(np.float32)
        pos = np.arange(L)
        slots = (bt[s, pos // bs].astype(np.int64) * bs + pos % bs).astype(np.uint32)
        oracle_mod.bf16_cache_write(k, v, kb, vb, slots, Hkv, hs, bs)
    # the same stored values as an f32 cache: bfloat16 bits are the upper half of binary32
    kf = (kb.astype(np.uint32) << 16).view(np.float32).copy()
    vf = (vb.astype(np.uint32) << 16).view(np.float32).copy()
    q = g.standard_normal((S, H, hs)).astype(np.float32)
    lens_a = np.array(lens, np.uint32)
    got = oracle_mod.bf16_paged_decode(q, kb, vb, bt, lens_a, 0.2, Hkv, bs, max_context_len=mcl)
    want = oracle_mod.f32_paged_decode(q, kf, vf, bt, lens_a, 0.2, Hkv, bs, max_context_len=mcl)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    units = np.array([[2, 5], [0, 1], [1, 0]], np.uint32)
    gu = oracle_mod.bf16_paged_decode_units(units, q, kb, vb, bt, lens_a, 0.2, Hkv, bs, max_context_len=mcl)
    assert np.array_equal(gu, np.stack([got[s, h] for s, h in units]))
