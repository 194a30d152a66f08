"""GPU parity of q8_norm_rope_decode_step: the decode step with the per-head
RMSNorm + partial rotary step applied to q and to the new K rows at position
context_lens[s]-1, all in one launch.

Two references on the same seeded inputs:

* The HIP path's own unfused composition: q8_norm_rope on q and on the new K
  rows, then q8_decode_step on the results.  The fused kernel takes every
  value at the same binary32 rounding points in the same lane order, so
  outputs and both caches must match bit for bit.
* The oracle: norm_rope on q, norm_rope_cache_write of the new rows at the
  appended slots, then paged_decode, all on the oracle's rotary table (copied
  to the device, so both sides rotate with the same cos/sin).  Cache words are
  exact except in K rows whose r = 1/sqrt(mean + eps) lies near a binary32
  rounding boundary (where the GPU's lane-tree sum of squares may round it the
  other way: a code may move by 1 at a near-tie, the scale word by 2 ulps);
  outputs within 1e-4 + 1e-4*|oracle|.
"""
import os

import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def appended_slots(bt, lens, bs, mcl):
    """The slot of position L-1 of every sequence the step appends to
    (1 <= L <= max_context_len, table covering it); PAD for the others."""
    slots = np.full(len(lens), wl.PAD_SLOT, dtype=np.uint32)
    for s, L in enumerate(lens):
        L = int(L)
        if 1 <= L <= mcl and (L - 1) // bs < bt.shape[1]:
            slots[s] = np.uint32(int(bt[s, (L - 1) // bs]) * bs + (L - 1) % bs)
    return slots


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return bool(torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32)))


def offset_dev(a: np.ndarray):
    """A device copy of `a` starting 4 bytes past a 16-byte boundary."""
    from gpu_util import f32_dev
    flat = np.concatenate([np.zeros(1, np.float32), np.ascontiguousarray(a, np.float32).reshape(-1)])
    return f32_dev(flat)[1:].view(a.shape)


def run_case(oracle_mod, seed, S, H, Hkv, bs, lens, rot, hs=128, mcl=None, P=8192, eps=1e-6, theta=10000.0,
             q_layout="packed", misaligned_params=False, check_oracle=True):
    """q_layout: "packed" ([S, H, hs] rows), "interleave" (each head followed by
    head_size gate values: head stride 2*hs) or "offset" (packed rows starting
    4 bytes past 16-byte alignment, with a padded row stride)."""
    from int8_paged_kv_amd import q8_decode_step, q8_norm_rope, q8_norm_rope_decode_step
    from gpu_util import RandomCase, assert_close, f32_dev, nan_out, u32_dev, u32_host
    from test_gpu_norm_rope import compare_k_rows
    what = "norm-rope step %s" % ((S, H, Hkv, hs, bs, list(lens), rot, mcl, P, q_layout, misaligned_params),)
    print(what, flush=True)
    c = RandomCase(oracle_mod, seed, S, H, Hkv, hs, bs, lens)    # positions 0 .. L-1 hold older rows
    mcl = int(c.lens.max()) if mcl is None else mcl
    g = np.random.default_rng(seed + 2000)
    nk = (g.standard_normal((S, Hkv, hs)) * g.uniform(0.05, 30, (S, 1, 1))).astype(np.float32)
    nv = g.standard_normal((S, Hkv, hs)).astype(np.float32)
    qw = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    kw = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    tab_h = oracle_mod.rope_table(P, rot, theta) if rot else None
    put = offset_dev if misaligned_params else f32_dev
    tab_d = put(tab_h) if rot else None
    qw_d, kw_d = put(qw), put(kw)
    nk_d, nv_d = f32_dev(nk), f32_dev(nv)
    kc0, vc0 = c.kc_d.clone(), c.vc_d.clone()
    # q rows in the requested layout; q_h is the [S, H, hs] values
    q_h = c.q
    if q_layout == "interleave":
        rows = np.concatenate([q_h, 100.0 * g.standard_normal((S, H, hs)).astype(np.float32)], axis=2)
        q_store = f32_dev(rows)                                     # [S, H, 2*hs]: q then gate per head
        q_d, x_stride, head_stride = q_store[:, :, :hs], H * 2 * hs, 2 * hs
    elif q_layout == "offset":
        rows = np.concatenate([q_h.reshape(S, H * hs), np.zeros((S, 3), np.float32)], axis=1)   # stride H*hs + 3
        q_store = offset_dev(rows)
        q_d, x_stride, head_stride = q_store[:, :H * hs].unflatten(1, (H, hs)), H * hs + 3, hs
    else:
        q_d, x_stride, head_stride = c.q_d, H * hs, hs
        q_store = c.q_d

    out = q8_norm_rope_decode_step(q_d, nk_d, nv_d, c.kc_d, c.vc_d, c.bt_d, c.cl_d, c.scale, Hkv, bs, mcl,
                                   qw_d, kw_d, tab_d, rot, eps, out=nan_out(S, H, hs))
    # the unfused composition on the GPU; positions past the table are clamped
    # to its last row on both paths (a sequence with no positions has no q use)
    pos = np.minimum(np.maximum(c.lens.astype(np.int64) - 1, 0), P - 1).astype(np.uint32)
    pos_d = u32_dev(pos)
    qx = q_store.as_strided((S, x_stride), (x_stride, 1)) if q_layout != "packed" else q_store.reshape(S, H * hs)
    qn_d = q8_norm_rope(qx, pos_d, qw_d, tab_d, rot, eps, H, hs, head_stride=head_stride)
    kn_d = q8_norm_rope(nk_d.view(S, Hkv * hs), pos_d, kw_d, tab_d, rot, eps, Hkv, hs)
    ref = q8_decode_step(qn_d, kn_d, nv_d, kc0, vc0, c.bt_d, c.cl_d, c.scale, Hkv, bs, mcl,
                         out=nan_out(S, H, hs))
    torch.cuda.synchronize()
    assert bits_equal(c.kc_d, kc0), what + ": key cache differs from the unfused composition"
    assert bits_equal(c.vc_d, vc0), what + ": value cache differs from the unfused composition"
    assert bits_equal(out, ref), what + ": output differs from the unfused composition"
    if not check_oracle:
        return out
    qn_h = oracle_mod.norm_rope(q_h, pos, qw, tab_h, rot, eps, H, hs)
    slots = appended_slots(c.bt, c.lens, bs, mcl)
    kc_h, vc_h = c.kc.copy(), c.vc.copy()
    oracle_mod.norm_rope_cache_write(nk, nv, kc_h, vc_h, slots, pos, kw, tab_h, rot, eps, Hkv, hs, bs)
    wpt = hs // 4 + 1
    shape = (-1, Hkv, bs, wpt)
    got_k, got_v = u32_host(c.kc_d), u32_host(c.vc_d)
    assert np.array_equal(got_v, vc_h), what + ": value cache words differ from the oracle"
    compare_k_rows(oracle_mod, got_k.reshape(shape), kc_h.reshape(shape), nk, slots, pos, kw, tab_h, rot, Hkv,
                   hs, bs)
    want = oracle_mod.paged_decode(qn_h, kc_h, vc_h, c.bt, c.lens, c.scale, Hkv, bs, max_context_len=mcl)
    assert_close(out.cpu().numpy(), want, what)
    return out


@pytest.mark.parametrize("S,H,Hkv,hs,bs,lens,rot", [
    (5, 8, 2, 128, 16, [900, 65, 1, 2000, 300], 64),   # 4 query heads per kv head: 32-position chunks, 16-row tiles
    (4, 8, 2, 128, 32, [0, 130, 0, 64], 128),          # empty sequences; 32-row tiles; whole head rotated
    (3, 8, 2, 128, 64, [300, 129, 128], 32),           # blocks larger than a chunk
    (3, 16, 2, 128, 16, [333, 65, 64], 64),            # 8 query heads per kv head: 64-position chunks
    (3, 16, 2, 128, 32, [700, 1, 95], 0),              # no rotation
    (3, 16, 2, 128, 64, [200, 64, 257], 64),
    (3, 32, 2, 128, 16, [150, 40, 700], 64),           # 16 query heads per kv head
    (4, 4, 2, 128, 16, [90, 31, 200, 33], 64),         # 2 query heads in a group of 4: padded heads stay zero
    (3, 2, 2, 128, 16, [77, 160, 5], 64),              # one query head per kv head
    (3, 8, 2, 128, 8, [61, 12, 130], 64),              # block_size 8: the generic tiled layout
    (4, 8, 2, 64, 16, [500, 33, 0, 97], 32),           # head_size 64: 16 lanes per q head
    (3, 16, 2, 64, 32, [260, 64, 31], 64),             # head_size 64, whole head rotated
    (3, 32, 2, 64, 16, [129, 300, 2], 16),             # head_size 64, 16 query heads per kv head
    (3, 4, 2, 256, 16, [400, 63, 129], 64),            # head_size 256: 64 lanes per q head
    (3, 16, 2, 256, 32, [77, 300, 64], 128),           # head_size 256, 8 query heads per kv head
    (2, 2, 2, 256, 64, [500, 190], 256),               # head_size 256, one query head per kv head, all rotated
])
def test_norm_rope_step_shapes(oracle_mod, S, H, Hkv, hs, bs, lens, rot):
    run_case(oracle_mod, hash((S, H, Hkv, hs, bs, rot)) % 10000, S, H, Hkv, bs, lens, rot, hs=hs)


@pytest.mark.parametrize("hs,H,layout,misaligned", [
    (128, 8, "interleave", False),     # q and gate interleaved per head (head stride 2*head_size)
    (256, 4, "interleave", False),
    (64, 8, "interleave", True),
    (128, 16, "offset", False),        # q rows 4 bytes off 16-byte alignment: scalar q loads
    (128, 8, "packed", True),          # weights and table 4 bytes off alignment: scalar parameter loads
    (256, 8, "offset", True),
])
def test_norm_rope_step_layouts(oracle_mod, hs, H, layout, misaligned):
    run_case(oracle_mod, 60 + hs + H, 4, H, 2, 16, [300, 1, 129, 64], 32, hs=hs, q_layout=layout,
             misaligned_params=misaligned)


def test_norm_rope_step_eps_zero(oracle_mod):
    """eps == 0 with nonzero vectors; the padded query heads of a group (zero
    rows, whose r would be infinite) must not disturb the real ones."""
    run_case(oracle_mod, 91, 4, 4, 2, 16, [150, 40, 700, 1], 64, eps=0.0)


def test_norm_rope_step_clamped(oracle_mod):
    """Sequences longer than max_context_len attend their first positions and
    get no new row; their q rows are still rotated at context_lens[s]-1."""
    run_case(oracle_mod, 92, 3, 8, 2, 16, [500, 100, 300], 64, mcl=256)


def test_norm_rope_step_positions_past_table(oracle_mod):
    """Positions past the rotary table take its last row (the table's
    documented clamp), on the fused path as on q8_norm_rope."""
    run_case(oracle_mod, 93, 4, 8, 2, 16, [1500, 100, 999, 1000], 64, P=1000)


@pytest.mark.parametrize("waves", [7, 333, 4096])
def test_norm_rope_step_wavefront_boundaries(oracle_mod, waves):
    os.environ["Q8KV_DECODE_WAVES"] = str(waves)
    try:
        run_case(oracle_mod, 40 + waves, 13, 8, 2, 16, [0, 63, 64, 65, 255, 256, 257, 0, 1023, 1024, 1025, 2049, 1],
                 64)
    finally:
        os.environ.pop("Q8KV_DECODE_WAVES", None)


def test_norm_rope_step_many_sequences(oracle_mod):
    """More than 64 sequences (the cursor's table lookups instead of the
    one-load window), ragged lengths."""
    g = np.random.default_rng(94)
    lens = g.integers(0, 600, 150)
    lens[::17] = 0
    run_case(oracle_mod, 94, 150, 8, 2, 16, lens.tolist(), 64)


def test_norm_rope_step_unsupported_shapes():
    from int8_paged_kv_amd import Q8Error, q8_norm_rope_decode_step
    from gpu_util import f32_dev, u32_dev
    S, Hkv, bs = 2, 2, 16
    for H, hs in ((4, 96), (32, 256)):          # head_size 96; 16 query heads per kv head at head_size 256
        q = torch.zeros((S, H, hs), dtype=torch.float32, device="cuda:0")
        k = torch.zeros((S, Hkv * hs), dtype=torch.float32, device="cuda:0")
        kc = torch.zeros(4 * Hkv * bs * (hs // 4 + 1), dtype=torch.int32, device="cuda:0")
        w = f32_dev(np.ones(hs, np.float32))
        tab = f32_dev(np.ones((16, 32), np.float32))
        with pytest.raises(Q8Error) as e:
            q8_norm_rope_decode_step(q, k, k, kc, kc.clone(), u32_dev(np.zeros((S, 4), np.uint32)),
                                     u32_dev(np.array([3, 5], np.uint32)), 0.1, Hkv, bs, 64, w, w, tab, 32, 1e-6)
        assert e.value.status == 5


def test_norm_rope_step_full_size_llama(oracle_mod):
    """The Llama-3-8B-shaped batch of the step benchmark (S=64, H=32, Hkv=8,
    block_size 16, lengths U[512, 4096]) in the bench's launch configuration,
    with rot 64 over an 8192-position table: bit-exact against the unfused
    HIP composition, and the appended rows and every output against the oracle."""
    from int8_paged_kv_amd import q8_decode_step, q8_norm_rope, q8_norm_rope_decode_step
    from gpu_util import Filled, assert_close, f32_dev, nan_out, u32_dev, u32_host
    from test_gpu_norm_rope import compare_k_rows
    w = wl.llama()
    f = Filled(w, oracle_mod, with_step=False)
    slots, k, v = w.step_write()
    S, H, Hkv, hs, bs = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size, w.block_size
    rot, P, eps = hs // 2, 8192, 1e-6
    g = np.random.default_rng(12)
    kw = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    qw = (1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32)
    tab_h = oracle_mod.rope_table(P, rot, 10000.0)
    tab_d, qw_d, kw_d = f32_dev(tab_h), f32_dev(qw), f32_dev(kw)
    k_d, v_d = f32_dev(k), f32_dev(v)
    kc0, vc0 = f.kc_d.clone(), f.vc_d.clone()
    mcl = w.max_context_len
    out = q8_norm_rope_decode_step(f.q_d, k_d, v_d, f.kc_d, f.vc_d, f.bt_d, f.cl_d, w.scale, Hkv, bs, mcl,
                                   qw_d, kw_d, tab_d, rot, eps, out=nan_out(S, H, hs))
    pos = (np.minimum(w.context_lens.astype(np.int64), mcl) - 1).astype(np.uint32)
    pos_d = u32_dev(pos)
    qn_d = q8_norm_rope(f.q_d.reshape(S, H * hs), pos_d, qw_d, tab_d, rot, eps, H, hs)
    kn_d = q8_norm_rope(k_d.view(S, Hkv * hs), pos_d, kw_d, tab_d, rot, eps, Hkv, hs)
    ref = q8_decode_step(qn_d, kn_d, v_d, kc0, vc0, f.bt_d, f.cl_d, w.scale, Hkv, bs, mcl, out=nan_out(S, H, hs))
    torch.cuda.synchronize()
    assert bits_equal(f.kc_d, kc0) and bits_equal(f.vc_d, vc0), "caches differ from the unfused composition"
    assert bits_equal(out, ref), "output differs from the unfused composition"
    qn_h = oracle_mod.norm_rope(f.q, pos, qw, tab_h, rot, eps, H, hs)
    oracle_mod.norm_rope_cache_write(k, v, f.kc_h, f.vc_h, slots, pos, kw, tab_h, rot, eps, Hkv, hs, bs)
    shape = (-1, Hkv, bs, hs // 4 + 1)
    assert np.array_equal(u32_host(f.vc_d), f.vc_h), "value cache words differ from the oracle"
    compare_k_rows(oracle_mod, u32_host(f.kc_d).reshape(shape), f.kc_h.reshape(shape), k.reshape(S, Hkv, hs),
                   slots, pos, kw, tab_h, rot, Hkv, hs, bs)
    want = oracle_mod.paged_decode(qn_h, f.kc_h, f.vc_h, w.block_tables, w.context_lens, w.scale, Hkv, bs,
                                   max_context_len=mcl)
    assert_close(out.cpu().numpy(), want, "llama norm-rope step")
