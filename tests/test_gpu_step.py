"""GPU parity of q8_decode_step (each sequence's new K/V row appended at its
last position and attended, in one launch) against the oracle's cache write
of those rows followed by its decode: cache words bit-exact over the whole
caches, outputs within 1e-4 + 1e-4*|oracle| (no NaN anywhere)."""
import os

import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def appended_slots(bt, lens, bs, mcl):
    """The slot of position L-1 of every sequence that the step appends to
    (1 <= L <= max_context_len, table covering it); PAD for the others."""
    slots = np.full(len(lens), wl.PAD_SLOT, dtype=np.uint32)
    for s, L in enumerate(lens):
        L = int(L)
        if 1 <= L <= mcl and (L - 1) // bs < bt.shape[1]:
            slots[s] = np.uint32(int(bt[s, (L - 1) // bs]) * bs + (L - 1) % bs)
    return slots


def run_step_case(oracle_mod, seed, S, H, Hkv, hs, bs, lens, mcl=None, **kw):
    from int8_paged_kv_amd import q8_decode_step
    from gpu_util import RandomCase, assert_close, f32_dev, nan_out, u32_host
    c = RandomCase(oracle_mod, seed, S, H, Hkv, hs, bs, lens)     # positions 0 .. L-1 hold older rows
    mcl = int(c.lens.max()) if mcl is None else mcl
    g = np.random.default_rng(seed + 1000)
    nk = g.standard_normal((S, Hkv, hs)).astype(np.float32)
    nv = g.standard_normal((S, Hkv, hs)).astype(np.float32)
    nk[:, :, 5] *= 30                      # a large entry sets amax
    out = q8_decode_step(c.q_d, f32_dev(nk), f32_dev(nv), c.kc_d, c.vc_d, c.bt_d, c.cl_d, c.scale, Hkv, bs,
                         mcl, out=nan_out(S, H, hs), **kw)
    torch.cuda.synchronize()
    slots = appended_slots(c.bt, c.lens, bs, mcl)
    oracle_mod.cache_write(nk, nv, c.kc, c.vc, slots, Hkv, hs, bs)
    assert np.array_equal(u32_host(c.kc_d), c.kc), "key cache words differ"
    assert np.array_equal(u32_host(c.vc_d), c.vc), "value cache words differ"
    want = oracle_mod.paged_decode(c.q, c.kc, c.vc, c.bt, c.lens, c.scale, Hkv, bs, max_context_len=mcl)
    assert_close(out.cpu().numpy(), want, "step %s" % ((S, H, Hkv, hs, bs, list(lens), mcl),))


@pytest.mark.parametrize("S,H,Hkv,hs,bs,lens", [
    (5, 8, 2, 128, 16, [900, 65, 1, 2000, 300]),     # new row opening a chunk, one-token sequence
    (4, 8, 2, 128, 16, [0, 130, 0, 64]),             # empty sequences append nothing; last row of a chunk
    (3, 32, 2, 64, 16, [150, 40, 700]),              # n_rep 16: two query-head groups share the new row
    (3, 4, 2, 68, 16, [90, 31, 200]),                # head_size 68 (padded lane layout)
    (3, 4, 2, 128, 5, [61, 12, 130]),                # block_size 5: row gather
    (3, 4, 2, 128, 128, [300, 129, 128]),            # block larger than a chunk
    (2, 8, 1, 256, 16, [333, 70]),                   # head_size 256
    (3, 16, 2, 128, 32, [333, 65, 64]),              # n_rep 8
])
def test_step_shapes(oracle_mod, S, H, Hkv, hs, bs, lens):
    run_step_case(oracle_mod, hash((S, H, Hkv, hs, bs)) % 10000, S, H, Hkv, hs, bs, lens)


def test_step_clamped_sequences_are_not_appended(oracle_mod):
    """A sequence longer than max_context_len attends its first positions and
    gets no new row."""
    run_step_case(oracle_mod, 77, 3, 8, 2, 128, 16, [500, 100, 300], mcl=256)


@pytest.mark.parametrize("waves", [7, 333, 4096])
def test_step_wavefront_boundaries(oracle_mod, waves):
    os.environ["Q8KV_DECODE_WAVES"] = str(waves)
    try:
        run_step_case(oracle_mod, 40 + waves, 13, 8, 2, 128, 16,
                      [0, 63, 64, 65, 255, 256, 257, 0, 1023, 1024, 1025, 2049, 1])
    finally:
        os.environ.pop("Q8KV_DECODE_WAVES", None)


def test_step_full_size_llama(oracle_mod):
    """The Llama-3-8B-shaped batch in the launch configuration the bench
    times: caches filled up to L-1, then one step appends at L-1 and attends;
    both caches bit-exact, every output against the oracle."""
    from int8_paged_kv_amd import q8_decode_step
    from gpu_util import Filled, assert_close, f32_dev, nan_out, u32_host, u32_dev
    w = wl.llama()
    f = Filled(w, oracle_mod, with_step=False)
    slots, k, v = w.step_write()
    assert np.array_equal(slots, appended_slots(w.block_tables, w.context_lens, w.block_size, w.max_context_len))
    out = q8_decode_step(f.q_d, f32_dev(k), f32_dev(v), f.kc_d, f.vc_d, f.bt_d, f.cl_d, w.scale, w.num_kv_heads,
                         w.block_size, w.max_context_len, out=nan_out(w.num_seqs, w.num_heads, w.head_size))
    torch.cuda.synchronize()
    oracle_mod.cache_write(k, v, f.kc_h, f.vc_h, slots, w.num_kv_heads, w.head_size, w.block_size)
    assert np.array_equal(u32_host(f.kc_d), f.kc_h), "key cache words differ"
    assert np.array_equal(u32_host(f.vc_d), f.vc_h), "value cache words differ"
    assert_close(out.cpu().numpy(), f.decode_oracle(oracle_mod), "llama step")
