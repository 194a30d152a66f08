"""GPU checks of libq8kv_debug.so, the build with device-side content checks
(Q8_DEBUG_BOUNDS): on valid inputs it raises no flag and gives the release
library's results bit for bit; each broken caller contract raises its flag.
Every kernel still clamps reads into the cache and skips writes past it, so
the broken inputs here stay in bounds on the device."""
import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SLOT, BLOCK, TABLE, VISIBLE = 1, 2, 4, 8


@pytest.fixture
def debug_lib():
    from int8_paged_kv_amd import _binding
    prev = _binding.use_library(_binding.load_debug_library())
    _binding.bounds_flags(clear=True)
    yield _binding
    _binding.bounds_flags(clear=True)
    _binding.use_library(prev)


def test_valid_inputs_raise_nothing_and_match_release(oracle_mod, debug_lib):
    from gpu_util import RandomCase
    g = np.random.default_rng(81)
    cases = [RandomCase(oracle_mod, 8101, 5, 32, 8, 128, 16, [900, 0, 65, 1, 2500]),
             RandomCase(oracle_mod, 8102, 3, 8, 8, 256, 16, [300, 17, 64]),
             RandomCase(oracle_mod, 8103, 2, 16, 2, 128, 32, [700, 90]),
             RandomCase(oracle_mod, 8104, 2, 4, 2, 64, 5, [61, 12])]
    outs_dbg = [c.gpu() for c in cases]
    c = cases[0]
    vis = np.zeros((c.S, 700), np.uint32)
    nvis = np.zeros(c.S, np.uint32)
    for s, L in enumerate(c.lens):
        n = min(int(L), 700)
        vis[s, :n] = np.sort(g.choice(int(L), n, replace=False)) if n else []
        nvis[s] = n
    outs_dbg.append(c.gpu(vis=vis, nvis=nvis))
    assert debug_lib.bounds_flags() == 0
    prev = debug_lib.use_library(None)          # the release library for the next calls
    try:
        outs_rel = [cc.gpu() for cc in cases] + [c.gpu(vis=vis, nvis=nvis)]
    finally:
        debug_lib.use_library(prev)
    for a, b in zip(outs_dbg, outs_rel):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_slot_past_the_cache(oracle_mod, debug_lib):
    from gpu_util import f32_dev, u32_dev, u32_host
    from int8_paged_kv_amd import q8_cache_write
    g = np.random.default_rng(82)
    T, hkv, hs, bs, nb = 20, 2, 64, 16, 4
    k = g.standard_normal((T, hkv, hs)).astype(np.float32)
    v = g.standard_normal((T, hkv, hs)).astype(np.float32)
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    slots[5] = nb * bs + 3                     # past the cache, not the pad value
    kh, vh = wl.poison_cache(nb, hkv, bs, hs), wl.poison_cache(nb, hkv, bs, hs)
    kd, vd = u32_dev(kh), u32_dev(vh)
    q8_cache_write(f32_dev(k), f32_dev(v), kd, vd, u32_dev(slots), hkv, hs, bs)
    assert debug_lib.bounds_flags() == SLOT
    ok = np.ones(T, bool)
    ok[5] = False
    oracle_mod.cache_write(k[ok], v[ok], kh, vh, slots[ok], hkv, hs, bs)
    assert np.array_equal(u32_host(kd), kh) and np.array_equal(u32_host(vd), vh)   # nothing written for it


def test_block_id_past_the_cache(oracle_mod, debug_lib):
    from gpu_util import RandomCase, u32_dev
    c = RandomCase(oracle_mod, 8201, 2, 8, 2, 128, 16, [300, 100])
    bt = c.bt.copy()
    bt[1, 2] = c.num_blocks + 5                # attended position 32..47 of sequence 1
    c.bt_d = u32_dev(bt)
    c.gpu()
    assert debug_lib.bounds_flags() & BLOCK


def test_positions_past_the_table_row(oracle_mod, debug_lib):
    from gpu_util import RandomCase, u32_dev
    c = RandomCase(oracle_mod, 8301, 2, 8, 2, 128, 16, [300, 100])
    lens = c.lens.copy()
    lens[1] = c.max_nb * c.bs + 40             # more positions than the row has blocks for
    c.cl_d = u32_dev(lens)
    c.gpu(max_context_len=int(lens.max()))
    assert debug_lib.bounds_flags() & TABLE


def test_visible_list_contracts(oracle_mod, debug_lib):
    from gpu_util import RandomCase
    c = RandomCase(oracle_mod, 8401, 2, 8, 2, 128, 16, [600, 300])
    vis = np.zeros((c.S, 200), np.uint32)
    nvis = np.array([150, 120], np.uint32)
    vis[0, :150] = np.arange(150)              # 0..149: tile runs, ascending
    vis[1, :120] = np.sort(np.random.default_rng(5).choice(300, 120, replace=False))
    c.gpu(vis=vis, nvis=nvis)
    assert debug_lib.bounds_flags() == 0
    bad = vis.copy()
    bad[1, [10, 11]] = bad[1, [11, 10]]        # two positions swapped: not ascending
    c.gpu(vis=bad, nvis=nvis)
    assert debug_lib.bounds_flags() & VISIBLE
    bad = vis.copy()
    bad[0, 64:128] = np.arange(64, 128)[::-1]  # a chunk of the right endpoints, not ascending inside
    bad[0, 64], bad[0, 127] = 64, 127
    c.gpu(vis=bad, nvis=nvis)
    assert debug_lib.bounds_flags() & VISIBLE
    c.gpu(vis=vis, nvis=np.array([150, 250], np.uint32))      # past vis_stride
    assert debug_lib.bounds_flags() & VISIBLE


def test_step_append_block_past_the_cache(oracle_mod, debug_lib):
    from gpu_util import RandomCase, f32_dev, u32_dev, u32_host
    from int8_paged_kv_amd import q8_decode_step
    c = RandomCase(oracle_mod, 8501, 2, 8, 2, 128, 16, [300, 100])
    bt = c.bt.copy()
    bt[1, (100 - 1) // 16] = c.num_blocks + 9  # the block of sequence 1's new (last) position
    g = np.random.default_rng(85)
    nk = g.standard_normal((2, 2, 128)).astype(np.float32)
    nv = g.standard_normal((2, 2, 128)).astype(np.float32)
    before = u32_host(c.kc_d).copy()
    q8_decode_step(c.q_d, f32_dev(nk), f32_dev(nv), c.kc_d, c.vc_d, u32_dev(bt), c.cl_d, c.scale, 2, 16, 300)
    assert debug_lib.bounds_flags() & BLOCK
    after = u32_host(c.kc_d)
    # sequence 0's new row was written; nothing else changed (no clamped write into another block)
    changed = np.nonzero(np.any(after != before, axis=-1))
    rows = set(zip(*changed))
    p = 300 - 1
    assert rows <= {(int(c.bt[0, p // 16]), h, p % 16) for h in range(2)}
