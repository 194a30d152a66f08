"""The seeded workload generators produce inputs inside the caller contract (CPU only)."""
import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl


@pytest.mark.parametrize("name", sorted(wl.WORKLOADS))
def test_tables_slots_and_lists_are_in_contract(name):
    w = wl.get(name)
    S = w.num_seqs
    assert w.block_tables.shape[0] == S and w.block_tables.dtype == np.uint32
    assert w.num_heads % w.num_kv_heads == 0 and w.head_size % 4 == 0 and w.head_size <= 256
    used = []
    for s in range(S):
        n = -(-int(w.context_lens[s]) // w.block_size)
        assert n <= w.max_num_blocks_per_seq
        used.append(w.block_tables[s, :n])
    used = np.concatenate(used)
    assert used.max() < w.num_blocks
    assert np.unique(used).size == used.size          # no block shared between sequences
    slots = w.fill_slots()
    assert np.unique(slots).size == slots.size        # distinct slots within the fill
    assert slots.max() < w.num_blocks * w.block_size
    step = w.step_write()
    if step is not None:
        assert not np.isin(step[0], slots).any()
    if w.visible_pos is not None:
        assert np.all(w.num_visible <= w.vis_stride)
        for s in range(S):
            p = w.visible_pos[s, :w.num_visible[s]]
            assert np.all(np.diff(p.astype(np.int64)) > 0)
            assert p.max() < w.context_lens[s]
            assert np.array_equal(np.sort(w.fill_positions[s]), p)


def test_tiny_shapes_and_determinism():
    a, b = wl.tiny(), wl.tiny()
    assert np.array_equal(a.block_tables, b.block_tables)
    assert a.context_lens.tolist() == [37, 64]
    assert sorted(a.block_tables.reshape(-1).tolist()) == list(range(16))
    (s1, k1, v1), = list(a.fill_chunks())
    (s2, k2, v2), = list(b.fill_chunks())
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2) and k1.shape == (101, 2, 64)
    assert a.effective_kv_bytes() == 101 * 2 * 2 * 68


def test_llama_effective_bytes_near_expected():
    w = wl.llama()
    assert 512 <= w.context_lens.min() and w.context_lens.max() <= 4096
    assert w.step_write()[0].shape == (64,)
    # about 147k attended tokens: 311 MB of codes + scales
    assert 2.5e8 < w.effective_kv_bytes() < 3.7e8


def test_mha_write_pads_and_zero_vectors():
    w = wl.mha256()
    slots, k, v = wl.mha256_write(w)
    assert (slots == wl.PAD_SLOT).sum() == 410
    real = slots[slots != wl.PAD_SLOT]
    assert np.unique(real).size == real.size
    assert not np.isin(real, w.fill_slots()).any()
    for arr in (k, v):
        assert (np.abs(arr).max(axis=2) == 0).sum() == 328


def test_long_outlier_channels():
    w = wl.long_context()
    assert w.outlier_k.sum() == 20 and w.outlier_v.sum() == 20
    sl, k, v = next(w.fill_chunks(chunk_tokens=4096))
    big = np.abs(k[:, w.outlier_k]).mean()
    small = np.abs(k[:, ~w.outlier_k]).mean()
    assert 15 < big / small < 25
