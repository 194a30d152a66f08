"""Pins of the oracle's block selection into a visible list (CPU only).

The "attention.rs" page fixes the list's shape in its per-row decode loop:
t_len = base_pos + b + 1, blocks = t_len / ratio, a row is selective when
blocks > kblk (= budget / ratio) and then attends kblk*ratio + (t_len -
blocks*ratio) positions, else all t_len; lists sit vis_stride = budget + ratio
apart.  The select kernel is not printed; the reading is a top-kblk of the
complete blocks by score (ties to the lower index), positions ascending, then
the trailing incomplete block.  Pinned by a hand-worked example, by a
sort-based brute force on small inputs full of ties, by the page's n_vis
formula, and by the invariants any such list must have.
"""
import numpy as np
import pytest

import oracle


def test_hand_example_with_ties_and_tail():
    # blocks of 4 positions; scores 3, 1, 5, 5, 0 and a 2-position tail; keep 2 blocks
    vis, nv = oracle.index_select(np.array([[3, 1, 5, 5, 0]], np.float32), np.array([22]), 4, 2, 12)
    assert nv[0] == 10
    assert vis[0, :10].tolist() == [8, 9, 10, 11, 12, 13, 14, 15, 20, 21]
    # three-way tie for the second place: the lowest index among the tied wins
    vis, nv = oracle.index_select(np.array([[2, 7, 2, 2]], np.float32), np.array([16]), 4, 2, 12)
    assert vis[0, :nv[0]].tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    # signed zeros compare equal: a tie, decided by index
    vis, nv = oracle.index_select(np.array([[-0.0, 0.0, -1.0]], np.float32), np.array([12]), 4, 1, 8)
    assert vis[0, :nv[0]].tolist() == [0, 1, 2, 3]


def brute(scores, t_len, ratio, k):
    blocks = t_len // ratio
    order = sorted(range(blocks), key=lambda j: (-float(scores[j]), j))
    keep = sorted(order[:k])
    return [j * ratio + p for j in keep for p in range(ratio)] + list(range(blocks * ratio, t_len))


@pytest.mark.parametrize("ratio,k", [(1, 3), (4, 2), (16, 5), (64, 32)])
def test_brute_force_with_many_ties(ratio, k):
    g = np.random.default_rng(ratio * 100 + k)
    R = 40
    max_blocks = 3 * k + 7
    scores = g.integers(-3, 4, (R, max_blocks)).astype(np.float32)     # few distinct values: many ties
    lens = g.integers(0, max_blocks * ratio + ratio, R).astype(np.uint32)
    lens = np.minimum(lens, max_blocks * ratio + ratio - 1)
    vis, nv = oracle.index_select(scores, lens, ratio, k, k * ratio + ratio)
    for r in range(R):
        assert vis[r, :nv[r]].tolist() == brute(scores[r], int(lens[r]), ratio, k)


@pytest.mark.parametrize("ratio,k", [(64, 32), (16, 4)])
def test_visible_count_follows_the_page(ratio, k):
    g = np.random.default_rng(7)
    R = 200
    lens = g.integers(0, 4 * k * ratio, R).astype(np.uint32)
    scores = g.standard_normal((R, 4 * k)).astype(np.float32)
    vis, nv = oracle.index_select(scores, lens, ratio, k, k * ratio + ratio)
    for r in range(R):
        t_len = int(lens[r])
        blocks = t_len // ratio
        want = k * ratio + (t_len - blocks * ratio) if blocks > k else t_len
        assert nv[r] == want
        lst = vis[r, :nv[r]]
        if blocks <= k:
            assert lst.tolist() == list(range(t_len))               # dense: every position
        assert np.all(np.diff(lst.astype(np.int64)) > 0)              # ascending, distinct
        assert np.all(lst < t_len)
        assert lst[nv[r] - (t_len - blocks * ratio):].tolist() == list(range(blocks * ratio, t_len))  # the tail
        full = lst[:nv[r] - (t_len - blocks * ratio)].reshape(-1, ratio)
        assert np.all(full[:, 0] % ratio == 0) and np.all(np.diff(full, axis=1) == 1)   # whole blocks
        chosen = set((full[:, 0] // ratio).tolist())
        rest = [j for j in range(blocks) if j not in chosen]
        if chosen and rest:                                          # a top-k by score
            assert min(scores[r, j] for j in chosen) >= max(scores[r, j] for j in rest)


def test_out_of_contract_rejected():
    with pytest.raises(Exception):
        oracle.index_select(np.zeros((1, 8), np.float32), np.array([20]), 4, 2, 11)    # vis_stride < (k+1)*ratio
    with pytest.raises(Exception):
        oracle.index_select(np.array([[1, np.nan, 2]], np.float32), np.array([12]), 4, 1, 8)
    with pytest.raises(Exception):
        oracle.index_select(np.zeros((1, 2), np.float32), np.array([12]), 4, 1, 8)     # 3 blocks, 2 scores


def brute_mask(scores, t_len, ratio, k, words):
    """Bit j set for each kept complete block j and for the trailing block."""
    blocks = t_len // ratio
    keep = sorted(range(blocks), key=lambda j: (-float(scores[j]), j))[:k]
    bits = set(keep) | ({blocks} if t_len % ratio else set())
    m = [0] * words
    for j in bits:
        m[j // 32] |= 1 << (j % 32)
    return m


def test_mask_hand_example():
    # blocks 2 and 3 kept, positions 20..21 of block 5 as the tail: bits 2, 3, 5
    _, _, m = oracle.index_select(np.array([[3, 1, 5, 5, 0]], np.float32), np.array([22]), 4, 2, 12, mask_stride=2)
    assert m[0].tolist() == [0b101100, 0]
    # dense row (3 complete blocks <= k = 4) with a tail: blocks 0..3
    _, _, m = oracle.index_select(np.zeros((1, 4), np.float32), np.array([13]), 4, 4, 20, mask_stride=1)
    assert m[0].tolist() == [0b1111]
    # empty row: no bits, every word still written
    _, _, m = oracle.index_select(np.zeros((1, 4), np.float32), np.array([0]), 4, 1, 8, mask_stride=3)
    assert m[0].tolist() == [0, 0, 0]


@pytest.mark.parametrize("ratio,k,max_blocks", [(1, 40, 127), (4, 2, 13), (64, 32, 100)])
def test_mask_brute_force_across_words(ratio, k, max_blocks):
    g = np.random.default_rng(ratio * 7 + k)
    R = 30
    words = (max_blocks + 1 + 31) // 32
    scores = g.integers(-3, 4, (R, max_blocks)).astype(np.float32)
    lens = g.integers(0, max_blocks * ratio + ratio, R).astype(np.uint32)
    _, nv, m = oracle.index_select(scores, lens, ratio, k, k * ratio + ratio, mask_stride=words)
    for r in range(R):
        assert m[r].tolist() == brute_mask(scores[r], int(lens[r]), ratio, k, words)
        # popcount * ratio covers the list: whole blocks plus at most one partial one
        pc = sum(bin(int(w)).count("1") for w in m[r])
        assert pc == -(-int(nv[r]) // ratio)


def test_mask_too_narrow_rejected():
    with pytest.raises(Exception):    # the tail block 32 needs a second word
        oracle.index_select(np.zeros((1, 40), np.float32), np.array([32 * 4 + 1]), 4, 40, 164, mask_stride=1)
