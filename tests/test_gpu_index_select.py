"""GPU parity of q8_index_select against the oracle: visible lists and counts are
index work, so they must be identical, entry by entry (ties resolved to the
lower block index on both sides); entries past a row's count stay untouched.
The selected-token workload's lists are then rebuilt from block scores and fed
to the visible-list decode."""
import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 0xDEADBEEF


def run_select(oracle_mod, scores, lens, ratio, k, vis_stride, mask_stride=0):
    """With mask_stride > 0 the block bitmask is requested too; every mask word
    is written, so the sentinel must be gone from all of them."""
    from int8_paged_kv_amd import q8_index_select
    from gpu_util import f32_dev, u32_dev, u32_host
    R = lens.shape[0]
    vis_d = u32_dev(np.full((R, vis_stride), SENTINEL, np.uint32))
    nv_d = u32_dev(np.full(R, SENTINEL, np.uint32))
    mask_d = u32_dev(np.full((R, mask_stride), SENTINEL, np.uint32)) if mask_stride else None
    q8_index_select(f32_dev(scores), u32_dev(lens), ratio, k, vis_stride, visible_pos=vis_d, num_visible=nv_d,
                    mask_stride=mask_stride, visible_mask=mask_d)
    torch.cuda.synchronize()
    vis, nv = u32_host(vis_d), u32_host(nv_d)
    want = oracle_mod.index_select(scores, lens, ratio, k, vis_stride, mask_stride=mask_stride)
    want_vis, want_nv = want[0], want[1]
    assert np.array_equal(nv, want_nv), "visible counts differ"
    for r in range(R):
        n = int(want_nv[r])
        assert np.array_equal(vis[r, :n], want_vis[r, :n]), "row %d: visible lists differ" % r
        assert np.all(vis[r, n:] == SENTINEL), "row %d: entries past the count were written" % r
    if mask_stride:
        mask = u32_host(mask_d)
        bad = np.nonzero(np.any(mask != want[2], axis=1))[0]
        assert bad.size == 0, "block bitmasks differ in rows %s" % bad[:8].tolist()
    return vis, nv


@pytest.mark.parametrize("ratio,k,max_blocks,kind", [
    (64, 32, 1024, "normal"),
    (64, 32, 1024, "ties"),
    (16, 5, 300, "ties"),
    (4, 1, 50, "ties"),
    (1, 3, 16384, "normal"),       # the largest row the kernel holds
    (1, 200, 16384, "ties"),
    (8, 0, 40, "normal"),          # selective rows keep only their tail
    (32, 7, 64, "zeros"),          # every score +-0: ties decided by index alone
])
def test_matches_oracle(oracle_mod, ratio, k, max_blocks, kind):
    g = np.random.default_rng(ratio * 1000 + k + max_blocks)
    R = 24
    if kind == "normal":
        scores = g.standard_normal((R, max_blocks)).astype(np.float32)
    elif kind == "ties":
        scores = g.integers(-2, 3, (R, max_blocks)).astype(np.float32)
    else:
        scores = np.where(g.random((R, max_blocks)) < 0.5, -0.0, 0.0).astype(np.float32)
    top = max_blocks * ratio + ratio - 1
    lens = g.integers(0, top + 1, R).astype(np.uint32)
    lens[:6] = [0, ratio - 1, k * ratio, k * ratio + ratio - 1, (k + 1) * ratio, top]   # edges of the dense case
    run_select(oracle_mod, scores, lens, ratio, k, k * ratio + ratio)
    # the bitmask too, one spare word past the widest row
    run_select(oracle_mod, scores, lens, ratio, k, k * ratio + ratio, (max_blocks + 1 + 31) // 32 + 1)


@pytest.mark.parametrize("max_blocks", [255, 256, 257, 1023, 1024, 1025, 2049])
def test_mask_at_chunk_edges(oracle_mod, max_blocks):
    """Rows whose trailing block is the first block past a scan chunk (1024
    blocks), the last one inside it, or a word or wave edge; every row selective."""
    g = np.random.default_rng(max_blocks)
    ratio, k = 4, 9
    R = 20
    scores = g.standard_normal((R, max_blocks)).astype(np.float32)
    lens = np.array([b * ratio + t for b in (max_blocks, max_blocks - 1, 2048, 1024, 1023, 256, 255, 224, 32, 31, 40)
                     for t in (0, 3) if b <= max_blocks], np.uint32)[:R]
    lens = np.resize(lens, R).astype(np.uint32)
    run_select(oracle_mod, scores, lens, ratio, k, k * ratio + ratio, (max_blocks + 1 + 31) // 32)


def test_rebuilds_selected_workload_and_decodes(oracle_mod):
    """Scores that rank each sequence's 32 visible blocks first reproduce the
    selected-token workload's lists; the decode over them matches the oracle."""
    from gpu_util import Filled, assert_close, u32_dev
    from int8_paged_kv_amd import q8_paged_decode
    w = wl.selected()
    ratio, k = 64, 32
    vis_stride = w.visible_pos.shape[1]
    g = np.random.default_rng(55)
    nblocks = int(w.context_lens.max()) // ratio
    scores = (g.random((w.num_seqs, nblocks)) * 0.5).astype(np.float32)
    for s in range(w.num_seqs):
        n = int(w.num_visible[s])
        blocks = np.unique(w.visible_pos[s, :n] // ratio)[:k]
        scores[s, blocks] = 1.0 + g.random(k).astype(np.float32)
    vis, nv = run_select(oracle_mod, scores, w.context_lens.astype(np.uint32), ratio, k, vis_stride)
    for s in range(w.num_seqs):
        n = int(w.num_visible[s])
        assert nv[s] == n and np.array_equal(vis[s, :n], w.visible_pos[s, :n])
    f = Filled(w, oracle_mod)
    out = q8_paged_decode(f.q_d, f.kc_d, f.vc_d, u32_dev(w.block_tables), u32_dev(w.context_lens), w.scale,
                          w.num_kv_heads, w.block_size, visible_pos=u32_dev(vis), num_visible=u32_dev(nv))
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), f.decode_oracle(oracle_mod), "decode over the selected lists")
