"""GPU parity of q8_paged_decode against the oracle, element by element:
|gpu - oracle| <= 1e-4 + 1e-4*|oracle| on every output (no NaN anywhere), plus
exact closed forms and bit-identical invariances of the HIP path itself."""
import os

import numpy as np
import pytest

from int8_paged_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture
def decode_waves():
    """Force the planner's persistent wavefront count for one test, which moves
    every boundary between wavefronts' chunk ranges."""
    def set_(n):
        os.environ["Q8KV_DECODE_WAVES"] = str(n)
    yield set_
    os.environ.pop("Q8KV_DECODE_WAVES", None)


def test_tiny_workload(oracle_mod):
    from gpu_util import Filled, assert_close
    f = Filled(wl.tiny(), oracle_mod)
    assert_close(f.decode_gpu(), f.decode_oracle(oracle_mod), "tiny")


@pytest.mark.parametrize("S,H,Hkv,hs,bs,lens", [
    (3, 4, 2, 64, 16, [0, 1, 17]),              # empty, one token, partial block
    (2, 4, 2, 64, 16, [0, 0]),                  # nothing to attend anywhere: zero rows
    (2, 8, 8, 128, 16, [100, 33]),              # MHA (n_rep 1)
    (2, 4, 2, 128, 16, [300, 64]),              # n_rep 2
    (2, 6, 2, 128, 16, [129, 70]),              # n_rep 3
    (2, 10, 2, 128, 16, [90, 200]),             # n_rep 5: one group of 8, three slots unused
    (2, 16, 2, 128, 32, [333, 65]),             # n_rep 8
    (2, 32, 2, 64, 16, [150, 40]),              # n_rep 16: two groups of 8
    (2, 4, 1, 4, 16, [50, 3]),                  # head_size 4
    (2, 4, 2, 68, 16, [90, 31]),                # head_size 68 (padded lane layout)
    (2, 4, 2, 192, 16, [77, 130]),              # head_size 192
    (2, 4, 2, 256, 16, [200, 5]),               # head_size 256
    (2, 4, 2, 128, 1, [40, 9]),                 # block_size 1: row gather path
    (2, 4, 2, 128, 5, [61, 12]),                # block_size 5: row gather path
    (2, 4, 2, 64, 8, [100, 7]),
    (2, 4, 2, 128, 64, [200, 64]),
    (2, 4, 2, 128, 128, [300, 129]),            # block larger than a chunk
])
def test_shapes_and_paths(oracle_mod, S, H, Hkv, hs, bs, lens):
    from gpu_util import RandomCase, assert_close
    c = RandomCase(oracle_mod, hash((S, H, Hkv, hs, bs)) % 10000, S, H, Hkv, hs, bs, lens)
    assert_close(c.gpu(), c.oracle(oracle_mod), "shape %s" % ((S, H, Hkv, hs, bs, lens),))


@pytest.mark.parametrize("waves", [1, 7, 64, 84, 86, 88, 333, 4096])
def test_wavefront_range_boundaries(oracle_mod, decode_waves, waves):
    """Chunk ranges of the persistent wavefronts: one wave for everything,
    waves spanning several sequences (and empty ones), sequences split over
    many waves, and one chunk per wave.  These lengths make 100 chunks in 11
    non-empty sequences per row group (2 row groups), 477 weighted cost units:
    84 and 86 waves leave 11.4 and 11.1 units per wave (weighted split), 88
    leave 10.8 (chunks alone)."""
    from gpu_util import RandomCase, assert_close
    lens = [0, 63, 64, 65, 255, 256, 257, 0, 1023, 1024, 1025, 2049, 1]
    decode_waves(waves)
    c = RandomCase(oracle_mod, 5 + waves, len(lens), 8, 2, 128, 16, lens, outliers=True)
    assert_close(c.gpu(), c.oracle(oracle_mod), "waves %d" % waves)


@pytest.mark.parametrize("waves", [2, 3, 5, 8, 64, 4096])
def test_empty_sequences_at_range_boundaries(oracle_mod, decode_waves, waves):
    """Empty sequences between two non-empty ones whose chunks fall in
    different wavefronts' ranges, at the start, and at the end: every one of
    them gets zero rows (the output starts as NaN)."""
    from gpu_util import RandomCase, assert_close
    lens = [0, 64, 0, 0, 64, 0, 130, 0, 1, 0, 0, 64, 0]
    decode_waves(waves)
    c = RandomCase(oracle_mod, 90 + waves, len(lens), 8, 2, 128, 16, lens)
    assert_close(c.gpu(), c.oracle(oracle_mod), "waves %d" % waves)


def test_context_clamp_and_q_stride(oracle_mod):
    from gpu_util import RandomCase, assert_close
    c = RandomCase(oracle_mod, 21, 3, 8, 2, 128, 16, [500, 90, 260], q_pad=24)
    assert_close(c.gpu(max_context_len=200), c.oracle(oracle_mod, max_context_len=200), "clamp")


def test_one_token_returns_dequantized_v_exactly(oracle_mod):
    from gpu_util import RandomCase
    c = RandomCase(oracle_mod, 22, 4, 8, 2, 128, 16, [1, 1, 1, 1])
    got = c.gpu()
    for s in range(c.S):
        for h in range(c.H):
            row = c.vc[c.bt[s, 0], h // 4, 0]
            want = row[:32].copy().view(np.int8).astype(np.float32) * row[32:33].copy().view(np.float32)
            assert np.array_equal(got[s, h], want), (s, h)


@pytest.mark.parametrize("kind", ["dense_list", "aligned_runs", "gaps", "empty_and_single"])
def test_visible_lists(oracle_mod, kind, decode_waves):
    from gpu_util import RandomCase, assert_close
    lens = [3000, 1500, 777]
    c = RandomCase(oracle_mod, 31, 3, 8, 2, 128, 16, lens)
    g = np.random.default_rng(32)
    stride = 3000
    vis = np.zeros((3, stride), np.uint32)
    nvis = np.zeros(3, np.uint32)
    for s, L in enumerate(lens):
        if kind == "dense_list":
            p = np.arange(L)
        elif kind == "aligned_runs":
            nb64 = L // 64
            b = np.sort(g.choice(nb64, size=min(8, nb64), replace=False))
            p = np.concatenate([(b[:, None] * 64 + np.arange(64)).reshape(-1), np.arange(nb64 * 64, L)])
        elif kind == "gaps":
            p = np.sort(g.choice(L, size=L // 3, replace=False))
        else:
            p = np.array([], dtype=np.int64) if s == 0 else np.array([L - 1])
        vis[s, :p.size] = p
        nvis[s] = p.size
    if kind == "gaps":
        decode_waves(37)
    got = c.gpu(vis=vis, nvis=nvis)
    assert_close(got, c.oracle(oracle_mod, vis=vis, nvis=nvis), kind)
    if kind == "dense_list":
        assert_close(got, c.gpu(), "visible [0, L) vs dense")


def test_determinism_and_block_relabel(oracle_mod):
    """Repeated calls are bit-identical; moving blocks to other physical ids
    (with consistent tables) does not change a single bit."""
    from gpu_util import RandomCase, u32_dev
    c = RandomCase(oracle_mod, 41, 4, 16, 2, 128, 16, [900, 64, 1, 2000], spare_blocks=9)
    a = c.gpu()
    assert np.array_equal(a, c.gpu())
    perm = np.random.default_rng(42).permutation(c.num_blocks + 1)
    kc2, vc2 = np.empty_like(c.kc), np.empty_like(c.vc)
    kc2[perm], vc2[perm] = c.kc, c.vc
    c.kc_d, c.vc_d = u32_dev(kc2), u32_dev(vc2)
    c.bt_d = u32_dev(perm[c.bt].astype(np.uint32))
    assert np.array_equal(a, c.gpu())


def test_gqa_equals_duplicated_mha(oracle_mod):
    from gpu_util import RandomCase, u32_dev
    c = RandomCase(oracle_mod, 51, 2, 8, 2, 128, 16, [700, 300])
    a = c.gpu()
    c.kc_d, c.vc_d = u32_dev(np.repeat(c.kc, 4, axis=1)), u32_dev(np.repeat(c.vc, 4, axis=1))
    c.Hkv = 8
    b = c.gpu()
    assert np.all(np.abs(a - b) <= 1e-6 + 1e-6 * np.abs(a))


def test_workspace_reuse_leaves_counters_zero(oracle_mod, decode_waves):
    """One zero-filled workspace serves several calls of different shapes:
    every call is correct and leaves the arrival counters at zero."""
    from int8_paged_kv_amd import q8_paged_decode_workspace_bytes
    from gpu_util import RandomCase, assert_close
    decode_waves(96)
    cases = [RandomCase(oracle_mod, 71, 5, 8, 2, 128, 16, [900, 65, 0, 2000, 300]),
             RandomCase(oracle_mod, 72, 3, 16, 2, 64, 16, [1500, 10, 700]),
             RandomCase(oracle_mod, 73, 5, 8, 2, 128, 16, [130, 1200, 64, 640, 3])]
    need = max(q8_paged_decode_workspace_bytes(c.S, c.H, c.Hkv, c.hs, c.bs, int(c.lens.max())) for c in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    for i, c in enumerate(cases * 2):
        assert_close(c.gpu(workspace=ws), c.oracle(oracle_mod), "reuse %d" % i)
        n_rep = c.H // c.Hkv
        groups = -(-n_rep // (8 if n_rep > 4 else 4))
        counters = ws[:c.Hkv * groups * c.S * 4].cpu().numpy()
        assert not counters.any(), "arrival counters not left at zero"


def test_workspace_too_small_is_rejected(oracle_mod):
    from int8_paged_kv_amd import Q8Error
    from gpu_util import RandomCase
    c = RandomCase(oracle_mod, 61, 2, 4, 2, 128, 16, [5000, 10])
    ws = torch.empty(64, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(Q8Error):
        c.gpu(workspace=ws)


@pytest.mark.parametrize("name", ["llama", "long", "mha256", "selected"])
def test_full_size_workloads(oracle_mod, name):
    """Every workload at full size, in the launch configuration the bench times:
    the fill and step writes are checked bit-exact over the whole caches, and
    every decode output against the oracle."""
    from gpu_util import Filled, assert_close, u32_host
    w = wl.get(name)
    f = Filled(w, oracle_mod)
    assert np.array_equal(u32_host(f.kc_d), f.kc_h), name + ": key cache words differ"
    assert np.array_equal(u32_host(f.vc_d), f.vc_h), name + ": value cache words differ"
    assert_close(f.decode_gpu(), f.decode_oracle(oracle_mod), name)
