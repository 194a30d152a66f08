"""GPU parity of q8_paged_decode_noalloc (the decode that uses the library's
own scratch array instead of a caller workspace) against q8_paged_decode with
its workspace, through the C ABI: two calls in a row, the second with a
smaller input, so the second runs on the scratch the first left behind; both
are also held to the oracle's tolerance."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _both(case, mcl=None, vis=None, nvis=None):
    from gpu_util import nan_out, u32_dev
    from int8_paged_kv_amd import q8_paged_decode, q8_paged_decode_noalloc
    mcl = int(case.lens.max()) if mcl is None else mcl
    visd = None if vis is None else u32_dev(vis)
    nvisd = None if nvis is None else u32_dev(nvis)
    out_ws = nan_out(case.S, case.H, case.hs)
    out_na = nan_out(case.S, case.H, case.hs)
    q8_paged_decode(case.q_d, case.kc_d, case.vc_d, case.bt_d, case.cl_d, case.scale, case.Hkv, case.bs,
                    max_context_len=mcl, visible_pos=visd, num_visible=nvisd, out=out_ws)
    q8_paged_decode_noalloc(case.q_d, case.kc_d, case.vc_d, case.bt_d, case.cl_d, case.scale, case.Hkv, case.bs,
                            max_context_len=mcl, visible_pos=visd, num_visible=nvisd, out=out_na)
    torch.cuda.synchronize()
    return out_ws.cpu().numpy(), out_na.cpu().numpy()


def test_noalloc_matches_workspace_decode_twice(oracle_mod):
    from gpu_util import RandomCase, assert_close
    g = np.random.default_rng(71)
    # first call: a Llama-shaped batch (sequences split over several waves, partial records in the scratch)
    lens1 = g.integers(512, 3000, 40).tolist()
    big = RandomCase(oracle_mod, 7101, 40, 32, 8, 128, 16, lens1)
    print("noalloc call 1: S=40 H=32 Hkv=8 hs=128 bs=16", flush=True)
    ws1, na1 = _both(big)
    assert np.array_equal(ws1.view(np.uint32), na1.view(np.uint32)), "call 1 differs from the workspace decode"
    assert_close(na1, big.oracle(oracle_mod), "noalloc call 1 vs oracle")
    # second call: smaller, other shapes, an empty sequence; the scratch keeps call 1's records
    small = RandomCase(oracle_mod, 7102, 5, 8, 2, 64, 16, [700, 0, 65, 1, 250])
    print("noalloc call 2: S=5 H=8 Hkv=2 hs=64 bs=16", flush=True)
    ws2, na2 = _both(small)
    assert np.array_equal(ws2.view(np.uint32), na2.view(np.uint32)), "call 2 differs from the workspace decode"
    assert_close(na2, small.oracle(oracle_mod), "noalloc call 2 vs oracle")


def test_noalloc_visible_list_and_clamp(oracle_mod):
    from gpu_util import RandomCase, assert_close
    g = np.random.default_rng(72)
    case = RandomCase(oracle_mod, 7201, 6, 16, 4, 128, 16, [900, 130, 64, 2000, 5, 777])
    print("noalloc: clamped dense call, then a visible-list call", flush=True)
    ws, na = _both(case, mcl=700)
    assert np.array_equal(ws.view(np.uint32), na.view(np.uint32))
    assert_close(na, case.oracle(oracle_mod, max_context_len=700), "noalloc clamp")
    stride = 1100
    vis = np.zeros((case.S, stride), dtype=np.uint32)
    nvis = np.zeros(case.S, dtype=np.uint32)
    for s, L in enumerate(case.lens):
        n = min(int(L), int(g.integers(0, stride)))
        vis[s, :n] = np.sort(g.choice(int(L), n, replace=False))
        nvis[s] = n
    ws, na = _both(case, vis=vis, nvis=nvis)
    assert np.array_equal(ws.view(np.uint32), na.view(np.uint32))
    assert_close(na, case.oracle(oracle_mod, vis=vis, nvis=nvis), "noalloc visible list")
