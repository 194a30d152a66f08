"""GPU parity of q8_paged_decode_rows (several causal query rows per
sequence at its last positions) against the oracle's decode of every row
over its own prefix: element by element within 1e-4 + 1e-4*|oracle|, empty
prefixes giving zero rows (the output starts as NaN)."""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run_rows_case(oracle_mod, seed, S, H, Hkv, hs, bs, lens, nb, mcl=None):
    from int8_paged_kv_amd import q8_paged_decode_rows
    from gpu_util import RandomCase, assert_close, f32_dev, nan_out
    c = RandomCase(oracle_mod, seed, S, H, Hkv, hs, bs, lens)
    mcl = int(c.lens.max()) if mcl is None else mcl
    g = np.random.default_rng(seed + 500)
    q = g.standard_normal((S * nb, H, hs)).astype(np.float32)
    out = q8_paged_decode_rows(f32_dev(q), c.kc_d, c.vc_d, c.bt_d, c.cl_d, c.scale, Hkv, bs, mcl, nb,
                               out=nan_out(S * nb, H, hs))
    torch.cuda.synchronize()
    # the oracle decodes every row as its own sequence over its causal prefix
    rows_bt = np.repeat(c.bt, nb, axis=0)
    rows_len = np.array([max(0, int(c.lens[v // nb]) - nb + v % nb + 1) for v in range(S * nb)], dtype=np.uint32)
    want = oracle_mod.paged_decode(q, c.kc, c.vc, rows_bt, rows_len, c.scale, Hkv, bs, max_context_len=mcl)
    assert_close(out.cpu().numpy(), want, "rows %s" % ((S, H, Hkv, hs, bs, list(lens), nb, mcl),))


@pytest.mark.parametrize("S,H,Hkv,hs,bs,lens,nb", [
    (3, 8, 2, 128, 16, [900, 3, 130], 4),              # a sequence shorter than its rows: empty first row
    (2, 8, 2, 128, 16, [500, 64], 1),                  # one row per sequence: plain decode
    (9, 8, 2, 128, 16, [70, 1, 0, 200, 65, 64, 128, 900, 33], 8),   # 72 rows: more than one 64-lane window
    (2, 16, 2, 128, 32, [333, 129], 5),                # n_rep 8
    (2, 4, 2, 64, 5, [61, 12], 3),                     # block_size 5: row gather
    (2, 4, 1, 256, 16, [300, 90], 4),                  # head_size 256
])
def test_rows_shapes(oracle_mod, S, H, Hkv, hs, bs, lens, nb):
    run_rows_case(oracle_mod, hash((S, H, Hkv, hs, bs, nb)) % 10000, S, H, Hkv, hs, bs, lens, nb)


def test_rows_clamped(oracle_mod):
    """Rows whose prefix passes max_context_len attend its first positions."""
    run_rows_case(oracle_mod, 31, 3, 8, 2, 128, 16, [400, 250, 100], 4, mcl=256)


@pytest.mark.parametrize("waves", [7, 333])
def test_rows_wavefront_boundaries(oracle_mod, waves):
    os.environ["Q8KV_DECODE_WAVES"] = str(waves)
    try:
        run_rows_case(oracle_mod, 60 + waves, 5, 8, 2, 128, 16, [0, 63, 1025, 257, 2049], 4)
    finally:
        os.environ.pop("Q8KV_DECODE_WAVES", None)


def test_rows_match_single_row_decodes(oracle_mod):
    """Row b of a multi-row call equals a plain decode of the same q row with
    the context length L - nb + b + 1 (within the tolerance: the partition of
    the work differs between the calls)."""
    from int8_paged_kv_amd import q8_paged_decode, q8_paged_decode_rows
    from gpu_util import RandomCase, assert_close, f32_dev, u32_dev
    nb = 4
    c = RandomCase(oracle_mod, 91, 4, 8, 2, 128, 16, [300, 700, 64, 5])
    g = np.random.default_rng(92)
    q = g.standard_normal((4 * nb, 8, 128)).astype(np.float32)
    qd = f32_dev(q)
    multi = q8_paged_decode_rows(qd, c.kc_d, c.vc_d, c.bt_d, c.cl_d, c.scale, 2, 16, 700, nb).cpu().numpy()
    for b in range(nb):
        lens_b = np.array([max(0, int(L) - nb + b + 1) for L in c.lens], dtype=np.uint32)
        single = q8_paged_decode(qd[b::nb].contiguous(), c.kc_d, c.vc_d, c.bt_d, u32_dev(lens_b), c.scale, 2, 16,
                                 max_context_len=700)
        assert_close(multi[b::nb], single.cpu().numpy(), "row %d" % b)


def test_rows_full_size_llama(oracle_mod):
    """The Llama-shaped batch with 4 rows per sequence in the launch
    configuration the bench times (16 (row, head) pairs per kv head: two row
    groups side by side): every row against the oracle over its prefix."""
    from int8_paged_kv_amd import q8_paged_decode_rows, q8_paged_decode_workspace_bytes
    from int8_paged_kv_amd import workloads as wl
    from gpu_util import Filled, assert_close, f32_dev, nan_out
    w = wl.get("llama")
    f = Filled(w, oracle_mod)
    nb = 4
    S, H, Hkv, hs, mcl = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size, w.max_context_len
    q = np.random.default_rng(11).standard_normal((S * nb, H, hs)).astype(np.float32)
    ws = torch.zeros(max(1, q8_paged_decode_workspace_bytes(S, H * nb, Hkv, hs, w.block_size, mcl)),
                     dtype=torch.uint8, device="cuda:0")
    out = q8_paged_decode_rows(f32_dev(q), f.kc_d, f.vc_d, f.bt_d, f.cl_d, w.scale, Hkv, w.block_size, mcl, nb,
                               out=nan_out(S * nb, H, hs), workspace=ws)
    torch.cuda.synchronize()
    rows_bt = np.repeat(w.block_tables, nb, axis=0)
    rows_len = np.array([max(0, int(L) - nb + b + 1) for L in w.context_lens for b in range(nb)], dtype=np.uint32)
    want = oracle_mod.paged_decode(q, f.kc_h, f.vc_h, rows_bt, rows_len, w.scale, Hkv, w.block_size,
                                   max_context_len=mcl)
    assert_close(out.cpu().numpy(), want, "4-row decode of the Llama-shaped batch")
