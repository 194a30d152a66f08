"""Randomized GPU parity sweep against the oracle: decode (dense and
visible-list), the one-launch step, multi-row decode, the cache writer
(bit-exact; small and batched sizes, pads), block selection (lists, counts
and bitmasks bit-exact), the q + K/V norm and rotary launch, the decode step
with the norm and rotary step inside it, and the f32- and bf16-cache decodes, over random head
sizes, block sizes, GQA ratios, batch sizes on both sides of the 64-sequence
window, length mixes (empty, one token, block and chunk edges, long), clamps
and forced wavefront counts.  Every case is drawn from a fixed seed and named
by its index, so a failure is reproducible on the CPU side from its parameters
(printed in the assertion message)."""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 432
HEAD_SIZES = [16, 32, 48, 64, 68, 96, 128, 192, 256]
BLOCK_SIZES = [1, 4, 5, 8, 16, 32, 64, 128]
KV_HEADS = [1, 2, 3, 4, 8]
N_REPS = [1, 2, 3, 4, 5, 7, 8, 12, 16]
WAVES = [None, None, 1, 7, 64, 333, 2048]


def draw(i):
    g = np.random.default_rng(900 + i)
    kind = ["decode", "decode", "visible", "step", "rows", "write", "select", "normrope", "f32"][i % 9]
    hs = int(g.choice(HEAD_SIZES))
    bs = int(g.choice(BLOCK_SIZES))
    hkv = int(g.choice(KV_HEADS))
    n_rep = int(g.choice(N_REPS))
    while hkv * n_rep > 64:
        n_rep = max(1, n_rep // 2)
    S = int(g.choice([1, 2, 5, 17, 63, 64, 65, 80]))
    edges = [0, 1, bs - 1 if bs > 1 else 1, bs, bs + 1, 63, 64, 65, 127, 128, 129]
    budget = 40000 // max(1, S)                   # keeps the oracle's work small
    lens = []
    for _ in range(S):
        r = g.random()
        if r < 0.15:
            lens.append(0)
        elif r < 0.45:
            lens.append(int(g.choice(edges)))
        else:
            lens.append(int(g.integers(1, max(2, min(2500, budget)))))
    waves = WAVES[int(g.integers(len(WAVES)))]
    mcl = None
    if kind != "visible" and g.random() < 0.25 and max(lens) > 2:
        mcl = int(g.integers(1, max(lens)))           # clamp some sequences
    nb = int(g.integers(1, 7))
    return dict(kind=kind, hs=hs, bs=bs, Hkv=hkv, H=hkv * n_rep, S=S, lens=lens, waves=waves, mcl=mcl, nb=nb,
                seed=1000 + i)


def run_write_case(oracle_mod, p):
    """q8_cache_write of T tokens (some pads) into a poisoned cache: every word bit-exact."""
    from int8_paged_kv_amd import PAD_SLOT, q8_cache_write
    from int8_paged_kv_amd import workloads as wl
    from gpu_util import f32_dev, u32_dev, u32_host
    g = np.random.default_rng(p["seed"] + 3)
    hs, bs, hkv = p["hs"], p["bs"], p["Hkv"]
    T = int(g.choice([1, 7, 64, 513, 4099, 40000 // hkv + 3]))
    nb = T // bs + 3
    key = (g.standard_normal((T, hkv, hs)) * g.uniform(0.01, 50, (T, 1, 1))).astype(np.float32)
    val = g.standard_normal((T, hkv, hs)).astype(np.float32)
    key[g.random((T, hkv)) < 0.02] = 0.0                  # zero vectors: scale word 1.0
    slots = g.choice(nb * bs, size=T, replace=False).astype(np.uint32)
    slots[g.random(T) < 0.1] = PAD_SLOT
    kh, vh = wl.poison_cache(nb, hkv, bs, hs), wl.poison_cache(nb, hkv, bs, hs)
    kd, vd = u32_dev(kh), u32_dev(vh)
    q8_cache_write(f32_dev(key), f32_dev(val), kd, vd, u32_dev(slots), hkv, hs, bs)
    torch.cuda.synchronize()
    oracle_mod.cache_write(key, val, kh, vh, slots, hkv, hs, bs)
    assert np.array_equal(u32_host(kd), kh), "key cache words differ (T=%d)" % T
    assert np.array_equal(u32_host(vd), vh), "value cache words differ (T=%d)" % T


def run_select_case(oracle_mod, p):
    """q8_index_select over random rows: lists, counts and bitmasks bit-exact."""
    from test_gpu_index_select import run_select
    g = np.random.default_rng(p["seed"] + 4)
    ratio = int(g.choice([1, 4, 16, 64]))
    k = int(g.integers(0, 41))
    max_blocks = int(g.integers(1, 3001))
    R = int(g.integers(1, 41))
    if g.random() < 0.5:
        scores = g.integers(-3, 4, (R, max_blocks)).astype(np.float32)       # many ties
    else:
        scores = g.standard_normal((R, max_blocks)).astype(np.float32)
    lens = g.integers(0, max_blocks * ratio + ratio, R).astype(np.uint32)
    vis_stride = k * ratio + ratio + int(g.integers(0, 5))
    mask_stride = (max_blocks + 1 + 31) // 32 + int(g.integers(0, 3))
    run_select(oracle_mod, scores, lens, ratio, k, vis_stride, mask_stride)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(oracle_mod, i):
    p = draw(i)
    name = "case %d: %s" % (i, {k: (v if k != "lens" else v[:12]) for k, v in p.items()})
    if p["waves"] is not None:
        os.environ["Q8KV_DECODE_WAVES"] = str(p["waves"])
    try:
        if p["kind"] == "write":
            run_write_case(oracle_mod, p)
        elif p["kind"] == "f32":
            from test_gpu_bf16 import Bf16Gpu
            from test_gpu_f32 import F32Gpu
            from gpu_util import assert_close
            hs = {16: 16, 32: 32, 48: 64, 64: 64, 68: 64, 96: 128, 128: 128, 192: 256, 256: 256}[p["hs"]]
            if p["waves"] is not None:
                os.environ["Q8KV_F32_DECODE_WAVES"] = str(p["waves"])
            cls = Bf16Gpu if (i // 9) % 2 else F32Gpu          # alternate the two baseline caches
            c = cls(oracle_mod, p["seed"], p["S"], p["H"], p["Hkv"], hs, p["bs"], p["lens"])
            assert_close(c.gpu(max_context_len=p["mcl"]), c.oracle(oracle_mod, max_context_len=p["mcl"]), name)
        elif p["kind"] == "select":
            run_select_case(oracle_mod, p)
        elif p["kind"] == "normrope":
            from test_gpu_norm_rope import test_norm_rope_qk_cache_write as run_qk
            g = np.random.default_rng(p["seed"] + 5)
            hs = int(g.choice([32, 64, 96, 128, 192, 256]))
            rot = 8 * int(g.integers(0, hs // 8 + 1))
            run_qk(oracle_mod, int(g.choice([0, 1, 9, 64])), int(g.integers(1, 9)), int(g.choice([0, 3, 64, 700])),
                   p["Hkv"], hs, rot)
        elif p["kind"] == "step":
            from test_gpu_step import run_step_case
            run_step_case(oracle_mod, p["seed"], p["S"], p["H"], p["Hkv"], p["hs"], p["bs"], p["lens"], mcl=p["mcl"])
        elif p["kind"] == "rows":
            from test_gpu_rows import run_rows_case
            run_rows_case(oracle_mod, p["seed"], p["S"], p["H"], p["Hkv"], p["hs"], p["bs"], p["lens"], p["nb"],
                          mcl=p["mcl"])
        else:
            from gpu_util import RandomCase, assert_close
            c = RandomCase(oracle_mod, p["seed"], p["S"], p["H"], p["Hkv"], p["hs"], p["bs"], p["lens"])
            vis = nvis = None
            if p["kind"] == "visible":
                g = np.random.default_rng(p["seed"] + 7)
                stride = max(1, max(p["lens"]))
                vis = np.zeros((p["S"], stride), np.uint32)
                nvis = np.zeros(p["S"], np.uint32)
                for s, L in enumerate(p["lens"]):
                    if L == 0:
                        continue
                    keep = g.random(L) < g.choice([0.1, 0.5, 1.0])
                    pos = np.nonzero(keep)[0]
                    vis[s, :pos.size] = pos
                    nvis[s] = pos.size
            got = c.gpu(max_context_len=p["mcl"], vis=vis, nvis=nvis)
            want = c.oracle(oracle_mod, max_context_len=p["mcl"], vis=vis, nvis=nvis)
            assert_close(got, want, name)
    except AssertionError as e:
        raise AssertionError("%s: %s" % (name, e)) from None
    finally:
        os.environ.pop("Q8KV_DECODE_WAVES", None)
        os.environ.pop("Q8KV_F32_DECODE_WAVES", None)


N_NR_CASES = 48


def draw_nr(i):
    """A random decode step with the norm + rotary step (its supported shapes)."""
    g = np.random.default_rng(5000 + i)
    hs = int(g.choice([64, 128, 256]))
    bs = int(g.choice([4, 8, 16, 32, 64, 128]))
    hkv = int(g.choice(KV_HEADS))
    n_rep = int(g.choice([r for r in N_REPS if hs < 256 or r <= 8]))
    while hkv * n_rep > 64:
        n_rep = max(1, n_rep // 2)
    S = int(g.choice([1, 2, 5, 17, 63, 64, 65, 80]))
    edges = [0, 1, bs - 1 if bs > 1 else 1, bs, bs + 1, 31, 32, 33, 63, 64, 65, 129]
    budget = 30000 // max(1, S)
    lens = [0 if r < 0.1 else int(g.choice(edges)) if r < 0.4 else int(g.integers(1, max(2, min(2000, budget))))
            for r in g.random(S)]
    mcl = int(g.integers(1, max(lens))) if g.random() < 0.25 and max(lens) > 2 else None
    P = int(g.choice([8192, max(2, max(lens) // 2)]))           # sometimes positions past the table
    return dict(hs=hs, bs=bs, Hkv=hkv, H=hkv * n_rep, S=S, lens=lens, mcl=mcl, P=P,
                rot=8 * int(g.integers(0, hs // 8 + 1)), eps=float(g.choice([0.0, 1e-6, 1e-5])),
                layout=str(g.choice(["packed", "packed", "interleave", "offset"])),
                misaligned=bool(g.random() < 0.3), waves=WAVES[int(g.integers(len(WAVES)))], seed=6000 + i)


@pytest.mark.parametrize("i", range(N_NR_CASES))
def test_random_norm_rope_step_case(oracle_mod, i):
    """q8_norm_rope_decode_step: bit-exact against q8_norm_rope + q8_decode_step,
    and against the oracle's norm_rope -> norm_rope_cache_write -> paged_decode."""
    from test_gpu_norm_rope_step import run_case
    p = draw_nr(i)
    name = "nr case %d: %s" % (i, {k: (v if k != "lens" else v[:12]) for k, v in p.items()})
    if p["waves"] is not None:
        os.environ["Q8KV_DECODE_WAVES"] = str(p["waves"])
    try:
        run_case(oracle_mod, p["seed"], p["S"], p["H"], p["Hkv"], p["bs"], p["lens"], p["rot"], hs=p["hs"],
                 mcl=p["mcl"], P=p["P"], eps=p["eps"], q_layout=p["layout"], misaligned_params=p["misaligned"])
    except AssertionError as e:
        raise AssertionError("%s: %s" % (name, e)) from None
    finally:
        os.environ.pop("Q8KV_DECODE_WAVES", None)
