"""Shared helpers of the GPU parity tests: device copies of the seeded inputs and
the HIP path driven through the C ABI binding, with the oracle run on the same
inputs on the host."""
import numpy as np
import torch

from int8_paged_kv_amd import workloads as wl

DEV = "cuda:0"
ATOL = 1e-4
RTOL = 1e-4


def u32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    """uint16 bfloat16 encodings to a device int16 tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def nan_out(S: int, H: int, hs: int) -> torch.Tensor:
    """Output buffer filled with NaN, so a row the decode never writes fails
    the comparison instead of passing on memory that happens to be zero."""
    return torch.full((S, H, hs), float("nan"), dtype=torch.float32, device="cuda:0")


def u32_host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def assert_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    """Per element |got - want| <= 1e-4 + 1e-4*|want| (and no NaN anywhere)."""
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol = ATOL + RTOL * np.abs(want.astype(np.float64))
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError("%s: %d elements out of tolerance; worst at %s: got %r want %r"
                             % (what, int(bad.sum()), i, got[i], want[i]))


class Filled:
    """A workload's caches filled by the HIP writer (device) and the oracle (host)."""

    def __init__(self, w: wl.Workload, oracle, check_write=True, with_step=True):
        from int8_paged_kv_amd import q8_cache_write
        self.w = w
        kh, vh = w.empty_caches()
        self.kc_d, self.vc_d = u32_dev(kh), u32_dev(vh)
        for slots, k, v in w.fill_chunks():
            q8_cache_write(f32_dev(k), f32_dev(v), self.kc_d, self.vc_d, u32_dev(slots),
                           w.num_kv_heads, w.head_size, w.block_size)
            if check_write:
                oracle.cache_write(k, v, kh, vh, slots, w.num_kv_heads, w.head_size, w.block_size)
        step = w.step_write() if with_step else None
        if step is not None:
            slots, k, v = step
            q8_cache_write(f32_dev(k), f32_dev(v), self.kc_d, self.vc_d, u32_dev(slots),
                           w.num_kv_heads, w.head_size, w.block_size)
            if check_write:
                oracle.cache_write(k, v, kh, vh, slots, w.num_kv_heads, w.head_size, w.block_size)
        torch.cuda.synchronize()
        self.kc_h, self.vc_h = (kh, vh) if check_write else (None, None)
        self.q = w.q()
        self.q_d = f32_dev(self.q)
        self.bt_d = u32_dev(w.block_tables)
        self.cl_d = u32_dev(w.context_lens)
        self.vis_d = None if w.visible_pos is None else u32_dev(w.visible_pos)
        self.nvis_d = None if w.num_visible is None else u32_dev(w.num_visible)

    def decode_gpu(self, **kw):
        from int8_paged_kv_amd import q8_paged_decode
        w = self.w
        kw.setdefault("out", nan_out(w.num_seqs, w.num_heads, w.head_size))
        out = q8_paged_decode(self.q_d, self.kc_d, self.vc_d, self.bt_d, self.cl_d, w.scale, w.num_kv_heads,
                              w.block_size, max_context_len=w.max_context_len, visible_pos=self.vis_d,
                              num_visible=self.nvis_d, **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def decode_oracle(self, oracle, kc=None, vc=None):
        w = self.w
        return oracle.paged_decode(self.q, self.kc_h if kc is None else kc, self.vc_h if vc is None else vc,
                                   w.block_tables, w.context_lens, w.scale, w.num_kv_heads, w.block_size,
                                   max_context_len=w.max_context_len, visible_pos=w.visible_pos,
                                   num_visible=w.num_visible)


class RandomCase:
    """A random paged cache filled on the host by the oracle writer, copied to the
    device; used to test the decode kernels in isolation."""

    def __init__(self, oracle, seed, S, H, Hkv, hs, bs, lens, spare_blocks=2, q_pad=0, outliers=False):
        g = np.random.default_rng(seed)
        self.S, self.H, self.Hkv, self.hs, self.bs = S, H, Hkv, hs, bs
        self.lens = np.asarray(lens, dtype=np.uint32)
        nbs = [-(-int(L) // bs) for L in self.lens]
        self.max_nb = max(nbs + [1])
        self.num_blocks = sum(nbs) + spare_blocks
        perm = g.permutation(self.num_blocks).astype(np.uint32)
        self.bt = np.full((S, self.max_nb), self.num_blocks, dtype=np.uint32)   # poison block
        at = 0
        for s, nb in enumerate(nbs):
            self.bt[s, :nb] = perm[at:at + nb]
            at += nb
        self.kc = wl.poison_cache(self.num_blocks + 1, Hkv, bs, hs)
        self.vc = wl.poison_cache(self.num_blocks + 1, Hkv, bs, hs)
        for s in range(S):
            L = int(self.lens[s])
            if not L:
                continue
            K = g.standard_normal((L, Hkv, hs)).astype(np.float32)
            V = g.standard_normal((L, Hkv, hs)).astype(np.float32)
            if outliers:
                K[:, :, ::17] *= 20
                V[:, :, 3::29] *= 20
            pos = np.arange(L)
            slots = (self.bt[s, pos // bs].astype(np.int64) * bs + pos % bs).astype(np.uint32)
            oracle.cache_write(K, V, self.kc, self.vc, slots, Hkv, hs, bs)
        qfull = g.standard_normal((S, H * hs + q_pad)).astype(np.float32)
        self.q_store = qfull
        self.q = np.ascontiguousarray(qfull[:, :H * hs].reshape(S, H, hs))
        self.scale = float(np.float32(1.0 / np.sqrt(hs)))
        self.kc_d, self.vc_d = u32_dev(self.kc), u32_dev(self.vc)
        qd = f32_dev(qfull)
        self.q_d = qd[:, :H * hs].view(S, H, hs) if q_pad == 0 else qd.as_strided((S, H, hs), (H * hs + q_pad, hs, 1))
        self.bt_d = u32_dev(self.bt)
        self.cl_d = u32_dev(self.lens)

    def gpu(self, max_context_len=None, vis=None, nvis=None, **kw):
        from int8_paged_kv_amd import q8_paged_decode
        mcl = int(self.lens.max()) if max_context_len is None else max_context_len
        kw.setdefault("out", nan_out(self.S, self.H, self.hs))
        out = q8_paged_decode(self.q_d, self.kc_d, self.vc_d, self.bt_d, self.cl_d, self.scale, self.Hkv,
                              self.bs, max_context_len=mcl,
                              visible_pos=None if vis is None else u32_dev(vis),
                              num_visible=None if nvis is None else u32_dev(nvis), **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle(self, oracle, max_context_len=None, vis=None, nvis=None):
        return oracle.paged_decode(self.q, self.kc, self.vc, self.bt, self.lens, self.scale, self.Hkv, self.bs,
                                   max_context_len=max_context_len, visible_pos=vis, num_visible=nvis)
