"""Seeded synthetic workloads for the int8 paged KV cache.

This module only draws inputs: block tables, context lengths, slot mappings,
visible-position lists, f32 Q/K/V and poison-filled empty caches.  It holds
none of the method's arithmetic (no quantization, no attention), so both the
HIP path and the CPU oracle can consume the same inputs.

Every random draw comes from its own ``numpy.random.PCG64`` stream keyed by
``SeedSequence([seed, purpose, index])``, so any chunk of the cache fill can be
regenerated on its own.  The shapes follow the workloads named for this path:
a tiny parity case, a Llama-3-8B-shaped decode batch, a 32K long-context batch
with outlier channels, an MHA head_size=256 batch with a padded cache write,
and a selected-token decode over visible-position lists.
"""
from __future__ import annotations

import dataclasses
from typing import Iterator, List, Optional, Tuple

import numpy as np

PAD_SLOT = 0xFFFFFFFF
# Unwritten cache rows hold these: code bytes 0x7F and a NaN scale word, so a
# decode that reads a row it should not see produces NaN.
POISON_CODE_WORD = 0x7F7F7F7F
POISON_SCALE_WORD = 0x7FC00000

FILL_CHUNK_TOKENS = 65536

# stream purposes
_LENS, _TABLES, _FILL_K, _FILL_V, _Q, _STEP_K, _STEP_V, _MASKS, _OUTLIERS, _VIS = range(10)


def rng(seed: int, purpose: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, purpose, index])))


def poison_cache(num_blocks_total: int, num_kv_heads: int, block_size: int, head_size: int) -> np.ndarray:
    """A u32 cache [num_blocks_total, Hkv, bs, hs/4+1] with every row poisoned."""
    wpt = head_size // 4 + 1
    c = np.full((num_blocks_total, num_kv_heads, block_size, wpt), POISON_CODE_WORD, dtype=np.uint32)
    c[..., wpt - 1] = POISON_SCALE_WORD
    return c


def poison_cache_f32(num_blocks_total: int, num_kv_heads: int, block_size: int, head_size: int) -> np.ndarray:
    """An f32 cache [num_blocks_total, Hkv, bs, hs] with every element NaN."""
    return np.full((num_blocks_total, num_kv_heads, block_size, head_size), np.nan, dtype=np.float32)


POISON_BF16 = 0x7FC1      # a quiet NaN encoding


def poison_cache_bf16(num_blocks_total: int, num_kv_heads: int, block_size: int, head_size: int) -> np.ndarray:
    """A bfloat16 cache [num_blocks_total, Hkv, bs, hs] (uint16 encodings) with every element NaN."""
    return np.full((num_blocks_total, num_kv_heads, block_size, head_size), POISON_BF16, dtype=np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int                  # usable blocks; the cache holds one more (poison) block
    block_tables: np.ndarray         # u32 [S, max_num_blocks_per_seq]
    context_lens: np.ndarray         # u32 [S]
    scale: float
    fill_positions: List[np.ndarray]  # per seq: logical positions written before the step
    step_positions: Optional[np.ndarray] = None   # per seq position written by the step write
    visible_pos: Optional[np.ndarray] = None      # u32 [S, vis_stride]
    num_visible: Optional[np.ndarray] = None      # u32 [S]
    outlier_k: Optional[np.ndarray] = None        # bool [Hkv, hs] channels scaled x20
    outlier_v: Optional[np.ndarray] = None
    description: str = ""

    @property
    def poison_block(self) -> int:
        return self.num_blocks

    @property
    def max_num_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def vis_stride(self) -> int:
        return 0 if self.visible_pos is None else int(self.visible_pos.shape[1])

    @property
    def words_per_token(self) -> int:
        return self.head_size // 4 + 1

    def attended_counts(self) -> np.ndarray:
        """Number of positions each sequence attends in the decode step."""
        if self.num_visible is not None:
            return self.num_visible.astype(np.int64)
        return np.minimum(self.context_lens, self.max_context_len).astype(np.int64)

    def effective_kv_bytes(self) -> int:
        """Codes + scale word of every attended row, for K and V."""
        return int(self.attended_counts().sum()) * self.num_kv_heads * 2 * (self.head_size + 4)

    def empty_caches(self) -> Tuple[np.ndarray, np.ndarray]:
        args = (self.num_blocks + 1, self.num_kv_heads, self.block_size, self.head_size)
        return poison_cache(*args), poison_cache(*args)

    def slots_of(self, s: int, positions: np.ndarray) -> np.ndarray:
        bs = self.block_size
        return (self.block_tables[s, positions // bs].astype(np.uint64) * bs + positions % bs).astype(np.uint32)

    def _kv(self, purpose_k: int, purpose_v: int, index: int, T: int) -> Tuple[np.ndarray, np.ndarray]:
        shape = (T, self.num_kv_heads, self.head_size)
        k = rng(self.seed, purpose_k, index).standard_normal(shape, dtype=np.float32)
        v = rng(self.seed, purpose_v, index).standard_normal(shape, dtype=np.float32)
        if self.outlier_k is not None:
            k[:, self.outlier_k] *= np.float32(20.0)
        if self.outlier_v is not None:
            v[:, self.outlier_v] *= np.float32(20.0)
        return k, v

    def fill_slots(self) -> np.ndarray:
        return np.concatenate([self.slots_of(s, p) for s, p in enumerate(self.fill_positions)]
                              or [np.zeros(0, np.uint32)]).astype(np.uint32)

    def fill_chunks(self, chunk_tokens: int = FILL_CHUNK_TOKENS) -> Iterator[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
        """Yield (slot_mapping u32 [T], key f32 [T,Hkv,hs], value f32 [T,Hkv,hs]) chunks."""
        slots = self.fill_slots()
        for ci, start in enumerate(range(0, slots.shape[0], chunk_tokens)):
            sl = slots[start:start + chunk_tokens]
            k, v = self._kv(_FILL_K, _FILL_V, ci, sl.shape[0])
            yield sl, k, v

    def q(self) -> np.ndarray:
        return rng(self.seed, _Q).standard_normal((self.num_seqs, self.num_heads, self.head_size),
                                                 dtype=np.float32)

    def step_write(self) -> Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
        """The cache write of the decode step, or None when the workload has none."""
        if self.step_positions is None:
            return None
        slots = np.array([self.slots_of(s, np.array([p]))[0] for s, p in enumerate(self.step_positions)],
                         dtype=np.uint32)
        k, v = self._kv(_STEP_K, _STEP_V, 0, slots.shape[0])
        return slots, k, v


def tiny() -> Workload:
    """S=2, H=4, Hkv=2, hs=64, bs=16, L={37,64}; 16 blocks, tables a random permutation."""
    seed = 1
    S, H, Hkv, hs, bs, nblk = 2, 4, 2, 64, 16, 16
    lens = np.array([37, 64], dtype=np.uint32)
    bt = rng(seed, _TABLES).permutation(nblk).astype(np.uint32).reshape(S, nblk // S)
    fill = [np.arange(int(L), dtype=np.int64) for L in lens]
    return Workload("tiny", seed, S, H, Hkv, hs, bs, nblk, bt, lens, 1.0 / 8.0, fill,
                    description="tiny parity case")


def _deal_tables(seed: int, lens: np.ndarray, bs: int, num_blocks: int, max_nb: int,
                 poison: int) -> np.ndarray:
    """Blocks drawn in order from a shuffled pool; unused entries -> poison block."""
    pool = rng(seed, _TABLES).permutation(num_blocks).astype(np.uint32)
    bt = np.full((lens.shape[0], max_nb), poison, dtype=np.uint32)
    at = 0
    for s, L in enumerate(lens):
        nb = -(-int(L) // bs)
        if at + nb > num_blocks or nb > max_nb:
            raise ValueError("block pool too small")
        bt[s, :nb] = pool[at:at + nb]
        at += nb
    return bt


def llama() -> Workload:
    """Llama-3-8B-shaped decode: S=64, H=32, Hkv=8, hs=128, bs=16, L~U[512,4096],
    blocks from a shuffled pool of 20000; the step writes each seq's newest token."""
    seed = 2
    S, H, Hkv, hs, bs, nblk, max_nb = 64, 32, 8, 128, 16, 20000, 256
    lens = rng(seed, _LENS).integers(512, 4096, size=S, endpoint=True).astype(np.uint32)
    bt = _deal_tables(seed, lens, bs, nblk, max_nb, nblk)
    fill = [np.arange(int(L) - 1, dtype=np.int64) for L in lens]
    step = np.array([int(L) - 1 for L in lens], dtype=np.int64)
    return Workload("llama", seed, S, H, Hkv, hs, bs, nblk, bt, lens, float(np.float32(1.0 / np.sqrt(128.0))),
                    fill, step_positions=step,
                    description="Llama-3-8B-shaped decode (S=64, H=32, Hkv=8, hs=128, bs=16, L~U[512,4096])")


def long_context() -> Workload:
    """S=8, H=64, Hkv=8, hs=128, bs=32, L=32768 each; fragmented random tables;
    K/V with 2% of (kv head, dim) channels scaled x20."""
    seed = 3
    S, H, Hkv, hs, bs, L = 8, 64, 8, 128, 32, 32768
    nb_seq = L // bs
    nblk = 2 * S * nb_seq
    lens = np.full(S, L, dtype=np.uint32)
    bt = rng(seed, _TABLES).choice(nblk, size=S * nb_seq, replace=False).astype(np.uint32).reshape(S, nb_seq)
    n_out = int(round(0.02 * Hkv * hs))
    ok = np.zeros(Hkv * hs, dtype=bool)
    ok[rng(seed, _OUTLIERS, 0).choice(Hkv * hs, size=n_out, replace=False)] = True
    ov = np.zeros(Hkv * hs, dtype=bool)
    ov[rng(seed, _OUTLIERS, 1).choice(Hkv * hs, size=n_out, replace=False)] = True
    fill = [np.arange(L, dtype=np.int64) for _ in range(S)]
    return Workload("long", seed, S, H, Hkv, hs, bs, nblk, bt, lens, float(np.float32(1.0 / np.sqrt(128.0))), fill,
                    outlier_k=ok.reshape(Hkv, hs), outlier_v=ov.reshape(Hkv, hs),
                    description="long context (S=8, H=64, Hkv=8, hs=128, bs=32, L=32768, 2% outlier channels)")


def mha256() -> Workload:
    """MHA hs=256: S=128, H=Hkv=16, bs=16, L~U[1024,2048]; 20000 blocks."""
    seed = 4
    S, H, Hkv, hs, bs, nblk, max_nb = 128, 16, 16, 256, 16, 20000, 128
    lens = rng(seed, _LENS).integers(1024, 2048, size=S, endpoint=True).astype(np.uint32)
    bt = _deal_tables(seed, lens, bs, nblk, max_nb, nblk)
    fill = [np.arange(int(L), dtype=np.int64) for L in lens]
    return Workload("mha256", seed, S, H, Hkv, hs, bs, nblk, bt, lens, 1.0 / 16.0, fill,
                    description="MHA head_size=256 (S=128, H=Hkv=16, bs=16, L~U[1024,2048])")


def mha256_write(w: Optional[Workload] = None, T: int = 4096):
    """The 4096-token cache write of the MHA config: 10% pad slots, 0.5% all-zero
    (token, head) vectors drawn independently for K and V, and distinct slots
    taken from blocks that no block table uses.

    Returns (slot_mapping u32 [T], key f32 [T,Hkv,hs], value f32 [T,Hkv,hs])."""
    w = w or mha256()
    used = np.zeros(w.num_blocks, dtype=bool)
    for s, L in enumerate(w.context_lens):
        used[w.block_tables[s, :-(-int(L) // w.block_size)]] = True
    free_blocks = np.nonzero(~used)[0].astype(np.int64)
    free_slots = (free_blocks[:, None] * w.block_size + np.arange(w.block_size)[None, :]).reshape(-1)
    g = rng(w.seed, _MASKS)
    n_pad = int(round(0.10 * T))
    pad = np.zeros(T, dtype=bool)
    pad[g.choice(T, size=n_pad, replace=False)] = True
    slots = np.full(T, PAD_SLOT, dtype=np.uint32)
    slots[~pad] = g.choice(free_slots, size=T - n_pad, replace=False).astype(np.uint32)
    k, v = w._kv(_STEP_K, _STEP_V, 0, T)
    n_zero = int(round(0.005 * T * w.num_kv_heads))
    for arr in (k, v):
        idx = g.choice(T * w.num_kv_heads, size=n_zero, replace=False)
        arr.reshape(T * w.num_kv_heads, w.head_size)[idx] = 0.0
    return slots, k, v


def selected() -> Workload:
    """Selected-token decode: S=16, H=32, Hkv=4, hs=128, bs=16, 65536-token capacity
    per seq; each seq attends 32 random complete 64-token blocks plus the trailing
    partial block (the indexer's visible-list shape).  Only visible rows are written."""
    seed = 5
    S, H, Hkv, hs, bs = 16, 32, 4, 128, 16
    cap, ratio, budget_blocks = 65536, 64, 32
    nb_seq = cap // bs
    nblk = S * nb_seq
    bt = rng(seed, _TABLES).permutation(nblk).astype(np.uint32).reshape(S, nb_seq)
    g = rng(seed, _VIS)
    tail = g.integers(1, 63, size=S, endpoint=True)
    t_len = cap - ratio + tail                      # positions 0 .. t_len-1 exist
    complete = (cap - ratio) // ratio                # 1023 complete 64-token blocks
    vis_stride = budget_blocks * ratio + ratio       # budget + ratio
    vis = np.zeros((S, vis_stride), dtype=np.uint32)
    nvis = np.zeros(S, dtype=np.uint32)
    fill = []
    for s in range(S):
        blocks = np.sort(g.choice(complete, size=budget_blocks, replace=False))
        pos = np.concatenate([(blocks[:, None] * ratio + np.arange(ratio)[None, :]).reshape(-1),
                              np.arange(complete * ratio, int(t_len[s]))]).astype(np.int64)
        vis[s, :pos.shape[0]] = pos
        nvis[s] = pos.shape[0]
        fill.append(pos)
    return Workload("selected", seed, S, H, Hkv, hs, bs, nblk, bt, t_len.astype(np.uint32),
                    float(np.float32(1.0 / np.sqrt(128.0))), fill, visible_pos=vis, num_visible=nvis,
                    description="selected-token decode (S=16, H=32, Hkv=4, hs=128, bs=16, ~2080 visible rows/seq)")


WORKLOADS = {"tiny": tiny, "llama": llama, "long": long_context, "mha256": mha256, "selected": selected}


def get(name: str) -> Workload:
    return WORKLOADS[name]()
