"""Thin ctypes binding of libq8kv.so.

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
There is no CPU fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PAD_SLOT = 0xFFFFFFFF
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq8kv.so")

_STATUS = {0: "Q8_OK", 1: "Q8_ERR_NULL", 2: "Q8_ERR_SHAPE", 3: "Q8_ERR_WORKSPACE",
           4: "Q8_ERR_HIP", 5: "Q8_ERR_UNSUPPORTED"}


class Q8Error(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        msg = "%s returned %s" % (what, _STATUS.get(status, str(status)))
        if hip_error:
            msg += " (hipError %d)" % hip_error
        super().__init__(msg)
        self.status = status


DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq8kv_debug.so")

_lib = None


def load_library() -> ctypes.CDLL:
    """Load libq8kv.so (built by int8_paged_kv_amd/build.py); raise if it is absent."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def load_debug_library() -> ctypes.CDLL:
    """Load libq8kv_debug.so, the build with device-side content checks
    (q8_bounds_flags reads them back).  It is not the one the other calls here
    use; use_library() swaps it in."""
    return _open(DEBUG_LIB_PATH)


def use_library(lib: Optional[ctypes.CDLL]) -> Optional[ctypes.CDLL]:
    """Make `lib` the library every call of this binding goes to (None: the
    release library on next use); returns the previous one."""
    global _lib
    prev, _lib = _lib, lib
    return prev


def bounds_flags(clear: bool = True) -> int:
    """The current device's flag word of failed content checks (debug build;
    see include/q8kv.h), after waiting for the device."""
    lib = load_library()
    f = ctypes.c_uint32(0)
    st = lib.q8_bounds_flags(ctypes.byref(f), 1 if clear else 0)
    _check(st, "q8_bounds_flags")
    return int(f.value)


def _open(path: str) -> ctypes.CDLL:
    """Open one build of the library and declare its entry points."""
    if not os.path.exists(path):
        raise ImportError("%s is not built; run int8_paged_kv_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    P, U = ctypes.c_void_p, ctypes.c_uint32
    lib.q8_cache_write.argtypes = [P, U, P, U, P, P, P, U, U, U, U, U, P]
    lib.q8_cache_write.restype = ctypes.c_int
    lib.q8_paged_decode_workspace_bytes.argtypes = [U, U, U, U, U, U]
    lib.q8_paged_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.q8_paged_decode.argtypes = [P, P, U, P, P, P, U, P, U, P, P, U,
                                    U, U, U, U, U, U, ctypes.c_float, P, ctypes.c_size_t, P]
    lib.q8_paged_decode.restype = ctypes.c_int
    lib.q8_paged_decode_noalloc.argtypes = [P, P, U, P, P, P, U, P, U, P, P, U,
                                            U, U, U, U, U, U, ctypes.c_float, P]
    lib.q8_paged_decode_noalloc.restype = ctypes.c_int
    lib.q8_decode_step.argtypes = [P, P, U, P, U, P, U, P, P, P, U, P, U,
                                   U, U, U, U, U, U, ctypes.c_float, P, ctypes.c_size_t, P]
    lib.q8_decode_step.restype = ctypes.c_int
    lib.q8_paged_decode_rows.argtypes = [P, P, U, P, P, P, U, P, U, U,
                                         U, U, U, U, U, U, ctypes.c_float, P, ctypes.c_size_t, P]
    lib.q8_paged_decode_rows.restype = ctypes.c_int
    lib.q8_f32_cache_write.argtypes = [P, U, P, U, P, P, P, U, U, U, U, U, P]
    lib.q8_f32_cache_write.restype = ctypes.c_int
    lib.q8_f32_paged_decode_workspace_bytes.argtypes = [U, U, U, U]
    lib.q8_f32_paged_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.q8_f32_paged_decode.argtypes = [P, P, U, P, P, P, U, P, U,
                                        U, U, U, U, U, U, ctypes.c_float, P, ctypes.c_size_t, P]
    lib.q8_f32_paged_decode.restype = ctypes.c_int
    lib.q8_bf16_cache_write.argtypes = [P, U, P, U, P, P, P, U, U, U, U, U, P]
    lib.q8_bf16_cache_write.restype = ctypes.c_int
    lib.q8_bf16_paged_decode_workspace_bytes.argtypes = [U, U, U, U]
    lib.q8_bf16_paged_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.q8_bf16_paged_decode.argtypes = lib.q8_f32_paged_decode.argtypes
    lib.q8_bf16_paged_decode.restype = ctypes.c_int
    F = ctypes.c_float
    lib.q8_rope_table.argtypes = [P, U, U, F, P]
    lib.q8_rope_table.restype = ctypes.c_int
    lib.q8_norm_rope.argtypes = [P, U, P, U, U, U, U, U, P, P, P, U, U, F, P]
    lib.q8_norm_rope.restype = ctypes.c_int
    lib.q8_norm_rope_cache_write.argtypes = [P, U, P, U, P, P, P, P, P, P, U, U, F, U, U, U, U, U, P]
    lib.q8_norm_rope_cache_write.restype = ctypes.c_int
    lib.q8_norm_rope_qk_cache_write.argtypes = [P, U, P, U, U, U, U, P, P, P, U, P, U, P, P, P, P, P, P, U, U,
                                                F, U, U, U, U, U, P]
    lib.q8_norm_rope_qk_cache_write.restype = ctypes.c_int
    lib.q8_norm_rope_decode_step.argtypes = [P, P, U, U, P, U, P, U, P, P, P, U, P, U, P, P, P, U, U, F,
                                             U, U, U, U, U, U, F, P, ctypes.c_size_t, P]
    lib.q8_norm_rope_decode_step.restype = ctypes.c_int
    lib.q8_index_select.argtypes = [P, U, P, U, U, U, P, U, P, P, U, P]
    lib.q8_index_select.restype = ctypes.c_int
    lib.q8_last_hip_error.argtypes = []
    lib.q8_last_hip_error.restype = ctypes.c_int
    lib.q8_status_string.argtypes = [ctypes.c_int]
    lib.q8_status_string.restype = ctypes.c_char_p
    lib.q8_bounds_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
    lib.q8_bounds_flags.restype = ctypes.c_int
    return lib


def _check(status: int, what: str):
    if status != 0:
        lib = load_library()
        raise Q8Error(status, what, lib.q8_last_hip_error() if status == 4 else 0)


def _dev(t: Optional[torch.Tensor], name: str, dtype) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _u32(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    """uint32 arrays travel as int32 or uint32 tensors (same bits)."""
    if t is None:
        return None
    if t.dtype not in (torch.int32, torch.uint32):
        raise ValueError("%s must be an int32/uint32 tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return _dev(t, name, t.dtype)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _rows(x: torch.Tensor, name: str):
    """(pointer, row stride) of a [T, ...] f32 tensor whose rows are dense."""
    if x.dim() < 2 or (x.numel() and not x[0].is_contiguous()):
        raise ValueError("%s must be [T, num_kv_heads, head_size] with dense rows" % name)
    if x.shape[0] == 0:       # no rows: torch's row stride is arbitrary then; report the dense one
        return _dev(x, name, torch.float32), int(torch.Size(x.shape[1:]).numel())
    return _dev(x, name, torch.float32), x.stride(0)


def q8_cache_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, slot_mapping: torch.Tensor, num_kv_heads: int,
                   head_size: int, block_size: int, num_blocks: Optional[int] = None, stream=None) -> None:
    """Quantize + pack K/V rows into the paged caches (see include/q8kv.h)."""
    lib = load_library()
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    wpt = head_size // 4 + 1
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * wpt)
    st = lib.q8_cache_write(kp, ks, vp, vs, _u32(key_cache, "key_cache"), _u32(value_cache, "value_cache"),
                            _u32(slot_mapping, "slot_mapping"), slot_mapping.numel(), num_kv_heads,
                            head_size, block_size, num_blocks, _stream(stream))
    _check(st, "q8_cache_write")


def q8_paged_decode_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                                   block_size: int, max_positions: int) -> int:
    return int(load_library().q8_paged_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads,
                                                             head_size, block_size, max_positions))


def q8_paged_decode(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                    block_tables: torch.Tensor, context_lens: Optional[torch.Tensor], scale: float,
                    num_kv_heads: int, block_size: int, max_context_len: Optional[int] = None,
                    visible_pos: Optional[torch.Tensor] = None, num_visible: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    num_blocks: Optional[int] = None, stream=None) -> torch.Tensor:
    """Decode attention over the int8 paged cache; q is [S, H, hs] f32 (see include/q8kv.h).

    max_context_len must be given in dense mode (reading context_lens would
    synchronize).  In visible-list mode vis_stride is visible_pos.shape[1].
    A caller-provided workspace must have been zero-filled before its first
    use; every call leaves it ready for the next one."""
    lib = load_library()
    if q.dim() != 3 or (q.numel() and not q[0].is_contiguous()):
        raise ValueError("q must be [S, H, head_size] with dense rows")
    S, H, hs = q.shape
    if out is None:
        out = torch.empty((S, H, hs), dtype=torch.float32, device=q.device)
    elif not out.is_contiguous() or tuple(out.shape) != (S, H, hs):
        raise ValueError("out must be a contiguous [S, H, head_size] f32 tensor")
    vis = visible_pos is not None
    if vis:
        if visible_pos.dim() != 2:
            raise ValueError("visible_pos must be [S, vis_stride]")
        vis_stride = visible_pos.shape[1]
        max_pos = vis_stride
        mcl = 0
    else:
        vis_stride = 0
        if max_context_len is None:
            raise ValueError("max_context_len is required in dense mode")
        mcl = int(max_context_len)
        max_pos = mcl
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [S, max_num_blocks_per_seq]")
    wpt = hs // 4 + 1
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * wpt)
    need = lib.q8_paged_decode_workspace_bytes(S, H, num_kv_heads, hs, block_size, max_pos)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)   # zero before first use
    wp = None if workspace is None else workspace.data_ptr()
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.q8_paged_decode(_dev(out, "out", torch.float32), _dev(q, "q", torch.float32), q.stride(0),
                             _u32(key_cache, "key_cache"), _u32(value_cache, "value_cache"),
                             _u32(block_tables, "block_tables"), block_tables.shape[1],
                             _u32(context_lens, "context_lens"), mcl,
                             _u32(visible_pos, "visible_pos"), _u32(num_visible, "num_visible"), vis_stride,
                             S, H, num_kv_heads, hs, block_size, num_blocks, float(scale), wp, wb,
                             _stream(stream))
    _check(st, "q8_paged_decode")
    return out


def q8_paged_decode_noalloc(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: Optional[torch.Tensor], scale: float,
                            num_kv_heads: int, block_size: int, max_context_len: Optional[int] = None,
                            visible_pos: Optional[torch.Tensor] = None, num_visible: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, num_blocks: Optional[int] = None,
                            stream=None) -> torch.Tensor:
    """q8_paged_decode with the library's own scratch array instead of a
    workspace (see include/q8kv.h): nothing is allocated when `out` is given.
    Calls on one GPU must not overlap."""
    lib = load_library()
    if q.dim() != 3 or (q.numel() and not q[0].is_contiguous()):
        raise ValueError("q must be [S, H, head_size] with dense rows")
    S, H, hs = q.shape
    if out is None:
        out = torch.empty((S, H, hs), dtype=torch.float32, device=q.device)
    elif not out.is_contiguous() or tuple(out.shape) != (S, H, hs):
        raise ValueError("out must be a contiguous [S, H, head_size] f32 tensor")
    vis = visible_pos is not None
    if vis:
        if visible_pos.dim() != 2:
            raise ValueError("visible_pos must be [S, vis_stride]")
        vis_stride, mcl = visible_pos.shape[1], 0
    else:
        if max_context_len is None:
            raise ValueError("max_context_len is required in dense mode")
        vis_stride, mcl = 0, int(max_context_len)
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [S, max_num_blocks_per_seq]")
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * (hs // 4 + 1))
    st = lib.q8_paged_decode_noalloc(_dev(out, "out", torch.float32), _dev(q, "q", torch.float32), q.stride(0),
                                     _u32(key_cache, "key_cache"), _u32(value_cache, "value_cache"),
                                     _u32(block_tables, "block_tables"), block_tables.shape[1],
                                     _u32(context_lens, "context_lens"), mcl,
                                     _u32(visible_pos, "visible_pos"), _u32(num_visible, "num_visible"),
                                     vis_stride, S, H, num_kv_heads, hs, block_size, num_blocks, float(scale),
                                     _stream(stream))
    _check(st, "q8_paged_decode_noalloc")
    return out


def q8_decode_step(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                   num_kv_heads: int, block_size: int, max_context_len: int, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, num_blocks: Optional[int] = None,
                   stream=None) -> torch.Tensor:
    """One decode step in one launch: append each sequence's new K/V row at
    position context_lens[s]-1, then attend (see include/q8kv.h).  key and
    value are [S, num_kv_heads * head_size] (or [S, num_kv_heads, head_size])
    f32 with dense rows; the caches are updated in place."""
    lib = load_library()
    if q.dim() != 3 or (q.numel() and not q[0].is_contiguous()):
        raise ValueError("q must be [S, H, head_size] with dense rows")
    S, H, hs = q.shape
    if out is None:
        out = torch.empty((S, H, hs), dtype=torch.float32, device=q.device)
    elif not out.is_contiguous() or tuple(out.shape) != (S, H, hs):
        raise ValueError("out must be a contiguous [S, H, head_size] f32 tensor")
    kp, kst = _rows(key, "key")
    vp, vst = _rows(value, "value")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [S, max_num_blocks_per_seq]")
    wpt = hs // 4 + 1
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * wpt)
    mcl = int(max_context_len)
    need = lib.q8_paged_decode_workspace_bytes(S, H, num_kv_heads, hs, block_size, mcl)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)   # zero before first use
    wp = None if workspace is None else workspace.data_ptr()
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.q8_decode_step(_dev(out, "out", torch.float32), _dev(q, "q", torch.float32), q.stride(0),
                            kp, kst, vp, vst,
                            _u32(key_cache, "key_cache"), _u32(value_cache, "value_cache"),
                            _u32(block_tables, "block_tables"), block_tables.shape[1],
                            _u32(context_lens, "context_lens"), mcl,
                            S, H, num_kv_heads, hs, block_size, num_blocks, float(scale), wp, wb,
                            _stream(stream))
    _check(st, "q8_decode_step")
    return out


def q8_norm_rope_decode_step(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                             value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                             scale: float, num_kv_heads: int, block_size: int, max_context_len: int,
                             q_weight: torch.Tensor, k_weight: torch.Tensor, table: Optional[torch.Tensor], rot: int,
                             eps: float, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                             num_blocks: Optional[int] = None, stream=None) -> torch.Tensor:
    """q8_decode_step with the per-head RMSNorm + partial rotary step applied to q
    and to the new K rows at position context_lens[s]-1, in the same launch (see
    include/q8kv.h).  q is the un-normalized [S, H, head_size] f32 with unit
    element stride; its head stride may exceed head_size (a q/gate interleave,
    e.g. x[:, :, :head_size] of an [S, H, 2*head_size] tensor).  table is
    q8_rope_table's [num_positions, rot] (None when rot == 0)."""
    lib = load_library()
    if q.dim() != 3 or (q.numel() and q.stride(2) != 1):
        raise ValueError("q must be [S, H, head_size] with unit element stride")
    S, H, hs = q.shape
    if out is None:
        out = torch.empty((S, H, hs), dtype=torch.float32, device=q.device)
    elif not out.is_contiguous() or tuple(out.shape) != (S, H, hs):
        raise ValueError("out must be a contiguous [S, H, head_size] f32 tensor")
    kp, kst = _rows(key, "key")
    vp, vst = _rows(value, "value")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [S, max_num_blocks_per_seq]")
    wpt = hs // 4 + 1
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * wpt)
    mcl = int(max_context_len)
    need = lib.q8_paged_decode_workspace_bytes(S, H, num_kv_heads, hs, block_size, mcl)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)   # zero before first use
    wp = None if workspace is None else workspace.data_ptr()
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    num_positions = table.shape[0] if (table is not None and rot) else 0
    tab = _dev(table, "table", torch.float32) if (table is not None and rot) else None
    st = lib.q8_norm_rope_decode_step(_dev(out, "out", torch.float32), _dev(q, "q", torch.float32), q.stride(0),
                                      q.stride(1), kp, kst, vp, vst,
                                      _u32(key_cache, "key_cache"), _u32(value_cache, "value_cache"),
                                      _u32(block_tables, "block_tables"), block_tables.shape[1],
                                      _u32(context_lens, "context_lens"), mcl,
                                      _dev(q_weight, "q_weight", torch.float32),
                                      _dev(k_weight, "k_weight", torch.float32), tab, int(rot), num_positions,
                                      float(eps), S, H, num_kv_heads, hs, block_size, num_blocks, float(scale), wp,
                                      wb, _stream(stream))
    _check(st, "q8_norm_rope_decode_step")
    return out


def q8_paged_decode_rows(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, num_kv_heads: int,
                         block_size: int, max_context_len: int, rows_per_seq: int,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         num_blocks: Optional[int] = None, stream=None) -> torch.Tensor:
    """Multi-row causal decode (see include/q8kv.h): q is [S * nb, H, hs] f32
    (row b of sequence s at s*nb + b); row b attends the first
    context_lens[s] - nb + b + 1 positions.  Returns out [S * nb, H, hs]."""
    lib = load_library()
    if q.dim() != 3 or (q.numel() and not q[0].is_contiguous()):
        raise ValueError("q must be [S * rows_per_seq, H, head_size] with dense rows")
    R, H, hs = q.shape
    nb = int(rows_per_seq)
    if nb < 1 or R % nb:
        raise ValueError("q's row count must be a multiple of rows_per_seq")
    S = R // nb
    if out is None:
        out = torch.empty((R, H, hs), dtype=torch.float32, device=q.device)
    elif not out.is_contiguous() or tuple(out.shape) != (R, H, hs):
        raise ValueError("out must be a contiguous [S * rows_per_seq, H, head_size] f32 tensor")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [S, max_num_blocks_per_seq]")
    wpt = hs // 4 + 1
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * wpt)
    mcl = int(max_context_len)
    need = lib.q8_paged_decode_workspace_bytes(S, H * nb, num_kv_heads, hs, block_size, mcl)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)   # zero before first use
    wp = None if workspace is None else workspace.data_ptr()
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.q8_paged_decode_rows(_dev(out, "out", torch.float32), _dev(q, "q", torch.float32), q.stride(0),
                                  _u32(key_cache, "key_cache"), _u32(value_cache, "value_cache"),
                                  _u32(block_tables, "block_tables"), block_tables.shape[1],
                                  _u32(context_lens, "context_lens"), mcl, nb,
                                  S, H, num_kv_heads, hs, block_size, num_blocks, float(scale), wp, wb,
                                  _stream(stream))
    _check(st, "q8_paged_decode_rows")
    return out


def q8_f32_cache_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, slot_mapping: torch.Tensor, num_kv_heads: int,
                       head_size: int, block_size: int, num_blocks: Optional[int] = None, stream=None) -> None:
    """Copy K/V rows into the f32 paged caches [num_blocks, Hkv, block_size, head_size] (baseline)."""
    lib = load_library()
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * head_size)
    st = lib.q8_f32_cache_write(kp, ks, vp, vs, _dev(key_cache, "key_cache", torch.float32),
                                _dev(value_cache, "value_cache", torch.float32),
                                _u32(slot_mapping, "slot_mapping"), slot_mapping.numel(), num_kv_heads,
                                head_size, block_size, num_blocks, _stream(stream))
    _check(st, "q8_f32_cache_write")


def q8_f32_paged_decode_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int) -> int:
    return int(load_library().q8_f32_paged_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size))


def q8_f32_paged_decode(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                        num_kv_heads: int, block_size: int, max_context_len: Optional[int] = None,
                        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        num_blocks: Optional[int] = None, stream=None) -> torch.Tensor:
    """Single-query decode over the f32 paged caches (baseline); q is [S, H, hs] with dense heads.

    A caller-provided workspace must have been zero-filled before its first
    use; every completed call leaves it ready for the next.
    """
    lib = load_library()
    if q.dim() != 3 or q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [num_seqs, num_heads, head_size] with dense heads")
    S, H, hs = q.shape
    if out is None:
        out = torch.empty((S, H, hs), dtype=torch.float32, device=q.device)
    if not out.is_contiguous() or tuple(out.shape) != (S, H, hs):
        raise ValueError("out must be a dense [num_seqs, num_heads, head_size] tensor")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if context_lens.numel() else 0
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * hs)
    need = lib.q8_f32_paged_decode_workspace_bytes(S, H, num_kv_heads, hs)
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)   # zero before first use
    wp = workspace.data_ptr()
    wb = workspace.numel() * workspace.element_size()
    st = lib.q8_f32_paged_decode(_dev(out, "out", torch.float32), _dev(q, "q", torch.float32), q.stride(0),
                                 _dev(key_cache, "key_cache", torch.float32),
                                 _dev(value_cache, "value_cache", torch.float32),
                                 _u32(block_tables, "block_tables"), block_tables.shape[-1],
                                 _u32(context_lens, "context_lens"), max_context_len, S, H, num_kv_heads, hs,
                                 block_size, num_blocks, float(scale), wp, wb, _stream(stream))
    _check(st, "q8_f32_paged_decode")
    return out


def _bf16(t: torch.Tensor, name: str) -> int:
    """bfloat16 caches travel as torch.bfloat16 or int16 tensors (the same bits)."""
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype not in (torch.bfloat16, torch.int16):
        raise ValueError("%s must be bfloat16 (or int16 holding bfloat16 bits), got %s" % (name, t.dtype))
    return t.data_ptr()


def q8_bf16_cache_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                        value_cache: torch.Tensor, slot_mapping: torch.Tensor, num_kv_heads: int,
                        head_size: int, block_size: int, num_blocks: Optional[int] = None, stream=None) -> None:
    """Round K/V rows to bfloat16 (nearest, ties to even) into the bf16 paged caches
    [num_blocks, Hkv, block_size, head_size] (baseline)."""
    lib = load_library()
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * head_size)
    st = lib.q8_bf16_cache_write(kp, ks, vp, vs, _bf16(key_cache, "key_cache"), _bf16(value_cache, "value_cache"),
                                 _u32(slot_mapping, "slot_mapping"), slot_mapping.numel(), num_kv_heads,
                                 head_size, block_size, num_blocks, _stream(stream))
    _check(st, "q8_bf16_cache_write")


def q8_bf16_paged_decode_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int) -> int:
    return int(load_library().q8_bf16_paged_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size))


def q8_bf16_paged_decode(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                         num_kv_heads: int, block_size: int, max_context_len: Optional[int] = None,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         num_blocks: Optional[int] = None, stream=None) -> torch.Tensor:
    """Single-query decode over the bf16 paged caches (baseline); arguments as q8_f32_paged_decode."""
    lib = load_library()
    if q.dim() != 3 or q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("q must be [num_seqs, num_heads, head_size] with dense heads")
    S, H, hs = q.shape
    if out is None:
        out = torch.empty((S, H, hs), dtype=torch.float32, device=q.device)
    if not out.is_contiguous() or tuple(out.shape) != (S, H, hs):
        raise ValueError("out must be a dense [num_seqs, num_heads, head_size] tensor")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if context_lens.numel() else 0
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * hs)
    need = lib.q8_bf16_paged_decode_workspace_bytes(S, H, num_kv_heads, hs)
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)   # zero before first use
    wp = workspace.data_ptr()
    wb = workspace.numel() * workspace.element_size()
    st = lib.q8_bf16_paged_decode(_dev(out, "out", torch.float32), _dev(q, "q", torch.float32), q.stride(0),
                                  _bf16(key_cache, "key_cache"), _bf16(value_cache, "value_cache"),
                                  _u32(block_tables, "block_tables"), block_tables.shape[-1],
                                  _u32(context_lens, "context_lens"), max_context_len, S, H, num_kv_heads, hs,
                                  block_size, num_blocks, float(scale), wp, wb, _stream(stream))
    _check(st, "q8_bf16_paged_decode")
    return out


def q8_rope_table(num_positions: int, rot: int, theta: float, device=None, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Rotary table [num_positions, rot] f32: cos, then sin, of p * theta^(-2i/rot), i < rot/2."""
    lib = load_library()
    if out is None:
        out = torch.empty((num_positions, rot), dtype=torch.float32, device=device or "cuda")
    if not out.is_contiguous() or out.numel() != num_positions * rot:
        raise ValueError("out must be a dense [num_positions, rot] tensor")
    ptr = _dev(out, "table", torch.float32) if out.numel() else None
    _check(lib.q8_rope_table(ptr, num_positions, rot, float(theta), _stream(stream)), "q8_rope_table")
    return out


def q8_norm_rope(x: torch.Tensor, positions: Optional[torch.Tensor], weight: torch.Tensor,
                 table: Optional[torch.Tensor], rot: int, eps: float, num_heads: int, head_size: int,
                 head_stride: Optional[int] = None, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Per-head RMSNorm + partial rotary step on rows of heads (x is [T, ...] with dense rows;
    head h of row t starts at element h*head_stride of the row).  Returns [T, num_heads, head_size]."""
    lib = load_library()
    T = x.shape[0]
    xp, xs = _rows(x, "x")
    hst = head_size if head_stride is None else head_stride
    if out is None:
        out = torch.empty((T, num_heads, head_size), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (T, num_heads, head_size) or not out.is_contiguous():
        raise ValueError("out must be a dense [T, num_heads, head_size] tensor")
    num_positions = table.shape[0] if (table is not None and rot) else 0
    st = lib.q8_norm_rope(_dev(out, "out", torch.float32), num_heads * head_size, xp, xs, hst, T, num_heads,
                          head_size, _u32(positions, "positions") if positions is not None else None,
                          _dev(weight, "weight", torch.float32),
                          _dev(table, "table", torch.float32) if (table is not None and rot) else None,
                          rot, num_positions, float(eps), _stream(stream))
    _check(st, "q8_norm_rope")
    return out


def q8_norm_rope_cache_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                             value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                             positions: Optional[torch.Tensor], weight: torch.Tensor,
                             table: Optional[torch.Tensor], rot: int, eps: float, num_kv_heads: int,
                             head_size: int, block_size: int, num_blocks: Optional[int] = None,
                             stream=None) -> None:
    """q8_cache_write with K normalized and rotated at positions[t] first (see include/q8kv.h)."""
    lib = load_library()
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    wpt = head_size // 4 + 1
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * wpt)
    num_positions = table.shape[0] if (table is not None and rot) else 0
    st = lib.q8_norm_rope_cache_write(kp, ks, vp, vs, _u32(key_cache, "key_cache"), _u32(value_cache, "value_cache"),
                                      _u32(slot_mapping, "slot_mapping"),
                                      _u32(positions, "positions") if positions is not None else None,
                                      _dev(weight, "weight", torch.float32),
                                      _dev(table, "table", torch.float32) if (table is not None and rot) else None,
                                      rot, num_positions, float(eps), slot_mapping.numel(), num_kv_heads,
                                      head_size, block_size, num_blocks, _stream(stream))
    _check(st, "q8_norm_rope_cache_write")


def q8_norm_rope_qk_cache_write(q: torch.Tensor, q_positions: Optional[torch.Tensor], q_weight: torch.Tensor,
                                num_heads: int, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                                value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                                positions: Optional[torch.Tensor], k_weight: torch.Tensor,
                                table: Optional[torch.Tensor], rot: int, eps: float, num_kv_heads: int,
                                head_size: int, block_size: int, num_blocks: Optional[int] = None,
                                q_head_stride: Optional[int] = None, q_out: Optional[torch.Tensor] = None,
                                stream=None) -> torch.Tensor:
    """q8_norm_rope on q rows and q8_norm_rope_cache_write on the new K/V rows in one launch
    (see include/q8kv.h).  Returns q_out [T_q, num_heads, head_size]."""
    lib = load_library()
    Tq = q.shape[0]
    qp, qs = _rows(q, "q")
    hst = head_size if q_head_stride is None else q_head_stride
    if q_out is None:
        q_out = torch.empty((Tq, num_heads, head_size), dtype=torch.float32, device=q.device)
    if tuple(q_out.shape) != (Tq, num_heads, head_size) or not q_out.is_contiguous():
        raise ValueError("q_out must be a dense [T, num_heads, head_size] tensor")
    kp, ks = _rows(key, "key")
    vp, vs = _rows(value, "value")
    wpt = head_size // 4 + 1
    if num_blocks is None:
        num_blocks = key_cache.numel() // max(1, num_kv_heads * block_size * wpt)
    num_positions = table.shape[0] if (table is not None and rot) else 0
    tab = _dev(table, "table", torch.float32) if (table is not None and rot) else None
    st = lib.q8_norm_rope_qk_cache_write(
        _dev(q_out, "q_out", torch.float32), num_heads * head_size, qp, qs, hst, Tq, num_heads,
        _u32(q_positions, "q_positions") if q_positions is not None else None, _dev(q_weight, "q_weight", torch.float32),
        kp, ks, vp, vs, _u32(key_cache, "key_cache"), _u32(value_cache, "value_cache"),
        _u32(slot_mapping, "slot_mapping"), _u32(positions, "positions") if positions is not None else None,
        _dev(k_weight, "k_weight", torch.float32), tab, rot, num_positions, float(eps), slot_mapping.numel(),
        num_kv_heads, head_size, block_size, num_blocks, _stream(stream))
    _check(st, "q8_norm_rope_qk_cache_write")
    return q_out


def q8_index_select(scores: torch.Tensor, row_lens: torch.Tensor, ratio: int, k: int, vis_stride: int,
                    visible_pos: Optional[torch.Tensor] = None, num_visible: Optional[torch.Tensor] = None,
                    mask_stride: int = 0, visible_mask: Optional[torch.Tensor] = None, stream=None):
    """Visible lists from block scores [rows, max_blocks] (see include/q8kv.h).
    Returns (visible_pos [rows, vis_stride], num_visible [rows]) as int32 tensors of u32 bits;
    with mask_stride > 0 also the block bitmask [rows, mask_stride] as a third element."""
    lib = load_library()
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be [rows, max_blocks] with dense rows")
    R = scores.shape[0]
    if visible_pos is None:
        visible_pos = torch.zeros((R, vis_stride), dtype=torch.int32, device=scores.device)
    if num_visible is None:
        num_visible = torch.zeros((R,), dtype=torch.int32, device=scores.device)
    if mask_stride and visible_mask is None:
        visible_mask = torch.zeros((R, mask_stride), dtype=torch.int32, device=scores.device)
    if visible_mask is not None and (not mask_stride or tuple(visible_mask.shape) != (R, mask_stride)
                                     or not visible_mask.is_contiguous()):
        raise ValueError("visible_mask must be a contiguous [rows, mask_stride] tensor")
    st = lib.q8_index_select(_dev(scores, "scores", torch.float32), scores.stride(0), _u32(row_lens, "row_lens"), R,
                             ratio, k, _u32(visible_pos, "visible_pos"), vis_stride, _u32(num_visible, "num_visible"),
                             _u32(visible_mask, "visible_mask"), mask_stride, _stream(stream))
    _check(st, "q8_index_select")
    return (visible_pos, num_visible, visible_mask) if mask_stride else (visible_pos, num_visible)
