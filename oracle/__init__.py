"""CPU oracle for the int8 paged KV cache (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never do: the two implementations share no code.

The arithmetic lives in ``q8_oracle.c`` (plain C, binary32 quantizer and
binary64 decode); this module only builds it with gcc and marshals numpy arrays
through ctypes.  Each C function cites the page passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_oracle.c")
_LIB = os.path.join(_HERE, "libq8oracle.so")
PAD_SLOT = 0xFFFFFFFF

_ERRORS = {1: "shape", 2: "index out of range", 3: "input outside the contract", 4: "out of memory"}


def build(force: bool = True) -> str:
    """Compile q8_oracle.c into libq8oracle.so next to it (gcc, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        U = ctypes.c_uint32
        lib.q8o_quantize_row.argtypes = [P, U, P]
        lib.q8o_quantize_row.restype = ctypes.c_int
        lib.q8o_dequantize_row.argtypes = [P, U, P]
        lib.q8o_dequantize_row.restype = None
        lib.q8o_cache_write.argtypes = [P, U, P, U, P, P, P, U, U, U, U, U]
        lib.q8o_cache_write.restype = ctypes.c_int
        dec = [P, U, P, P, P, U, P, U, P, P, U, U, U, U, U, U, U, ctypes.c_float, ctypes.c_int]
        lib.q8o_paged_decode.argtypes = [P] + dec
        lib.q8o_paged_decode.restype = ctypes.c_int
        lib.q8o_paged_decode_units.argtypes = [P, P, U] + dec
        lib.q8o_paged_decode_units.restype = ctypes.c_int
        lib.q8o_f32_cache_write.argtypes = [P, U, P, U, P, P, P, U, U, U, U, U]
        lib.q8o_f32_cache_write.restype = ctypes.c_int
        f32dec = [P, U, P, P, P, U, P, U, U, U, U, U, U, U, ctypes.c_float, ctypes.c_int]
        lib.q8o_f32_paged_decode.argtypes = [P] + f32dec
        lib.q8o_f32_paged_decode.restype = ctypes.c_int
        lib.q8o_f32_paged_decode_units.argtypes = [P, P, U] + f32dec
        lib.q8o_f32_paged_decode_units.restype = ctypes.c_int
        lib.q8o_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.q8o_f32_to_bf16.restype = ctypes.c_uint16
        lib.q8o_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.q8o_bf16_to_f32.restype = ctypes.c_float
        lib.q8o_bf16_cache_write.argtypes = [P, U, P, U, P, P, P, U, U, U, U, U]
        lib.q8o_bf16_cache_write.restype = ctypes.c_int
        lib.q8o_bf16_paged_decode.argtypes = [P] + f32dec
        lib.q8o_bf16_paged_decode.restype = ctypes.c_int
        lib.q8o_bf16_paged_decode_units.argtypes = [P, P, U] + f32dec
        lib.q8o_bf16_paged_decode_units.restype = ctypes.c_int
        F = ctypes.c_float
        lib.q8o_rope_table.argtypes = [P, U, U, F]
        lib.q8o_rope_table.restype = ctypes.c_int
        lib.q8o_norm_rope_row.argtypes = [P, U, P, P, U, F, P]
        lib.q8o_norm_rope_row.restype = ctypes.c_int
        lib.q8o_norm_rope_row_f64.argtypes = [P, U, P, U, U, ctypes.c_double, ctypes.c_double, P]
        lib.q8o_norm_rope_row_f64.restype = ctypes.c_int
        lib.q8o_norm_rope.argtypes = [P, U, P, U, U, U, U, U, P, P, P, U, U, F]
        lib.q8o_norm_rope.restype = ctypes.c_int
        lib.q8o_norm_rope_cache_write.argtypes = [P, U, P, U, P, P, P, P, P, P, U, U, F, U, U, U, U, U]
        lib.q8o_norm_rope_cache_write.restype = ctypes.c_int
        lib.q8o_index_select.argtypes = [P, U, P, U, U, U, P, U, P, P, U]
        lib.q8o_index_select.restype = ctypes.c_int
        lib.q8o_max_threads.argtypes = []
        lib.q8o_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed: %s (code %d)" % (what, _ERRORS.get(rc, "?"), rc))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().q8o_max_threads())


def quantize_row(x) -> np.ndarray:
    """Pack one f32 vector into head_size/4 code words plus one scale word."""
    x = _c(x, np.float32)
    hs = x.shape[-1]
    row = np.zeros(hs // 4 + 1, dtype=np.uint32)
    _check(_load().q8o_quantize_row(_ptr(x), hs, _ptr(row)), "quantize_row")
    return row


def quantize_rows(x) -> np.ndarray:
    """Apply quantize_row to every vector along the last axis."""
    x = _c(x, np.float32)
    hs = x.shape[-1]
    flat = x.reshape(-1, hs)
    out = np.zeros((flat.shape[0], hs // 4 + 1), dtype=np.uint32)
    lib = _load()
    for i in range(flat.shape[0]):
        _check(lib.q8o_quantize_row(_ptr(flat[i]), hs, _ptr(out[i])), "quantize_row")
    return out.reshape(x.shape[:-1] + (hs // 4 + 1,))


def dequantize_row(row, head_size: int) -> np.ndarray:
    row = _c(row, np.uint32)
    out = np.zeros(head_size, dtype=np.float64)
    _load().q8o_dequantize_row(_ptr(row), head_size, _ptr(out))
    return out


def cache_write(key, value, key_cache, value_cache, slot_mapping, num_kv_heads, head_size,
                block_size, num_blocks=None, key_stride=None, value_stride=None):
    """Quantize + pack K and V rows into the caches, in place (numpy u32 arrays).

    key/value: f32 arrays whose first axis is the token; row t's head h starts at
    t*stride + h*head_size in the flattened array.
    """
    key = _c(key, np.float32)
    value = _c(value, np.float32)
    slot_mapping = _c(slot_mapping, np.uint32)
    for c in (key_cache, value_cache):
        if c.dtype != np.uint32 or not c.flags.c_contiguous:
            raise ValueError("caches must be contiguous uint32 arrays")
    T = slot_mapping.shape[0]
    ks = key_stride if key_stride is not None else (key.size // T if T else num_kv_heads * head_size)
    vs = value_stride if value_stride is not None else (value.size // T if T else num_kv_heads * head_size)
    wpt = head_size // 4 + 1
    nb = num_blocks if num_blocks is not None else key_cache.size // (num_kv_heads * block_size * wpt)
    _check(_load().q8o_cache_write(_ptr(key), ks, _ptr(value), vs, _ptr(key_cache),
                                   _ptr(value_cache), _ptr(slot_mapping), T, num_kv_heads,
                                   head_size, block_size, nb), "cache_write")


def _decode_common(q, key_cache, value_cache, block_tables, context_lens, max_context_len,
                   num_kv_heads, block_size, visible_pos, num_visible, vis_stride, num_blocks):
    q = _c(q, np.float32)
    S, H, hs = q.shape
    bt = _c(block_tables, np.uint32)
    cl = _c(context_lens, np.uint32)
    vp = None if visible_pos is None else _c(visible_pos, np.uint32)
    nv = None if num_visible is None else _c(num_visible, np.uint32)
    if vp is not None and vis_stride is None:
        vis_stride = vp.shape[-1]
    wpt = hs // 4 + 1
    nb = num_blocks if num_blocks is not None else key_cache.size // (num_kv_heads * block_size * wpt)
    if max_context_len is None:
        max_context_len = int(cl.max()) if cl.size else 0
    return q, S, H, hs, bt, cl, vp, nv, vis_stride or 0, nb, max_context_len


def paged_decode(q, key_cache, value_cache, block_tables, context_lens, scale, num_kv_heads,
                 block_size, max_context_len=None, visible_pos=None, num_visible=None,
                 vis_stride=None, num_blocks=None, nthreads=0) -> np.ndarray:
    """Decode every (seq, head); q is [S, H, hs] f32, result [S, H, hs] f32."""
    q, S, H, hs, bt, cl, vp, nv, vstr, nb, mcl = _decode_common(
        q, key_cache, value_cache, block_tables, context_lens, max_context_len, num_kv_heads,
        block_size, visible_pos, num_visible, vis_stride, num_blocks)
    out = np.zeros((S, H, hs), dtype=np.float32)
    _check(_load().q8o_paged_decode(_ptr(out), _ptr(q), H * hs, _ptr(key_cache), _ptr(value_cache),
                                    _ptr(bt), bt.shape[-1], _ptr(cl), mcl, _ptr(vp), _ptr(nv), vstr,
                                    S, H, num_kv_heads, hs, block_size, nb, float(scale), nthreads),
           "paged_decode")
    return out


def paged_decode_units(units, q, key_cache, value_cache, block_tables, context_lens, scale,
                       num_kv_heads, block_size, max_context_len=None, visible_pos=None,
                       num_visible=None, vis_stride=None, num_blocks=None, nthreads=0) -> np.ndarray:
    """Decode only the listed (seq, head) pairs; result [len(units), hs] f32."""
    q, S, H, hs, bt, cl, vp, nv, vstr, nb, mcl = _decode_common(
        q, key_cache, value_cache, block_tables, context_lens, max_context_len, num_kv_heads,
        block_size, visible_pos, num_visible, vis_stride, num_blocks)
    u = _c(np.asarray(units).reshape(-1, 2), np.uint32)
    out = np.zeros((u.shape[0], hs), dtype=np.float32)
    _check(_load().q8o_paged_decode_units(_ptr(out), _ptr(u), u.shape[0], _ptr(q), H * hs,
                                          _ptr(key_cache), _ptr(value_cache), _ptr(bt), bt.shape[-1],
                                          _ptr(cl), mcl, _ptr(vp), _ptr(nv), vstr, S, H,
                                          num_kv_heads, hs, block_size, nb, float(scale), nthreads),
           "paged_decode_units")
    return out


# ---- f32 cache baseline: layout [num_blocks, num_kv_heads, block_size, head_size] f32 ----

def f32_cache_write(key, value, key_cache, value_cache, slot_mapping, num_kv_heads, head_size,
                    block_size, num_blocks=None, key_stride=None, value_stride=None):
    """Copy K and V rows into the f32 caches at their slots, in place (numpy f32 arrays)."""
    key = _c(key, np.float32)
    value = _c(value, np.float32)
    slot_mapping = _c(slot_mapping, np.uint32)
    for c in (key_cache, value_cache):
        if c.dtype != np.float32 or not c.flags.c_contiguous:
            raise ValueError("f32 caches must be contiguous float32 arrays")
    T = slot_mapping.shape[0]
    ks = key_stride if key_stride is not None else (key.size // T if T else num_kv_heads * head_size)
    vs = value_stride if value_stride is not None else (value.size // T if T else num_kv_heads * head_size)
    nb = num_blocks if num_blocks is not None else key_cache.size // (num_kv_heads * block_size * head_size)
    _check(_load().q8o_f32_cache_write(_ptr(key), ks, _ptr(value), vs, _ptr(key_cache), _ptr(value_cache),
                                       _ptr(slot_mapping), T, num_kv_heads, head_size, block_size, nb),
           "f32_cache_write")


def _f32_common(q, key_cache, block_tables, context_lens, max_context_len, num_kv_heads, block_size,
                num_blocks):
    q = _c(q, np.float32)
    S, H, hs = q.shape
    bt = _c(block_tables, np.uint32)
    cl = _c(context_lens, np.uint32)
    for c in (key_cache,):
        if c.dtype != np.float32 or not c.flags.c_contiguous:
            raise ValueError("f32 caches must be contiguous float32 arrays")
    nb = num_blocks if num_blocks is not None else key_cache.size // (num_kv_heads * block_size * hs)
    if max_context_len is None:
        max_context_len = int(cl.max()) if cl.size else 0
    return q, S, H, hs, bt, cl, nb, max_context_len


def f32_paged_decode(q, key_cache, value_cache, block_tables, context_lens, scale, num_kv_heads,
                     block_size, max_context_len=None, num_blocks=None, nthreads=0) -> np.ndarray:
    """Decode every (seq, head) over an f32 paged cache; result [S, H, hs] f32."""
    q, S, H, hs, bt, cl, nb, mcl = _f32_common(q, key_cache, block_tables, context_lens,
                                               max_context_len, num_kv_heads, block_size, num_blocks)
    out = np.zeros((S, H, hs), dtype=np.float32)
    _check(_load().q8o_f32_paged_decode(_ptr(out), _ptr(q), H * hs, _ptr(key_cache), _ptr(value_cache),
                                        _ptr(bt), bt.shape[-1], _ptr(cl), mcl, S, H, num_kv_heads, hs,
                                        block_size, nb, float(scale), nthreads), "f32_paged_decode")
    return out


def f32_paged_decode_units(units, q, key_cache, value_cache, block_tables, context_lens, scale,
                           num_kv_heads, block_size, max_context_len=None, num_blocks=None,
                           nthreads=0) -> np.ndarray:
    """Decode only the listed (seq, head) pairs over an f32 cache; result [len(units), hs] f32."""
    q, S, H, hs, bt, cl, nb, mcl = _f32_common(q, key_cache, block_tables, context_lens,
                                               max_context_len, num_kv_heads, block_size, num_blocks)
    u = _c(np.asarray(units).reshape(-1, 2), np.uint32)
    out = np.zeros((u.shape[0], hs), dtype=np.float32)
    _check(_load().q8o_f32_paged_decode_units(_ptr(out), _ptr(u), u.shape[0], _ptr(q), H * hs,
                                              _ptr(key_cache), _ptr(value_cache), _ptr(bt), bt.shape[-1],
                                              _ptr(cl), mcl, S, H, num_kv_heads, hs, block_size, nb,
                                              float(scale), nthreads), "f32_paged_decode_units")
    return out


# ---------------------------------------------------------------- bf16 baseline ----

def f32_to_bf16(x) -> np.ndarray:
    """Round f32 values to bfloat16 (nearest, ties to even); returns their uint16 encodings."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = _load().q8o_f32_to_bf16
    return np.array([f(float(v)) for v in x.reshape(-1)], dtype=np.uint16).reshape(x.shape)


def bf16_to_f32(b) -> np.ndarray:
    """bfloat16 encodings (uint16) read as f32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_cache_write(key, value, key_cache, value_cache, slot_mapping, num_kv_heads, head_size,
                     block_size, num_blocks=None, key_stride=None, value_stride=None):
    """Round K and V rows to bfloat16 into the bf16 caches at their slots, in place (uint16 arrays)."""
    key = _c(key, np.float32)
    value = _c(value, np.float32)
    slot_mapping = _c(slot_mapping, np.uint32)
    for c in (key_cache, value_cache):
        if c.dtype != np.uint16 or not c.flags.c_contiguous:
            raise ValueError("bf16 caches must be contiguous uint16 arrays")
    T = slot_mapping.shape[0]
    ks = key_stride if key_stride is not None else (key.size // T if T else num_kv_heads * head_size)
    vs = value_stride if value_stride is not None else (value.size // T if T else num_kv_heads * head_size)
    nb = num_blocks if num_blocks is not None else key_cache.size // (num_kv_heads * block_size * head_size)
    _check(_load().q8o_bf16_cache_write(_ptr(key), ks, _ptr(value), vs, _ptr(key_cache), _ptr(value_cache),
                                        _ptr(slot_mapping), T, num_kv_heads, head_size, block_size, nb),
           "bf16_cache_write")


def _bf16_common(q, key_cache, block_tables, context_lens, max_context_len, num_kv_heads, block_size,
                 num_blocks):
    q = _c(q, np.float32)
    S, H, hs = q.shape
    bt = _c(block_tables, np.uint32)
    cl = _c(context_lens, np.uint32)
    if key_cache.dtype != np.uint16 or not key_cache.flags.c_contiguous:
        raise ValueError("bf16 caches must be contiguous uint16 arrays")
    nb = num_blocks if num_blocks is not None else key_cache.size // (num_kv_heads * block_size * hs)
    if max_context_len is None:
        max_context_len = int(cl.max()) if cl.size else 0
    return q, S, H, hs, bt, cl, nb, max_context_len


def bf16_paged_decode(q, key_cache, value_cache, block_tables, context_lens, scale, num_kv_heads,
                      block_size, max_context_len=None, num_blocks=None, nthreads=0) -> np.ndarray:
    """Decode every (seq, head) over a bf16 paged cache; result [S, H, hs] f32."""
    q, S, H, hs, bt, cl, nb, mcl = _bf16_common(q, key_cache, block_tables, context_lens,
                                                max_context_len, num_kv_heads, block_size, num_blocks)
    out = np.zeros((S, H, hs), dtype=np.float32)
    _check(_load().q8o_bf16_paged_decode(_ptr(out), _ptr(q), H * hs, _ptr(key_cache), _ptr(value_cache),
                                         _ptr(bt), bt.shape[-1], _ptr(cl), mcl, S, H, num_kv_heads, hs,
                                         block_size, nb, float(scale), nthreads), "bf16_paged_decode")
    return out


def bf16_paged_decode_units(units, q, key_cache, value_cache, block_tables, context_lens, scale,
                            num_kv_heads, block_size, max_context_len=None, num_blocks=None,
                            nthreads=0) -> np.ndarray:
    """Decode only the listed (seq, head) pairs over a bf16 cache; result [len(units), hs] f32."""
    q, S, H, hs, bt, cl, nb, mcl = _bf16_common(q, key_cache, block_tables, context_lens,
                                                max_context_len, num_kv_heads, block_size, num_blocks)
    u = _c(np.asarray(units).reshape(-1, 2), np.uint32)
    out = np.zeros((u.shape[0], hs), dtype=np.float32)
    _check(_load().q8o_bf16_paged_decode_units(_ptr(out), _ptr(u), u.shape[0], _ptr(q), H * hs,
                                               _ptr(key_cache), _ptr(value_cache), _ptr(bt), bt.shape[-1],
                                               _ptr(cl), mcl, S, H, num_kv_heads, hs, block_size, nb,
                                               float(scale), nthreads), "bf16_paged_decode_units")
    return out


# ---------------------------------------------------------------- norm + rotary ----

def rope_table(num_positions: int, rot: int, theta: float) -> np.ndarray:
    """[num_positions, rot] f32: cos then sin of p * theta^(-2i/rot), i < rot/2."""
    t = np.zeros((num_positions, max(rot, 1)), dtype=np.float32)
    _check(_load().q8o_rope_table(_ptr(t), num_positions, rot, float(theta)), "rope_table")
    return t[:, :rot] if rot else t[:, :0]


def norm_rope_row(x, weight, cs_row, rot: int, eps: float) -> np.ndarray:
    """One head vector through RMSNorm (weight) and the rotary step (table row cs_row)."""
    x = _c(x, np.float32)
    w = _c(weight, np.float32)
    cs = _c(cs_row if rot else np.zeros(1, np.float32), np.float32)
    y = np.zeros(x.shape[-1], dtype=np.float32)
    _check(_load().q8o_norm_rope_row(_ptr(x), x.shape[-1], _ptr(w), _ptr(cs), rot, float(eps), _ptr(y)),
           "norm_rope_row")
    return y


def norm_rope_row_f64(x, weight, pos: int, rot: int, theta: float, eps: float) -> np.ndarray:
    """The same definition in binary64 throughout, angles straight from theta."""
    x = _c(x, np.float32)
    w = _c(weight, np.float32)
    y = np.zeros(x.shape[-1], dtype=np.float64)
    _check(_load().q8o_norm_rope_row_f64(_ptr(x), x.shape[-1], _ptr(w), int(pos), rot, float(theta),
                                         float(eps), _ptr(y)), "norm_rope_row_f64")
    return y


def norm_rope(x, positions, weight, table, rot: int, eps: float, num_heads: int, head_size: int,
              x_stride=None, head_stride=None, out_stride=None, out=None) -> np.ndarray:
    """Rows of heads: head h of row t at x.flat[t*x_stride + h*head_stride], written
    to out.flat[t*out_stride + h*head_size]; returns [num_rows, num_heads,
    head_size] f32 (or, with out_stride and out given, out itself, written in place)."""
    x = _c(x, np.float32)
    positions = _c(positions, np.uint32)
    T = positions.shape[0]
    hst = head_size if head_stride is None else head_stride
    xs = x_stride if x_stride is not None else (x.size // T if T else num_heads * hst)
    table = _c(table if rot else np.zeros((1, 1), np.float32), np.float32)
    os_ = num_heads * head_size if out_stride is None else out_stride
    if out is None:
        out = np.zeros((T, num_heads, head_size) if out_stride is None else (T, os_), dtype=np.float32)
    if out.dtype != np.float32 or not out.flags.c_contiguous or out.size < T * os_:
        raise ValueError("out must be a contiguous f32 array of num_rows * out_stride elements")
    _check(_load().q8o_norm_rope(_ptr(out), os_, _ptr(x), xs, hst, T, num_heads, head_size,
                                 _ptr(positions), _ptr(_c(weight, np.float32)), _ptr(table), rot,
                                 table.shape[0] if rot else 0, float(eps)), "norm_rope")
    return out


def norm_rope_cache_write(key, value, key_cache, value_cache, slot_mapping, positions, weight, table, rot: int,
                          eps: float, num_kv_heads, head_size, block_size, num_blocks=None,
                          key_stride=None, value_stride=None):
    """cache_write with K rows first taken through norm_rope_row at positions[t] (in place)."""
    key = _c(key, np.float32)
    value = _c(value, np.float32)
    slot_mapping = _c(slot_mapping, np.uint32)
    positions = _c(positions, np.uint32)
    for c in (key_cache, value_cache):
        if c.dtype != np.uint32 or not c.flags.c_contiguous:
            raise ValueError("caches must be contiguous uint32 arrays")
    T = slot_mapping.shape[0]
    ks = key_stride if key_stride is not None else (key.size // T if T else num_kv_heads * head_size)
    vs = value_stride if value_stride is not None else (value.size // T if T else num_kv_heads * head_size)
    wpt = head_size // 4 + 1
    nb = num_blocks if num_blocks is not None else key_cache.size // (num_kv_heads * block_size * wpt)
    table = _c(table if rot else np.zeros((1, 1), np.float32), np.float32)
    _check(_load().q8o_norm_rope_cache_write(_ptr(key), ks, _ptr(value), vs, _ptr(key_cache), _ptr(value_cache),
                                             _ptr(slot_mapping), _ptr(positions), _ptr(_c(weight, np.float32)),
                                             _ptr(table), rot, table.shape[0] if rot else 0, float(eps), T,
                                             num_kv_heads, head_size, block_size, nb), "norm_rope_cache_write")


# ---------------------------------------------------------------- block select ----

def index_select(scores, row_lens, ratio: int, k: int, vis_stride: int, mask_stride: int = 0):
    """Visible lists from block scores: returns (visible_pos u32 [rows, vis_stride]
    (unused tail entries 0), num_visible u32 [rows]); with mask_stride > 0 also
    the block bitmask u32 [rows, mask_stride] (bit j of a row: the list holds a
    position of block j)."""
    scores = _c(scores, np.float32)
    row_lens = _c(row_lens, np.uint32)
    R = row_lens.shape[0]
    stride = scores.shape[-1] if scores.ndim > 1 else scores.size
    vis = np.zeros((R, vis_stride), dtype=np.uint32)
    nv = np.zeros(R, dtype=np.uint32)
    mask = np.zeros((R, mask_stride), dtype=np.uint32) if mask_stride else None
    _check(_load().q8o_index_select(_ptr(scores), stride, _ptr(row_lens), R, ratio, k, _ptr(vis), vis_stride,
                                    _ptr(nv), _ptr(mask), mask_stride), "index_select")
    return (vis, nv, mask) if mask_stride else (vis, nv)
