"""The C-ABI library loads and exports every symbol include/q8kv.h declares;
host-side validation rejects bad shapes before anything reaches a GPU (CPU only).

No call here launches a kernel: every call returns from argument validation
or is a pure host query."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from int8_paged_kv_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        import int8_paged_kv_amd.build as b
        b.build()
    return _binding.load_library()


def test_header_declares_the_two_operations():
    names = declared_functions()
    assert "q8_cache_write" in names and "q8_paged_decode" in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert lib.q8_status_string(0) == b"Q8_OK"
    assert lib.q8_status_string(3) == b"Q8_ERR_WORKSPACE"
    assert lib.q8_status_string(99) == b"Q8_UNKNOWN"
    assert lib.q8_last_hip_error() == 0


def test_pad_slot_constant_matches_header():
    from int8_paged_kv_amd import workloads, PAD_SLOT
    text = open(HEADER).read()
    assert re.search(r"#define Q8_PAD_SLOT 0xFFFFFFFFu", text)
    assert PAD_SLOT == workloads.PAD_SLOT == 0xFFFFFFFF


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("hs,bs,hkv,stride,want", [
    (0, 16, 2, 256, 2), (6, 16, 2, 256, 2), (260, 16, 1, 260, 2), (128, 0, 2, 256, 2),
    (128, 16, 0, 256, 2), (128, 16, 2, 255, 2),
])
def test_cache_write_shape_errors(lib, hs, bs, hkv, stride, want):
    assert lib.q8_cache_write(FAKE, stride, FAKE, stride, FAKE, FAKE, FAKE, 4, hkv, hs, bs, 8, None) == want


def test_cache_write_grid_limit(lib):
    # a batched write takes one workgroup per 16 tokens of a kv head: 2^28 * 8
    # of them is past the 2^31 - 1 a launch may ask for
    assert lib.q8_cache_write(FAKE, 1024, FAKE, 1024, FAKE, FAKE, FAKE, 0xFFFFFFFF, 8, 128, 16, 8, None) == 2
    assert lib.q8_cache_write(FAKE, 2048, FAKE, 2048, FAKE, FAKE, FAKE, 1 << 31, 16, 128, 16, 8, None) == 2


def test_cache_write_null_and_empty(lib):
    assert lib.q8_cache_write(None, 256, FAKE, 256, FAKE, FAKE, FAKE, 4, 2, 128, 16, 8, None) == 1
    assert lib.q8_cache_write(None, 256, None, 256, None, None, None, 0, 2, 128, 16, 8, None) == 0


def decode_args(**kw):
    a = dict(out=FAKE, q=FAKE, q_stride=4 * 128, kc=FAKE, vc=FAKE, bt=FAKE, max_nb=8, cl=FAKE, mcl=5000,
             vis=None, nvis=None, vis_stride=0, S=2, H=4, Hkv=2, hs=128, bs=16, nb=64, scale=0.1,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return [a[k] for k in ("out", "q", "q_stride", "kc", "vc", "bt", "max_nb", "cl", "mcl", "vis", "nvis",
                           "vis_stride", "S", "H", "Hkv", "hs", "bs", "nb", "scale", "ws", "wsb", "stream")]


@pytest.mark.parametrize("kw,want", [
    (dict(hs=130), 2), (dict(hs=512), 2), (dict(H=5), 2), (dict(Hkv=0), 2), (dict(bs=0), 2),
    (dict(q_stride=511), 2), (dict(vis=FAKE, nvis=FAKE, vis_stride=0), 2), (dict(max_nb=0), 2),
    (dict(scale=float("nan")), 2), (dict(out=None), 1), (dict(bt=None), 1), (dict(cl=None), 1),
    (dict(vis=FAKE, nvis=None, vis_stride=8), 1), (dict(ws=None), 3), (dict(wsb=16), 3),
    (dict(ws=ctypes.c_void_p(0x1004)), 3), (dict(out=ctypes.c_void_p(0x2004)), 5), (dict(S=0), 0),
])
def test_decode_validation(lib, kw, want):
    assert lib.q8_paged_decode(*decode_args(**kw)) == want


def test_workspace_size_matches_plan(lib):
    # At most 32 positions per sequence (a chunk holds 32 or 64): every
    # sequence lies in one wavefront's range, no partials.
    assert lib.q8_paged_decode_workspace_bytes(2, 4, 2, 128, 16, 32) == 0
    assert lib.q8_paged_decode_workspace_bytes(2, 4, 2, 128, 16, 33) > 0
    # Otherwise: per row group (kv head, group of 4, 8 or 16 query heads),
    # (waves per group + S - 1) records of (head_size + 2) floats per head.
    # Layout: arrival counters (one u32 per row group and sequence), then the
    # records' outputs, then their (max, sum) pairs, each 256-byte aligned.
    def want(S, hs, rg, group):
        recs = 2048 // rg + S - 1
        slots = rg * recs * group
        r256 = lambda b: (b + 255) // 256 * 256
        return r256(rg * S * 4) + r256(slots * hs * 4) + slots * 2 * 4
    assert lib.q8_paged_decode_workspace_bytes(64, 32, 8, 128, 16, 4096) == want(64, 128, 8, 4)
    # n_rep 8 uses groups of 8 query heads
    assert lib.q8_paged_decode_workspace_bytes(8, 64, 8, 128, 32, 32768) == want(8, 128, 8, 8)
    # n_rep 16: one group of 16 per kv head; n_rep 32: two groups of 16
    assert lib.q8_paged_decode_workspace_bytes(2, 32, 2, 64, 16, 500) == want(2, 64, 2, 16)
    assert lib.q8_paged_decode_workspace_bytes(2, 64, 2, 64, 16, 500) == want(2, 64, 4, 16)


def step_args(**kw):
    a = dict(out=FAKE, q=FAKE, q_stride=4 * 128, k=FAKE, ks=2 * 128, v=FAKE, vs=2 * 128, kc=FAKE, vc=FAKE,
             bt=FAKE, max_nb=8, cl=FAKE, mcl=5000, S=2, H=4, Hkv=2, hs=128, bs=16, nb=64, scale=0.1,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return [a[k] for k in ("out", "q", "q_stride", "k", "ks", "v", "vs", "kc", "vc", "bt", "max_nb", "cl", "mcl",
                           "S", "H", "Hkv", "hs", "bs", "nb", "scale", "ws", "wsb", "stream")]


@pytest.mark.parametrize("kw,want", [
    (dict(k=None), 1), (dict(v=None), 1), (dict(cl=None), 1), (dict(ks=255), 2), (dict(vs=100), 2),
    (dict(hs=130), 2), (dict(H=5), 2), (dict(wsb=16), 3), (dict(out=ctypes.c_void_p(0x2004)), 5), (dict(S=0), 0),
])
def test_decode_step_validation(lib, kw, want):
    assert lib.q8_decode_step(*step_args(**kw)) == want


def nr_step_args(**kw):
    a = dict(out=FAKE, q=FAKE, q_stride=4 * 128, qhs=0, k=FAKE, ks=2 * 128, v=FAKE, vs=2 * 128, kc=FAKE, vc=FAKE,
             bt=FAKE, max_nb=8, cl=FAKE, mcl=5000, qw=FAKE, kw=FAKE, tab=FAKE, rot=64, npos=8192, eps=1e-6,
             S=2, H=4, Hkv=2, hs=128, bs=16, nb=64, scale=0.1, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return [a[k] for k in ("out", "q", "q_stride", "qhs", "k", "ks", "v", "vs", "kc", "vc", "bt", "max_nb", "cl", "mcl",
                           "qw", "kw", "tab", "rot", "npos", "eps",
                           "S", "H", "Hkv", "hs", "bs", "nb", "scale", "ws", "wsb", "stream")]


@pytest.mark.parametrize("kw,want", [
    # the norm + rotary step's shape rules and operands
    (dict(rot=12), 2), (dict(rot=136), 2), (dict(eps=-1.0), 2), (dict(eps=float("inf")), 2), (dict(npos=0), 2),
    (dict(qw=None), 1), (dict(kw=None), 1), (dict(tab=None), 1),
    # those of the decode step
    (dict(k=None), 1), (dict(cl=None), 1), (dict(ks=255), 2), (dict(hs=130), 2), (dict(H=5), 2),
    (dict(wsb=16), 3), (dict(out=ctypes.c_void_p(0x2004)), 5), (dict(S=0), 0), (dict(S=0, qw=None), 0),
    # q head stride: below head_size, or a row too short for its heads
    (dict(qhs=100), 2), (dict(qhs=256, q_stride=4 * 256 - 129), 2), (dict(qhs=256, q_stride=4 * 256 - 128, wsb=16), 3),
    # shapes without a fused kernel: head sizes other than 64, 128 and 256,
    # misaligned caches, block sizes not nesting with the chunk (32 positions
    # at head_size <= 128 with up to 4 query heads per kv head, else 64)
    (dict(hs=96, rot=32, q_stride=4 * 96, ks=192, vs=192), 5), (dict(hs=32, rot=32, q_stride=4 * 32, ks=64, vs=64), 5),
    (dict(kc=ctypes.c_void_p(0x1004)), 5), (dict(vc=ctypes.c_void_p(0x1008)), 5), (dict(bs=48), 5),
    (dict(bs=6), 5), (dict(H=16, q_stride=16 * 128, bs=48), 5), (dict(H=32, q_stride=32 * 128, bs=96), 5),
    (dict(hs=256, q_stride=4 * 256, ks=512, vs=512, bs=96), 5),
])
def test_norm_rope_decode_step_validation(lib, kw, want):
    assert lib.q8_norm_rope_decode_step(*nr_step_args(**kw)) == want


def rows_args(**kw):
    a = dict(out=FAKE, q=FAKE, q_stride=4 * 128, kc=FAKE, vc=FAKE, bt=FAKE, max_nb=8, cl=FAKE, mcl=5000, nb=4,
             S=2, H=4, Hkv=2, hs=128, bs=16, nblk=64, scale=0.1, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return [a[k] for k in ("out", "q", "q_stride", "kc", "vc", "bt", "max_nb", "cl", "mcl", "nb", "S", "H", "Hkv",
                           "hs", "bs", "nblk", "scale", "ws", "wsb", "stream")]


@pytest.mark.parametrize("kw,want", [
    (dict(nb=0), 2), (dict(cl=None), 1), (dict(hs=130), 2), (dict(wsb=16), 3), (dict(S=0), 0),
    (dict(out=ctypes.c_void_p(0x2004)), 5),
])
def test_decode_rows_validation(lib, kw, want):
    assert lib.q8_paged_decode_rows(*rows_args(**kw)) == want


def f32_args(**kw):
    a = dict(out=FAKE, q=FAKE, q_stride=4 * 128, kc=FAKE, vc=FAKE, bt=FAKE, max_nb=8, cl=FAKE, mcl=5000,
             S=2, H=4, Hkv=2, hs=128, bs=16, nb=64, scale=0.1, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return [a[k] for k in ("out", "q", "q_stride", "kc", "vc", "bt", "max_nb", "cl", "mcl", "S", "H", "Hkv",
                           "hs", "bs", "nb", "scale", "ws", "wsb", "stream")]


@pytest.mark.parametrize("kw,want", [
    (dict(hs=130), 2), (dict(hs=512), 2), (dict(H=5), 2), (dict(bs=0), 2), (dict(q_stride=511), 2),
    (dict(scale=float("inf")), 2), (dict(max_nb=0), 2), (dict(hs=96, q_stride=4 * 96), 5),
    (dict(q_stride=514), 5), (dict(mcl=1 << 31), 5), (dict(out=None), 1), (dict(cl=None), 1),
    (dict(q=ctypes.c_void_p(0x1008)), 5), (dict(kc=ctypes.c_void_p(0x1004)), 5), (dict(ws=None), 3),
    (dict(wsb=16), 3), (dict(S=0), 0),
])
def test_f32_decode_validation(lib, kw, want):
    assert lib.q8_f32_paged_decode(*f32_args(**kw)) == want


def test_f32_workspace_size_matches_plan(lib):
    # 2048 persistent waves over the row groups (kv head, group of 4, 2 or 1
    # query heads); (waves per group + S - 1) records of (head_size + 2)
    # floats per head, after one arrival counter per (row group, sequence).
    def want(S, hs, rg, group):
        recs = 2048 // rg + S - 1
        slots = rg * recs * group
        r256 = lambda b: (b + 255) // 256 * 256
        return r256(rg * S * 4) + r256(slots * hs * 4) + slots * 2 * 4
    assert lib.q8_f32_paged_decode_workspace_bytes(64, 32, 8, 128) == want(64, 128, 8, 4)
    assert lib.q8_f32_paged_decode_workspace_bytes(3, 12, 2, 64) == want(3, 64, 6, 2)     # n_rep 6: 3 groups of 2
    assert lib.q8_f32_paged_decode_workspace_bytes(5, 6, 2, 32) == want(5, 32, 6, 1)      # n_rep 3: single heads
    assert lib.q8_f32_paged_decode_workspace_bytes(2, 4, 3, 128) == 0                     # inconsistent heads


@pytest.mark.parametrize("hs,bs,hkv,stride,nb,want", [
    (0, 16, 2, 256, 8, 2), (6, 16, 2, 256, 8, 2), (260, 16, 1, 260, 8, 2), (128, 0, 2, 256, 8, 2),
    (128, 16, 0, 256, 8, 2), (128, 16, 2, 255, 8, 2), (128, 16, 2, 256, 0, 2),
])
def test_f32_cache_write_shape_errors(lib, hs, bs, hkv, stride, nb, want):
    assert lib.q8_f32_cache_write(FAKE, stride, FAKE, stride, FAKE, FAKE, FAKE, 4, hkv, hs, bs, nb, None) == want


def test_f32_cache_write_null_empty_and_alignment(lib):
    assert lib.q8_f32_cache_write(None, 256, FAKE, 256, FAKE, FAKE, FAKE, 4, 2, 128, 16, 8, None) == 1
    assert lib.q8_f32_cache_write(None, 256, None, 256, None, None, None, 0, 2, 128, 16, 8, None) == 0
    assert lib.q8_f32_cache_write(FAKE, 256, FAKE, 256, ctypes.c_void_p(0x1004), FAKE, FAKE, 4, 2, 128, 16, 8,
                                  None) == 5


@pytest.mark.parametrize("kw,want", [
    (dict(hs=130), 2), (dict(hs=512), 2), (dict(H=5), 2), (dict(bs=0), 2), (dict(q_stride=511), 2),
    (dict(scale=float("inf")), 2), (dict(max_nb=0), 2), (dict(hs=96, q_stride=4 * 96), 5),
    (dict(q_stride=514), 5), (dict(mcl=1 << 31), 5), (dict(out=None), 1), (dict(cl=None), 1),
    (dict(kc=ctypes.c_void_p(0x1008)), 5), (dict(vc=ctypes.c_void_p(0x1002)), 5), (dict(ws=None), 3),
    (dict(wsb=16), 3), (dict(S=0), 0),
])
def test_bf16_decode_validation(lib, kw, want):
    assert lib.q8_bf16_paged_decode(*f32_args(**kw)) == want


def test_bf16_workspace_is_the_f32_plan(lib):
    for shape in [(64, 32, 8, 128), (3, 12, 2, 64), (5, 6, 2, 32), (1, 16, 16, 256), (2, 4, 3, 128)]:
        assert lib.q8_bf16_paged_decode_workspace_bytes(*shape) == lib.q8_f32_paged_decode_workspace_bytes(*shape)


@pytest.mark.parametrize("hs,bs,hkv,stride,nb,want", [
    (0, 16, 2, 256, 8, 2), (6, 16, 2, 256, 8, 2), (260, 16, 1, 260, 8, 2), (128, 0, 2, 256, 8, 2),
    (128, 16, 0, 256, 8, 2), (128, 16, 2, 255, 8, 2), (128, 16, 2, 256, 0, 2),
    (20, 16, 2, 40, 8, 5), (12, 16, 1, 12, 8, 5),        # head_size not a multiple of 8
])
def test_bf16_cache_write_shape_errors(lib, hs, bs, hkv, stride, nb, want):
    assert lib.q8_bf16_cache_write(FAKE, stride, FAKE, stride, FAKE, FAKE, FAKE, 4, hkv, hs, bs, nb, None) == want


def test_bf16_cache_write_null_empty_and_alignment(lib):
    assert lib.q8_bf16_cache_write(None, 256, FAKE, 256, FAKE, FAKE, FAKE, 4, 2, 128, 16, 8, None) == 1
    assert lib.q8_bf16_cache_write(None, 256, None, 256, None, None, None, 0, 2, 128, 16, 8, None) == 0
    assert lib.q8_bf16_cache_write(FAKE, 256, FAKE, 256, ctypes.c_void_p(0x1008), FAKE, FAKE, 4, 2, 128, 16, 8,
                                   None) == 5


# ---- per-head RMSNorm + partial rotary step ----

def test_rope_table_validation(lib):
    assert lib.q8_rope_table(FAKE, 16, 7, ctypes.c_float(10000.0), None) == 2      # odd rot
    assert lib.q8_rope_table(FAKE, 16, 8, ctypes.c_float(0.0), None) == 2          # theta not positive
    assert lib.q8_rope_table(FAKE, 16, 8, ctypes.c_float(float("inf")), None) == 2
    assert lib.q8_rope_table(None, 16, 8, ctypes.c_float(10000.0), None) == 1      # NULL table
    assert lib.q8_rope_table(None, 0, 8, ctypes.c_float(10000.0), None) == 0       # nothing to fill
    assert lib.q8_rope_table(None, 16, 0, ctypes.c_float(10000.0), None) == 0


@pytest.mark.parametrize("hs,rot,hstride,xstride,ostride,npos,eps,want", [
    (128, 64, 128, 4096, 4096, 16, 1e-6, 0),      # valid, but num_rows == 0 below: nothing enqueued
    (130, 64, 130, 4160, 4160, 16, 1e-6, 2),      # head_size not a multiple of 4
    (128, 60, 128, 4096, 4096, 16, 1e-6, 2),      # rot not a multiple of 8
    (64, 72, 64, 2048, 2048, 16, 1e-6, 2),        # rot above head_size
    (128, 64, 120, 4096, 4096, 16, 1e-6, 2),      # head_stride < head_size
    (128, 64, 128, 4000, 4096, 16, 1e-6, 2),      # x_stride too small for 32 heads
    (128, 64, 128, 4096, 4000, 16, 1e-6, 2),      # out_stride too small
    (128, 64, 128, 4096, 4096, 0, 1e-6, 2),       # rot > 0 without a table
    (128, 64, 128, 4096, 4096, 16, -1.0, 2),      # negative eps
])
def test_norm_rope_validation(lib, hs, rot, hstride, xstride, ostride, npos, eps, want):
    assert lib.q8_norm_rope(FAKE, ostride, FAKE, xstride, hstride, 0, 32, hs, FAKE, FAKE, FAKE, rot, npos,
                            ctypes.c_float(eps), None) == want


def test_norm_rope_nulls(lib):
    args = lambda out, x, pos, w, tab: (out, 4096, x, 4096, 128, 4, 32, 128, pos, w, tab, 64, 16,
                                        ctypes.c_float(1e-6), None)
    assert lib.q8_norm_rope(*args(None, FAKE, FAKE, FAKE, FAKE)) == 1
    assert lib.q8_norm_rope(*args(FAKE, FAKE, None, FAKE, FAKE)) == 1        # rot > 0 needs positions
    assert lib.q8_norm_rope(*args(FAKE, FAKE, FAKE, FAKE, None)) == 1        # and the table
    assert lib.q8_norm_rope(*args(FAKE, FAKE, FAKE, None, FAKE)) == 1


@pytest.mark.parametrize("hs,bs,hkv,stride,nb,rot,npos,want", [
    (0, 16, 2, 256, 8, 0, 0, 2), (128, 0, 2, 256, 8, 64, 16, 2), (128, 16, 0, 256, 8, 64, 16, 2),
    (128, 16, 2, 255, 8, 64, 16, 2), (128, 16, 2, 256, 0, 64, 16, 2), (128, 16, 2, 256, 8, 12, 16, 2),
    (128, 16, 2, 256, 8, 64, 0, 2),
])
def test_norm_rope_cache_write_validation(lib, hs, bs, hkv, stride, nb, rot, npos, want):
    assert lib.q8_norm_rope_cache_write(FAKE, stride, FAKE, stride, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, rot, npos,
                                        ctypes.c_float(1e-6), 4, hkv, hs, bs, nb, None) == want


def test_norm_rope_cache_write_nulls_and_empty(lib):
    assert lib.q8_norm_rope_cache_write(FAKE, 256, FAKE, 256, FAKE, FAKE, FAKE, None, FAKE, FAKE, 64, 16,
                                        ctypes.c_float(1e-6), 4, 2, 128, 16, 8, None) == 1
    assert lib.q8_norm_rope_cache_write(FAKE, 256, FAKE, 256, FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 16,
                                        ctypes.c_float(1e-6), 4, 2, 128, 16, 8, None) == 1
    assert lib.q8_norm_rope_cache_write(None, 256, None, 256, None, None, None, None, None, None, 64, 16,
                                        ctypes.c_float(1e-6), 0, 2, 128, 16, 8, None) == 0


def qk_call(lib, q_out=FAKE, q_head_stride=128, q_rows=4, heads=32, q_pos=FAKE, q_w=FAKE, key=FAKE, k_pos=FAKE,
            k_w=FAKE, table=FAKE, rot=64, npos=16, tokens=4, hkv=2, hs=128, bs=16, nb=8):
    return lib.q8_norm_rope_qk_cache_write(q_out, heads * hs, FAKE, heads * q_head_stride, q_head_stride, q_rows,
                                           heads, q_pos, q_w, key, hkv * hs, FAKE, hkv * hs, FAKE, FAKE, FAKE, k_pos,
                                           k_w, table, rot, npos, ctypes.c_float(1e-6), tokens, hkv, hs, bs, nb, None)


def test_norm_rope_qk_cache_write_validation(lib):
    """The union of q8_norm_rope's and q8_norm_rope_cache_write's rules; either side may be empty."""
    assert qk_call(lib, q_out=None, q_pos=None, q_w=None, key=None, k_pos=None, k_w=None, table=None,
                   q_rows=0, tokens=0) == 0                                  # both sides empty
    assert qk_call(lib, q_head_stride=127) == 2                             # q heads overlap
    assert qk_call(lib, rot=12) == 2                                        # rot not a multiple of 8
    assert qk_call(lib, bs=0, q_rows=0) == 2                                # the write's shape, q empty
    assert qk_call(lib, nb=0) == 2
    assert qk_call(lib, q_out=None) == 1
    assert qk_call(lib, q_pos=None) == 1                                    # rot > 0: q positions needed
    assert qk_call(lib, key=None) == 1
    assert qk_call(lib, k_w=None) == 1
    assert qk_call(lib, table=None, q_rows=0) == 1                          # the table, for the write alone


def test_index_select_validation(lib):
    assert lib.q8_index_select(FAKE, 64, FAKE, 4, 0, 2, FAKE, 128, FAKE, None, 0, None) == 2          # ratio 0
    assert lib.q8_index_select(FAKE, 64, FAKE, 4, 64, 32, FAKE, 2111, FAKE, None, 0, None) == 2       # (k+1)*ratio > vis_stride
    assert lib.q8_index_select(FAKE, 16385, FAKE, 4, 64, 32, FAKE, 2112, FAKE, None, 0, None) == 5    # too many blocks per row
    assert lib.q8_index_select(None, 64, FAKE, 4, 64, 32, FAKE, 2112, FAKE, None, 0, None) == 1
    assert lib.q8_index_select(FAKE, 64, FAKE, 4, 64, 32, FAKE, 2112, None, None, 0, None) == 1
    assert lib.q8_index_select(None, 64, None, 0, 64, 32, None, 2112, None, None, 0, None) == 0       # no rows
    assert lib.q8_index_select(FAKE, 64, FAKE, 4, 64, 32, FAKE, 2112, FAKE, FAKE, 2, None) == 2   # 65 blocks need 3 words
    assert lib.q8_index_select(FAKE, 63, FAKE, 0, 64, 32, FAKE, 2112, FAKE, FAKE, 2, None) == 0   # 64 blocks fit in 2


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """The no-alloc decode refuses shapes whose partial records exceed its
    fixed scratch array before touching the device; smaller shapes than the
    limit pass validation identically to q8_paged_decode's."""
    a = decode_args(S=100000, H=16, Hkv=16, hs=256, q_stride=16 * 256, mcl=5000)
    need = lib.q8_paged_decode_workspace_bytes(100000, 16, 16, 256, 16, 5000)
    assert need > (32 << 20)
    del a[19:21]        # no workspace arguments
    assert lib.q8_paged_decode_noalloc(*a) == 3


@pytest.mark.parametrize("kw,want", [
    (dict(hs=6), 2), (dict(H=3, Hkv=2), 2), (dict(q_stride=100), 2), (dict(q=None), 1),
    (dict(vis=FAKE, nvis=FAKE, vis_stride=0), 2),
])
def test_noalloc_validation_matches_decode(lib, kw, want):
    a = decode_args(**kw)
    assert lib.q8_paged_decode(*a) == want
    del a[19:21]
    assert lib.q8_paged_decode_noalloc(*a) == want


def test_bounds_flags_release_and_debug(lib):
    """The release library has no content checks (Q8_ERR_UNSUPPORTED, flags 0);
    the debug build exports every declared symbol as well."""
    f = ctypes.c_uint32(7)
    assert lib.q8_bounds_flags(ctypes.byref(f), 0) == 5 and f.value == 0
    assert lib.q8_bounds_flags(None, 0) == 1
    from int8_paged_kv_amd import _binding
    if not os.path.exists(_binding.DEBUG_LIB_PATH):
        pytest.skip("libq8kv_debug.so not built")
    dbg = _binding.load_debug_library()
    for name in declared_functions():
        assert hasattr(dbg, name), name
