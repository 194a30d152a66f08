#!/usr/bin/env python3
"""Benchmark of the int8 paged-KV decode step on one MI355X.

One step = the whole hot path on the Llama-3-8B-shaped batch (64 sequences,
32 query heads, 8 kv heads, head_size 128, block_size 16, context lengths
uniform in [512, 4096]): the 64 new tokens (one per sequence) quantized and
packed into the caches, and decode attention over every sequence's full
context, in one launch of q8_decode_step.

Inputs are resident in HBM before timing.  The step rotates over several
layer caches (copies of the filled cache at different addresses), as a model's
layers do, so each step reads its KV from HBM rather than from the 256 MB
Infinity Cache left warm by the previous step.  Before the W warmup steps, about
a second of untimed steps lets the GPU clock settle; then exactly K steps are
timed (wall clock, and HIP events on the launch stream around them).

Printed: one JSON line with the effective int8-KV read rate (codes + scale
word of every attended row, K and V) as GB/s, its fraction of the 8 TB/s HBM
peak, decode (seq, head)/s, the roofline entry of the step's kernel, and the
CPU oracle on the same workload (all cores of this process's share and one
thread).  Beside it (skipped with --no-reference): the same step as two
launches; 4-row causal decode; the f32- and bf16-cache steps; the norm + rotary step; the
selected-token step; the long-context and MHA head_size=256 decodes and the
padded 4096-token write; and the practical HBM ceiling (a streaming read and
the step's own tiles read without arithmetic, libq8kv_bench.so).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective int8 KV read GB/s (% of HBM peak) + decode (seq,head)/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q8_paged_decode_llama_traffic.txt")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--layers", type=int, default=8, help="layer caches rotated over (MALL defeat)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-hot", action="store_true", help="skip timing back-to-back steps on one cache")
    p.add_argument("--prime-s", type=float, default=1.0,
                   help="seconds of untimed steps before the warmup steps (the GPU clock settles)")
    p.add_argument("--no-reference", action="store_true",
                   help="skip timing the two-launch reference (cache write, then decode)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB five times (the known-size "
                        "kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


def copy_calibration(mib: int) -> None:
    """Five launches of torch's contiguous copy kernel over `mib` MiB: each
    reads and writes exactly mib * 2^20 bytes of HBM (source and destination
    are far larger than any cache once rotated over three buffer pairs)."""
    import torch
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    pairs = [(torch.ones(n, dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.int32, device=dev))
             for _ in range(3)]
    torch.cuda.synchronize()
    for i in range(5):
        src, dst = pairs[i % 3]
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n * 4, "launches": 5}), flush=True)


# The files the decode kernel (decode_split_kernel), the cache writer and their
# launches are built from; the committed HBM-traffic figures hold while their
# code is unchanged (comments and layout do not count).
DECODE_SOURCES = ("decode_kernel.h", "decode_split.h", "decode.hip", "decode_hs16.hip", "decode_hs32.hip",
                  "decode_hs48.hip", "decode_hs64.hip", "q8_pack.h", "lane_reduce.h", "wave_ops.h",
                  "q8kv_internal.h", "bounds.h", "cache_write.hip", "norm_rope_ops.h", "decode_nr16.hip",
                  "decode_nr32.hip", "decode_nr64.hip")


def code_only(text: str) -> str:
    """C++ source with its comments removed and whitespace collapsed (the
    sources hold no string literal with comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int8_paged_kv_amd", "csrc")
    for f in DECODE_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(digest: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    or None when it is absent or was taken on different kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.lstrip().startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_sources_sha256_16") != digest:
            return None
        return float(kv["hbm_bytes_per_step"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_threads() -> int:
    """Threads of the all-cores CPU leg: the host's cores, capped at the
    OMP_NUM_THREADS the machine sets for this process (its CPU share)."""
    return max(1, min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", "16") or 16)))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(oracle, w, qh, kh, vh, mcl, seconds):
    """The oracle's decode (binary64 plain definition) on the host, on all
    cores of this process's share and on one thread, over bounded samples of
    the same workload; rates in effective KV bytes per second, so they compare
    with the GPU line directly."""
    Hkv, hs, bs = w.num_kv_heads, w.head_size, w.block_size
    n_all = cpu_threads()

    def run(seqs, nthreads, budget):
        q = qh[seqs]
        bt, cl = w.block_tables[seqs], w.context_lens[seqs]
        B = int(np.minimum(cl, mcl).sum()) * Hkv * 2 * (hs + 4)
        reps, t = 0, 0.0
        while t < budget or reps == 0:
            c0 = time.perf_counter()
            oracle.paged_decode(q, kh, vh, bt, cl, w.scale, Hkv, bs, max_context_len=mcl, nthreads=nthreads)
            t += time.perf_counter() - c0
            reps += 1
        return B * reps / t / 1e9, reps, t, B

    all_seqs = np.arange(w.num_seqs)
    v_all, r_all, t_all, _ = run(all_seqs, n_all, seconds)
    few = all_seqs[:4]            # one thread: the first 4 sequences of the batch
    v_one, r_one, t_one, b_one = run(few, 1, seconds / 2)
    return {"value": round(v_all, 3), "unit": "GB/s", "cores": n_all, "kind": "oracle",
            "sample": "the full decode step (all %d (seq,head) rows of the Llama-shaped batch) repeated %d times "
                      "in %.1f s" % (w.num_seqs * w.num_heads, r_all, t_all),
            "single_thread": {"value": round(v_one, 3), "unit": "GB/s", "cores": 1,
                              "sample": "sequences 0-3 of the batch (%d effective KV bytes) repeated %d times in "
                                        "%.1f s" % (b_one, r_one, t_one)},
            "host": {"os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
                     "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}}


def _timed(fn, n, dev_sync=True):
    """Mean duration of n back-to-back launches (fn(i) enqueues launch i),
    from HIP events around them on the current stream, in microseconds."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def _fill_device(w, kc, vc, gen, chunk=65536):
    """Fill the caches with the workload's rows: its slots, K/V drawn N(0,1) on
    the device from `gen` (the timing does not depend on the values), with its
    outlier channels scaled x20."""
    import torch
    from int8_paged_kv_amd import q8_cache_write
    dev = kc.device
    slots = w.fill_slots()
    ok = None if w.outlier_k is None else torch.from_numpy(w.outlier_k).to(dev)
    ov = None if w.outlier_v is None else torch.from_numpy(w.outlier_v).to(dev)
    for st in range(0, slots.shape[0], chunk):
        sl = slots[st:st + chunk]
        T = sl.shape[0]
        k = torch.randn((T, w.num_kv_heads, w.head_size), generator=gen, device=dev, dtype=torch.float32)
        v = torch.randn((T, w.num_kv_heads, w.head_size), generator=gen, device=dev, dtype=torch.float32)
        if ok is not None:
            k[:, ok] *= 20.0
        if ov is not None:
            v[:, ov] *= 20.0
        sld = torch.from_numpy(sl.view(np.int32)).to(dev)
        q8_cache_write(k, v, kc, vc, sld, w.num_kv_heads, w.head_size, w.block_size)
        del k, v


def bench_long_context(dev):
    """Long-context decode: S=8 H=64 Hkv=8 hs=128 bs=32, 32768 positions each,
    fragmented tables (seed 3); two cache copies rotated (1.1 GB of K/V each)."""
    import torch
    from int8_paged_kv_amd import q8_paged_decode, q8_paged_decode_workspace_bytes
    from int8_paged_kv_amd import workloads as wl
    w = wl.long_context()
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    copies = []
    for _ in range(2):
        kh, vh = w.empty_caches()
        kc = torch.from_numpy(kh.view(np.int32)).to(dev)
        vc = torch.from_numpy(vh.view(np.int32)).to(dev)
        del kh, vh
        _fill_device(w, kc, vc, gen)
        copies.append((kc, vc))
    q = torch.from_numpy(w.q()).to(dev)
    bt = torch.from_numpy(w.block_tables.view(np.int32)).to(dev)
    cl = torch.from_numpy(w.context_lens.view(np.int32)).to(dev)
    ws = torch.zeros(max(1, q8_paged_decode_workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size,
                                                            w.block_size, w.max_context_len)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((w.num_seqs, w.num_heads, w.head_size), dtype=torch.float32, device=dev)

    def run(i):
        kc, vc = copies[i % 2]
        q8_paged_decode(q, kc, vc, bt, cl, w.scale, w.num_kv_heads, w.block_size,
                        max_context_len=w.max_context_len, out=out, workspace=ws)

    for i in range(6):
        run(i)
    us = _timed(run, 40)
    B = w.effective_kv_bytes()
    del copies
    return {"workload": w.description + " (seed 3)", "us_mean": round(us, 2), "effective_kv_bytes": B,
            "effective_GBps": round(B / (us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(B / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "seq_heads_per_s": round(w.num_seqs * w.num_heads / (us * 1e-6), 1),
            "traffic": read_leg_traffic("long_context"),
            "note": "q8_paged_decode, back-to-back launches over two rotated cache copies; K/V values drawn on "
                    "the device (same shapes, distribution and outlier channels; the full-size parity test "
                    "uses the host generator)"}


def bench_mha256(dev):
    """MHA head_size 256 (seed 4): the decode (S=128, H=Hkv=16, bs=16,
    L~U[1024,2048], 1.68 GB of K/V) and the 4096-token write with 10% pad
    slots and 0.5% all-zero vectors."""
    import torch
    from int8_paged_kv_amd import q8_cache_write, q8_paged_decode, q8_paged_decode_workspace_bytes
    from int8_paged_kv_amd import workloads as wl
    w = wl.mha256()
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    kh, vh = w.empty_caches()
    kc = torch.from_numpy(kh.view(np.int32)).to(dev)
    vc = torch.from_numpy(vh.view(np.int32)).to(dev)
    del kh, vh
    _fill_device(w, kc, vc, gen)
    q = torch.from_numpy(w.q()).to(dev)
    bt = torch.from_numpy(w.block_tables.view(np.int32)).to(dev)
    cl = torch.from_numpy(w.context_lens.view(np.int32)).to(dev)
    ws = torch.zeros(max(1, q8_paged_decode_workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size,
                                                            w.block_size, w.max_context_len)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((w.num_seqs, w.num_heads, w.head_size), dtype=torch.float32, device=dev)

    def run(i):
        q8_paged_decode(q, kc, vc, bt, cl, w.scale, w.num_kv_heads, w.block_size,
                        max_context_len=w.max_context_len, out=out, workspace=ws)

    for i in range(4):
        run(i)
    us = _timed(run, 20)
    B = w.effective_kv_bytes()
    dec = {"workload": w.description + " (seed 4)", "us_mean": round(us, 2), "effective_kv_bytes": B,
           "effective_GBps": round(B / (us * 1e-6) / 1e9, 1),
           "frac_hbm_peak": round(B / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "seq_heads_per_s": round(w.num_seqs * w.num_heads / (us * 1e-6), 1),
           "traffic": read_leg_traffic("mha256_decode"),
           "note": "q8_paged_decode, back-to-back launches (1.68 GB of K/V per launch, far above the 256 MB "
                   "Infinity Cache); K/V values drawn on the device"}
    # the padded bulk write: four copies of its inputs rotated, so they come from HBM
    slots, k, v = wl.mha256_write(w)
    T = slots.shape[0]
    sl = torch.from_numpy(slots.view(np.int32)).to(dev)
    ins = [(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)) for _ in range(4)]

    def write(i):
        kk, vv = ins[i % 4]
        q8_cache_write(kk, vv, kc, vc, sl, w.num_kv_heads, w.head_size, w.block_size)

    for i in range(4):
        write(i)
    usw = _timed(write, 40)
    n_real = int(np.count_nonzero(slots != wl.PAD_SLOT))
    Bw = n_real * w.num_kv_heads * (2 * w.head_size * 4 + 2 * (w.head_size + 4)) + 4 * T
    wr = {"workload": "4096-token write, MHA head_size 256, 10% pad slots, 0.5% zero vectors (seed 4)",
          "us_mean": round(usw, 2), "tokens": T, "pad_tokens": T - n_real, "algorithmic_bytes": Bw,
          "GBps": round(Bw / (usw * 1e-6) / 1e9, 1), "frac_hbm_peak": round(Bw / (usw * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
          "traffic": read_leg_traffic("mha256_write"),
          "note": "q8_cache_write; algorithmic bytes = f32 K and V of the non-pad tokens read, their packed rows "
                  "written, and the slots"}
    del kc, vc, ins
    return dec, wr


def bench_ceiling(dev, w, layers, bt):
    """The practical HBM ceiling beside the 8 TB/s peak: a streaming read of
    2 GiB, and the Llama step's own K/V tiles (every (block, kv head) run of
    16 rows the batch attends, in the decode's order) read without any
    arithmetic by the measurement kernels of libq8kv_bench.so."""
    import ctypes
    import torch
    from int8_paged_kv_amd import build as pkg_build
    if not os.path.exists(pkg_build.BENCH_LIB):
        return None
    lib = ctypes.CDLL(pkg_build.BENCH_LIB)
    lib.q8b_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32,
                                    ctypes.c_void_p]
    lib.q8b_tile_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32,
                                    ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    grid = 2048
    sink = torch.zeros(grid * 4, dtype=torch.int32, device=dev)
    nbytes = 2 << 30
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(2)]

    def sread(i):
        rc = lib.q8b_stream_read(bufs[i % 2].data_ptr(), nbytes, sink.data_ptr(), grid, stream)
        if rc:
            raise RuntimeError("q8b_stream_read: hipError %d" % rc)

    for i in range(4):
        sread(i)
    us_s = _timed(sread, 20)
    del bufs
    # tiles of the Llama batch: (sequence, block, kv head), kv head fastest
    wpt = w.head_size // 4 + 1
    tile_u4 = w.block_size * wpt // 4
    offs = []
    for s_, L in enumerate(w.context_lens):
        for j in range(-(-int(L) // w.block_size)):
            phys = int(w.block_tables[s_, j])
            for h in range(w.num_kv_heads):
                offs.append((phys * w.num_kv_heads + h) * tile_u4)
    tiles = torch.from_numpy(np.asarray(offs, dtype=np.int64)).to(dev)
    nt = len(offs)

    def gather(i):
        kc, vc = layers[i % len(layers)]
        rc = lib.q8b_tile_gather(kc.data_ptr(), vc.data_ptr(), tiles.data_ptr(), nt, tile_u4, sink.data_ptr(),
                                 grid // 4, stream)
        if rc:
            raise RuntimeError("q8b_tile_gather: hipError %d" % rc)

    for i in range(4):
        gather(i)
    us_g = _timed(gather, 40)
    Bt = nt * tile_u4 * 16 * 2
    return {"stream_read_GBps": round(nbytes / (us_s * 1e-6) / 1e9, 1), "stream_read_bytes": nbytes,
            "stream_read_us": round(us_s, 2),
            "tile_gather_GBps": round(Bt / (us_g * 1e-6) / 1e9, 1), "tile_gather_bytes": Bt,
            "tile_gather_us": round(us_g, 2), "tile_gather_waves": grid,
            "note": "libq8kv_bench.so: 16-byte nontemporal loads folded into one word per wave; the tile gather "
                    "reads the Llama step's %d K and V tiles of %d bytes (whole tiles, partial last blocks "
                    "included) from the same rotated layer caches the step reads, with no arithmetic, each wave "
                    "a contiguous range of the list two tiles at a time" % (nt, tile_u4 * 16)}


def read_leg_traffic(leg: str):
    """HBM bytes per launch of a bench leg's kernel from the committed all-kernel
    counter summary, or None when absent or taken on different kernel sources."""
    try:
        kv = {}
        with open(os.path.join(ROOT, "profiles", "bench_legs_traffic.txt")) as f:
            for line in f:
                if ":" in line and not line.lstrip().startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_sources_sha256_16") != kernel_sources_digest():
            return None
        return float(kv[leg + "_hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode step runs within a single GPU and has no multi-GPU "
              "form (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from int8_paged_kv_amd import (q8_cache_write, q8_decode_step, q8_paged_decode, q8_paged_decode_rows,
                                   q8_paged_decode_workspace_bytes, q8_f32_cache_write, q8_f32_paged_decode,
                                   q8_f32_paged_decode_workspace_bytes, q8_bf16_cache_write,
                                   q8_bf16_paged_decode, q8_bf16_paged_decode_workspace_bytes,
                                   q8_rope_table, q8_norm_rope,
                                   q8_norm_rope_cache_write, q8_norm_rope_qk_cache_write,
                                   q8_norm_rope_decode_step, q8_index_select, load_library)
    from int8_paged_kv_amd import workloads as wl

    load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.llama()

    def u32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    # ---- fill one cache, replicate it per layer ----
    t_setup = time.time()
    kh, vh = w.empty_caches()
    kc0, vc0 = u32(kh), u32(vh)
    fill_host = []
    for slots, k, v in w.fill_chunks():
        q8_cache_write(f32(k), f32(v), kc0, vc0, u32(slots), w.num_kv_heads, w.head_size, w.block_size)
        fill_host.append((slots, k, v))
    step_slots, step_k, step_v = w.step_write()
    torch.cuda.synchronize()
    layers = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(args.layers - 1)]
    q = f32(w.q())
    bt, cl = u32(w.block_tables), u32(w.context_lens)
    sk, sv, ss = f32(step_k), f32(step_v), u32(step_slots)
    S, H, Hkv, hs = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size
    mcl = w.max_context_len
    ws = torch.zeros(max(1, q8_paged_decode_workspace_bytes(S, H, Hkv, hs, w.block_size, mcl)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((S, H, hs), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    def step(i, ev=None):
        kc, vc = layers[i % len(layers)]
        if ev is not None:
            ev[0].record()
        q8_decode_step(q, sk, sv, kc, vc, bt, cl, w.scale, Hkv, w.block_size, mcl, out=out, workspace=ws)
        if ev is not None:
            ev[1].record()

    def step_two_launch(i, ev):
        kc, vc = layers[i % len(layers)]
        ev[0].record()
        q8_cache_write(sk, sv, kc, vc, ss, Hkv, hs, w.block_size)
        ev[1].record()
        q8_paged_decode(q, kc, vc, bt, cl, w.scale, Hkv, w.block_size, max_context_len=mcl,
                        out=out, workspace=ws)
        ev[2].record()

    # untimed priming (the clock settles; short runs otherwise time a ramp),
    # then exactly W warmup steps
    t_prime = time.perf_counter()
    n_prime = 0
    while time.perf_counter() - t_prime < args.prime_s:
        for i in range(50):
            step(i)
        torch.cuda.synchronize()
        n_prime += 50
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, wall clock, and HIP events on the
    # launch stream around the same K launches (their mean is the kernel's
    # average launch duration, back to back, as rocprofv3 sees it) ----
    ev_region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev_region[0].record()
    for i in range(args.steps):
        step(i)
    ev_region[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    region_us = ev_region[0].elapsed_time(ev_region[1]) * 1e3 / args.steps

    B = w.effective_kv_bytes()
    # ---- per-launch durations with HIP events around each launch (their
    # spread; each also holds the launch's own dispatch latency) ----
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t_dec = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3     # us, the one step launch
    # the same step as two launches, for reference
    reference = None
    if not args.no_reference:
        evs2 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step_two_launch(i, evs2[i])
        torch.cuda.synchronize()
        t_write = np.array([e[0].elapsed_time(e[1]) for e in evs2]) * 1e3
        t_dec2 = np.array([e[1].elapsed_time(e[2]) for e in evs2]) * 1e3
        reference = {"cache_write_us_mean": round(float(t_write.mean()), 2),
                     "decode_us_mean": round(float(t_dec2.mean()), 2),
                     "decode_effective_GBps": round(B / (float(t_dec2.mean()) * 1e-6) / 1e9, 1),
                     "tokens": int(step_slots.size)}

    # ---- multi-row causal decode: 4 verify rows per sequence at its last 4 positions ----
    multi = None
    if not args.no_reference:
        nbr = 4
        qr = torch.from_numpy(np.random.default_rng(11).standard_normal((S * nbr, H, hs)).astype(np.float32)).to(dev)
        outr = torch.empty((S * nbr, H, hs), dtype=torch.float32, device=dev)
        wsr = torch.zeros(max(1, q8_paged_decode_workspace_bytes(S, H * nbr, Hkv, hs, w.block_size, mcl)),
                          dtype=torch.uint8, device=dev)
        rows_len = [max(0, min(int(L), mcl) - nbr + b + 1) for L in w.context_lens for b in range(nbr)]
        Br = int(sum(rows_len)) * Hkv * 2 * (hs + 4)
        for i in range(3):
            kc, vc = layers[i % len(layers)]
            q8_paged_decode_rows(qr, kc, vc, bt, cl, w.scale, Hkv, w.block_size, mcl, nbr, out=outr, workspace=wsr)
        torch.cuda.synchronize()
        evr = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(20)]
        for i in range(20):
            kc, vc = layers[i % len(layers)]
            evr[i][0].record()
            q8_paged_decode_rows(qr, kc, vc, bt, cl, w.scale, Hkv, w.block_size, mcl, nbr, out=outr, workspace=wsr)
            evr[i][1].record()
        torch.cuda.synchronize()
        tr = np.array([e[0].elapsed_time(e[1]) for e in evr]) * 1e3
        Bd = B     # distinct K/V bytes: each sequence's longest row reads its whole context once
        multi = {"rows_per_seq": nbr, "us_mean": round(float(tr.mean()), 2),
                 "distinct_kv_bytes": Bd, "distinct_GBps": round(Bd / (float(tr.mean()) * 1e-6) / 1e9, 1),
                 "frac_hbm_peak": round(Bd / (float(tr.mean()) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 "per_row_kv_bytes": Br,
                 "per_row_rate_GBps": round(Br / (float(tr.mean()) * 1e-6) / 1e9, 1),
                 "note": "the roofline figure is distinct_GBps: the K/V rows each sequence holds, read once "
                         "for all its rows; per_row_rate counts every row's prefix separately (the rows share "
                         "the reads), so it is not a bandwidth"}

    # ---- the same step over f32 and bfloat16 paged caches (no scale word) ----
    def baseline_reference(kind, write_fn, decode_fn, ws_fn, dtype, poison, elem_bytes):
        nbt = w.num_blocks + 1          # the workload's caches carry one reserved block
        layers = []
        for li in range(2):             # a step reads 0.63 GB (bf16) or 1.27 GB (f32): both above the MALL
            kf = torch.full((nbt, Hkv, w.block_size, hs), poison, dtype=dtype, device=dev)
            vf = torch.full_like(kf, poison)
            layers.append((kf, vf))
        for slots, k, v in fill_host:
            sl, kd, vd = u32(slots), f32(k), f32(v)
            for kf, vf in layers:
                write_fn(kd, vd, kf, vf, sl, Hkv, hs, w.block_size)
        wsf = torch.zeros(max(16, ws_fn(S, H, Hkv, hs)), dtype=torch.uint8, device=dev)
        outf = torch.empty((S, H, hs), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

        def ref_step(i, ev=None):
            kf, vf = layers[i % len(layers)]
            if ev is not None:
                ev[0].record()
            write_fn(sk, sv, kf, vf, ss, Hkv, hs, w.block_size)
            if ev is not None:
                ev[1].record()
            decode_fn(q, kf, vf, bt, cl, w.scale, Hkv, w.block_size, max_context_len=mcl, out=outf, workspace=wsf)
            if ev is not None:
                ev[2].record()

        for i in range(5):
            ref_step(i)
        torch.cuda.synchronize()
        nf = min(100, max(20, args.steps // 4))
        evf = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nf)]
        for i in range(nf):
            ref_step(i, evf[i])
        torch.cuda.synchronize()
        tfw = np.array([e[0].elapsed_time(e[1]) for e in evf]) * 1e3
        tfd = np.array([e[1].elapsed_time(e[2]) for e in evf]) * 1e3
        Bf = int(w.attended_counts().sum()) * Hkv * 2 * hs * elem_bytes
        del layers
        return {"cache_write_us_mean": round(float(tfw.mean()), 2),
                "decode_us_mean": round(float(tfd.mean()), 2),
                "%s_kv_bytes" % kind: Bf,
                "decode_%s_kv_GBps" % kind: round(Bf / (float(tfd.mean()) * 1e-6) / 1e9, 1),
                "decode_frac_hbm_peak": round(Bf / (float(tfd.mean()) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "int8_step_speedup": round(float(tfw.mean() + tfd.mean()) / float(t_dec.mean()), 3),
                "note": "q8_%s_cache_write + q8_%s_paged_decode of the same step over the %s cache "
                        "[num_blocks, Hkv, bs, hs]; speedup = %s step time / int8 one-launch step time"
                        % (kind, kind, kind, kind)}

    f32ref = bf16ref = None
    if not args.no_reference:
        f32ref = baseline_reference("f32", q8_f32_cache_write, q8_f32_paged_decode,
                                    q8_f32_paged_decode_workspace_bytes, torch.float32, float("nan"), 4)
        bf16ref = baseline_reference("bf16", q8_bf16_cache_write, q8_bf16_paged_decode,
                                     q8_bf16_paged_decode_workspace_bytes, torch.bfloat16, float("nan"), 2)

    # ---- per-head RMSNorm + partial rotary step ahead of the write (rot = head_size/2) ----
    normrope = None
    if not args.no_reference:
        rot, P = hs // 2, 8192
        g = np.random.default_rng(12)
        table = q8_rope_table(P, rot, 10000.0, device=dev)
        kn = f32((1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32))
        qn = f32((1.0 + 0.1 * g.standard_normal(hs)).astype(np.float32))
        step_pos = u32(np.minimum(np.asarray(w.context_lens, dtype=np.int64), mcl) - 1)
        qnr = torch.empty_like(q)
        outn = torch.empty_like(out)      # the main step's output stays for the parity check
        q2 = q.view(S, H * hs)

        def nr_step(i, ev=None):
            kc, vc = layers[i % len(layers)]
            if ev is not None:
                ev[0].record()
            q8_norm_rope(q2, step_pos, qn, table, rot, 1e-6, H, hs, out=qnr)
            if ev is not None:
                ev[1].record()
            q8_norm_rope_cache_write(sk, sv, kc, vc, ss, step_pos, kn, table, rot, 1e-6, Hkv, hs, w.block_size)
            if ev is not None:
                ev[2].record()
            q8_paged_decode(qnr, kc, vc, bt, cl, w.scale, Hkv, w.block_size, max_context_len=mcl, out=outn,
                            workspace=ws)
            if ev is not None:
                ev[3].record()

        for i in range(5):
            nr_step(i)
        torch.cuda.synchronize()
        nn_ = 100
        evn = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nn_)]
        for i in range(nn_):
            nr_step(i, evn[i])
        torch.cuda.synchronize()
        tq = np.array([e[0].elapsed_time(e[1]) for e in evn]) * 1e3
        tw = np.array([e[1].elapsed_time(e[2]) for e in evn]) * 1e3
        td = np.array([e[2].elapsed_time(e[3]) for e in evn]) * 1e3

        # the same step with q rows and the K/V write in one launch (two launches in all)
        def nr_step2(i, ev=None):
            kc, vc = layers[i % len(layers)]
            if ev is not None:
                ev[0].record()
            q8_norm_rope_qk_cache_write(q2, step_pos, qn, H, sk, sv, kc, vc, ss, step_pos, kn, table, rot, 1e-6,
                                        Hkv, hs, w.block_size, q_out=qnr)
            if ev is not None:
                ev[1].record()
            q8_paged_decode(qnr, kc, vc, bt, cl, w.scale, Hkv, w.block_size, max_context_len=mcl, out=outn,
                            workspace=ws)
            if ev is not None:
                ev[2].record()

        for i in range(5):
            nr_step2(i)
        torch.cuda.synchronize()
        evn2 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nn_)]
        for i in range(nn_):
            nr_step2(i, evn2[i])
        torch.cuda.synchronize()
        tqk = np.array([e[0].elapsed_time(e[1]) for e in evn2]) * 1e3
        t2 = np.array([e[0].elapsed_time(e[2]) for e in evn2]) * 1e3
        t3 = np.array([e[0].elapsed_time(e[3]) for e in evn]) * 1e3

        # the whole step in one launch (q8_norm_rope_decode_step), against the
        # plain one-launch step and the two-launch form, each timed over
        # back-to-back steps on the cycled layers (HIP events at the ends only)
        def nr_fused(i):
            kc, vc = layers[i % len(layers)]
            q8_norm_rope_decode_step(q, sk, sv, kc, vc, bt, cl, w.scale, Hkv, w.block_size, mcl, qn, kn, table,
                                     rot, 1e-6, out=outn, workspace=ws)

        nb_ = max(100, args.steps)
        for i in range(10):
            nr_fused(i)
        t_fused = _timed(nr_fused, nb_)
        t_two = _timed(nr_step2, nb_)
        t_plain = _timed(lambda i: step(i), nb_)
        # the fused step's output against the two-launch form's, bit for bit
        # (same layer, the same rows appended)
        nr_fused(0)
        fused_out = outn.clone()
        nr_step2(0)
        torch.cuda.synchronize()
        fused_equal = bool(torch.equal(fused_out.view(torch.int32), outn.view(torch.int32)))
        # the headline step's algorithmic bytes: int8 KV read, plus the append (f32 K/V in, packed rows out, slots)
        B_nr = B + S * Hkv * (2 * hs * 4 + 2 * (hs + 4)) + 4 * S
        # bulk: 16384 tokens at scattered slots of a separate cache, fused vs plain writer
        Tb = 16384
        nbb = Tb // w.block_size + 64
        kb_ = torch.zeros(((nbb + 1) * Hkv * w.block_size * (hs // 4 + 1),), dtype=torch.int32, device=dev)
        vb_ = torch.zeros_like(kb_)
        bk = f32(g.standard_normal((Tb, Hkv, hs)).astype(np.float32))
        bv = f32(g.standard_normal((Tb, Hkv, hs)).astype(np.float32))
        bslots = u32(g.choice(nbb * w.block_size, size=Tb, replace=False).astype(np.uint32))
        bpos = u32(g.integers(0, P, Tb).astype(np.uint32))
        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(30)]
        for i in range(35):
            e = evb[i - 5] if i >= 5 else None
            if e is not None:
                e[0].record()
            q8_norm_rope_cache_write(bk, bv, kb_, vb_, bslots, bpos, kn, table, rot, 1e-6, Hkv, hs, w.block_size)
            if e is not None:
                e[1].record()
            q8_cache_write(bk, bv, kb_, vb_, bslots, Hkv, hs, w.block_size)
            if e is not None:
                e[2].record()
        torch.cuda.synchronize()
        tbf = np.array([e[0].elapsed_time(e[1]) for e in evb]) * 1e3
        tbp = np.array([e[1].elapsed_time(e[2]) for e in evb]) * 1e3
        Bb = Tb * Hkv * (2 * hs * 4 + 2 * (hs + 4)) + 4 * Tb       # f32 K/V read, packed rows written, slots
        normrope = {"rot": rot, "theta": 10000.0,
                    "q_norm_rope_us_mean": round(float(tq.mean()), 2),
                    "norm_rope_cache_write_us_mean": round(float(tw.mean()), 2),
                    "decode_us_mean": round(float(td.mean()), 2),
                    "three_launch_step_us_mean": round(float(t3.mean()), 2),
                    "qk_norm_rope_cache_write_us_mean": round(float(tqk.mean()), 2),
                    "two_launch_step_us_mean": round(float(t2.mean()), 2),
                    "fused_step_us": round(t_fused, 2),
                    "fused_step_GBps": round(B_nr / (t_fused * 1e-6) / 1e9, 1),
                    "fused_step_frac_hbm_peak": round(B_nr / (t_fused * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "two_launch_step_us_back_to_back": round(t_two, 2),
                    "plain_step_us_back_to_back": round(t_plain, 2),
                    "fused_step_equals_two_launch_bitwise": fused_equal,
                    "bulk_tokens": Tb,
                    "bulk_norm_rope_cache_write_us_mean": round(float(tbf.mean()), 2),
                    "bulk_plain_cache_write_us_mean": round(float(tbp.mean()), 2),
                    "bulk_algorithmic_bytes": Bb,
                    "bulk_norm_rope_GBps": round(Bb / (float(tbf.mean()) * 1e-6) / 1e9, 1),
                    "bulk_norm_rope_frac_hbm_peak": round(Bb / (float(tbf.mean()) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "note": "the step with q8_norm_rope on q rows and q8_norm_rope_cache_write for the new K/V "
                            "(three launches with the decode), the same with q8_norm_rope_qk_cache_write (two "
                            "launches), each launch bracketed by events; then q8_norm_rope_decode_step (one launch), "
                            "the two-launch form and the plain q8_decode_step timed over back-to-back steps "
                            "(events at the ends); then a 16384-token bulk write; positions L-1 for the step"}
        del kb_, vb_

    # ---- selected-token step: block scores -> visible lists -> visible-list decode ----
    selected = None
    if not args.no_reference:
        ws_ = wl.selected()
        ratio_, k_ = 64, 32
        kh5, vh5 = ws_.empty_caches()
        kc5, vc5 = u32(kh5), u32(vh5)
        del kh5, vh5
        for slots, k, v in ws_.fill_chunks():
            q8_cache_write(f32(k), f32(v), kc5, vc5, u32(slots), ws_.num_kv_heads, ws_.head_size, ws_.block_size)
        g5 = np.random.default_rng(13)
        nblk5 = int(ws_.context_lens.max()) // ratio_
        sc5 = (g5.random((ws_.num_seqs, nblk5)) * 0.5).astype(np.float32)
        for s_ in range(ws_.num_seqs):
            n_ = int(ws_.num_visible[s_])
            sc5[s_, np.unique(ws_.visible_pos[s_, :n_] // ratio_)[:k_]] = 1.0 + g5.random(k_).astype(np.float32)
        sc5d, cl5 = f32(sc5), u32(ws_.context_lens)
        vstride = ws_.visible_pos.shape[1]
        vis5 = torch.zeros((ws_.num_seqs, vstride), dtype=torch.int32, device=dev)
        nv5 = torch.zeros((ws_.num_seqs,), dtype=torch.int32, device=dev)
        mstride5 = (nblk5 + 1 + 31) // 32
        mask5 = torch.zeros((ws_.num_seqs, mstride5), dtype=torch.int32, device=dev)
        q5, bt5 = f32(ws_.q()), u32(ws_.block_tables)
        out5 = torch.empty((ws_.num_seqs, ws_.num_heads, ws_.head_size), dtype=torch.float32, device=dev)
        ws5 = torch.zeros(max(1, q8_paged_decode_workspace_bytes(ws_.num_seqs, ws_.num_heads, ws_.num_kv_heads,
                                                                 ws_.head_size, ws_.block_size, vstride)),
                          dtype=torch.uint8, device=dev)

        def sel_step(ev=None):
            if ev is not None:
                ev[0].record()
            q8_index_select(sc5d, cl5, ratio_, k_, vstride, visible_pos=vis5, num_visible=nv5,
                            mask_stride=mstride5, visible_mask=mask5)
            if ev is not None:
                ev[1].record()
            q8_paged_decode(q5, kc5, vc5, bt5, cl5, ws_.scale, ws_.num_kv_heads, ws_.block_size,
                            visible_pos=vis5, num_visible=nv5, out=out5, workspace=ws5)
            if ev is not None:
                ev[2].record()

        for _ in range(5):
            sel_step()
        torch.cuda.synchronize()
        ev5 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(100)]
        for e in ev5:
            sel_step(e)
        torch.cuda.synchronize()
        ts_ = np.array([e[0].elapsed_time(e[1]) for e in ev5]) * 1e3
        td_ = np.array([e[1].elapsed_time(e[2]) for e in ev5]) * 1e3
        B5 = ws_.effective_kv_bytes()
        selected = {"workload": "selected-token decode S=16 H=32 Hkv=4 hs=128 bs=16, 65536-token capacity, "
                                "32 of 1023 64-token blocks + tail per sequence (seed 5)",
                    "index_select_us_mean": round(float(ts_.mean()), 2),
                    "decode_us_mean": round(float(td_.mean()), 2),
                    "effective_kv_bytes": B5,
                    "decode_effective_GBps": round(B5 / (float(td_.mean()) * 1e-6) / 1e9, 1),
                    "lists_match_workload": bool(np.array_equal(nv5.cpu().numpy().view(np.uint32),
                                                                ws_.num_visible)),
                    "note": "q8_index_select over one score per complete block (16 rows x 1023, lists and block "
                            "bitmasks), then "
                            "q8_paged_decode over the lists; scores rank each sequence's workload blocks first"}
        del kc5, vc5

    hot = None
    if not args.no_hot:
        # the same step back to back on one cache copy: its 327 MB mostly still
        # in the 256 MB Infinity Cache from the previous step
        for i in range(5):
            step(0)
        us_hot = _timed(lambda i: step(0), max(20, min(args.steps, 200)))
        hot = {"us_mean_back_to_back": round(us_hot, 2),
               "effective_GBps": round(w.effective_kv_bytes() / (us_hot * 1e-6) / 1e9, 1),
               "note": "warm Infinity Cache: not a bound of the cold figure above"}

    # ---- the other configurations' decodes and the padded bulk write, and the
    # practical HBM ceiling of the decode's access pattern ----
    long_leg = mha_legs = ceiling = None
    if not args.no_reference:
        long_leg = bench_long_context(dev)
        mha_legs = bench_mha256(dev)
        ceiling = bench_ceiling(dev, w, layers, bt)

    # algorithmic bytes of the step's cache write: f32 K and V read, packed rows written
    Bw = int(step_slots.size) * Hkv * (2 * hs * 4 + 2 * (hs + 4)) + 4 * int(step_slots.size)
    step_s = ms_per_step * 1e-3
    value = B / step_s / 1e9
    dec_mean = float(t_dec.mean())
    achieved = (B + Bw) / (region_us * 1e-6) / 1e9
    digest = kernel_sources_digest()
    traffic = read_traffic(digest)

    # ---- correctness of the timed configuration + CPU oracle baseline ----
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle
        oracle.build(force=False)
        for slots, k, v in fill_host:
            oracle.cache_write(k, v, kh, vh, slots, Hkv, hs, w.block_size)
        oracle.cache_write(step_k, step_v, kh, vh, step_slots, Hkv, hs, w.block_size)
        qh = w.q()
        ref = oracle.paged_decode(qh, kh, vh, w.block_tables, w.context_lens, w.scale, Hkv, w.block_size,
                                  max_context_len=mcl, nthreads=cpu_threads())
        got = out.cpu().numpy()
        err = np.abs(got.astype(np.float64) - ref)
        parity = {"max_abs_err": float(err.max()),
                  "within_1e-4": bool(np.all(err <= 1e-4 + 1e-4 * np.abs(ref)))}
        cpu = cpu_baseline(oracle, w, qh, kh, vh, mcl, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped decode step (one launch): 64-token q8 cache append + q8 paged decode, "
                               "S=64 H=32 Hkv=8 hs=128 bs=16 L~U[512,4096] (seed 2), %d rotated layer caches"
                               % len(layers),
                   "num_seqs": S, "num_heads": H, "num_kv_heads": Hkv, "head_size": hs, "block_size": w.block_size,
                   "attended_tokens": int(w.attended_counts().sum()), "effective_kv_bytes": B,
                   "kv_storage": "int8 codes + f32 per-token scale"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(S * H / step_s, 1),
        "step_launch": {"us_mean_back_to_back": round(region_us, 2),
                        "effective_GBps": round(B / (region_us * 1e-6) / 1e9, 1),
                        "seq_heads_per_s": round(S * H / (region_us * 1e-6), 1),
                        "note": "HIP events on the launch stream around the timed region's K launches; "
                                "per_launch_events: an event pair around each launch (each also holds that "
                                "launch's dispatch latency)",
                        "per_launch_events": {"us_mean": round(dec_mean, 2),
                                              "us_median": round(float(np.median(t_dec)), 2),
                                              "us_p10": round(float(np.percentile(t_dec, 10)), 2),
                                              "us_p90": round(float(np.percentile(t_dec, 90)), 2)}},
        "two_launch_reference": reference,
        "multi_row_decode": multi,
        "f32_cache_reference": f32ref,
        "bf16_cache_reference": bf16ref,
        "norm_rope_step": normrope,
        "selected_step": selected,
        "long_context": long_leg,
        "mha256_decode": None if mha_legs is None else mha_legs[0],
        "mha256_write": None if mha_legs is None else mha_legs[1],
        "practical_ceiling": ceiling,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "q8_decode_step (one launch: decode_split_kernel, appending the step's tokens)",
                     "algorithmic_bytes_per_launch": B + Bw,
                     "launch_us": round(region_us, 2),
                     "launch_us_source": "HIP events around the timed region's launches on the launch stream, "
                                         "divided by their number"},
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "hot_single_cache": hot,
        "setup_s": round(setup_s, 1),
        "priming_steps": n_prime,
        "kernel_sources_sha256_16": digest,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
