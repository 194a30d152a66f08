#!/usr/bin/env python3
"""Turn rocprofv3 output of bench.py runs into the text summaries under profiles/.

Expected layout of DIR (what the commands printed in each summary write):
  DIR/trace/bench_kernel_stats.csv, DIR/trace/bench_kernel_trace.csv
      rocprofv3 --kernel-trace --stats -f csv -o bench, of bench.py
  DIR/pmc_FETCH_SIZE/bench_counter_collection.csv, DIR/pmc_WRITE_SIZE/...
      rocprofv3 --pmc FETCH_SIZE (resp. WRITE_SIZE) -f csv -o bench, of bench.py
  DIR/copy_FETCH_SIZE/copy_counter_collection.csv, DIR/copy_WRITE_SIZE/...
      the same counters over bench.py --copy-calibration MIB (a plain copy of
      known size), which give the factor from each counter to HBM bytes
  DIR/pmc_FETCH_SIZE.log, DIR/pmc_WRITE_SIZE.log, DIR/copy_FETCH_SIZE.log
      stdout of those runs (bench's JSON line carries the kernel-source digest)

Optionally DIR/trace_all/ and DIR/trace_all.log: the same trace of a run with
the reference legs (every kernel the bench times).

Writes profiles/q8_paged_decode_llama_kernel_trace.txt,
profiles/q8_paged_decode_llama_traffic.txt and, with trace_all,
profiles/llama_step_all_kernels_trace.txt; the latter is what bench.py reads
for roofline.traffic while the kernel sources still match its digest.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE_KERNELS = ("decode_split_kernel",)
WRITE_KERNEL = "cache_write_kernel"

TRACE_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d {d}/trace -o bench -f csv "
             "-- python3 /root/repo/bench.py --steps 200 --warmup 20 --no-cpu --no-reference --no-hot")
PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 rocprofv3 --pmc {c} -d {d}/pmc_{c} -o bench -f csv "
           "-- python3 /root/repo/bench.py --steps 3 --warmup 1 --no-cpu --no-reference --prime-s 0 --no-hot")
TRACE_ALL_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d {d}/trace_all -o bench -f csv "
                 "-- python3 /root/repo/bench.py --steps 200 --warmup 20 --no-cpu --no-hot")
L2_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum "
          "-d {d}/pmc_L2 -o bench -f csv -- python3 /root/repo/bench.py --steps 3 --warmup 1 --no-cpu --no-reference --prime-s 0 --no-hot")
PMC_ALL_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc {c} -d {d}/pmc_all_{c} -o bench "
               "-f csv -- python3 /root/repo/bench.py --steps 3 --warmup 1 --no-cpu --prime-s 0 --no-hot")
SQ_PASSES = (("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM",
              "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
             ("SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_SCA",
              "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM", "SQ_WAVES"))
SQ_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 rocprofv3 --pmc {cs} -d {d}/pmc_sq{i} -o bench "
          "-f csv -- python3 /root/repo/bench.py --steps 3 --warmup 1 --no-cpu --no-reference --prime-s 0 --no-hot")
COPY_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 90 rocprofv3 --pmc {c} -d {d}/copy_{c} -o copy -f csv "
            "-- python3 /root/repo/bench.py --copy-calibration {mib}")


def kname(name: str) -> str:
    """A kernel's name without its return type, namespaces and parameter list."""
    return name.replace("void ", "").replace("q8kv::", "").replace("(anonymous namespace)::", "").split("(")[0]


def short(name: str) -> str:
    for k in DECODE_KERNELS + (WRITE_KERNEL, "copyBuffer"):
        if k in name:
            return kname(name)
    return name[:60]


def last_json(path: str) -> dict:
    with open(path) as f:
        lines = [ln for ln in f.read().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1])


def counters(path: str):
    """{(kernel, grid): [counter value per dispatch]}"""
    out = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            out[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return out


def counters_by_name(path: str):
    """{(kernel, grid, counter): [value per dispatch]}"""
    out = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            out[(r["Kernel_Name"], int(r["Grid_Size"]), r["Counter_Name"])].append(float(r["Counter_Value"]))
    return out


def step_dispatches(cnt, step_grid_of):
    """Counter values of the decode-step launches: the grid the step uses for each kernel."""
    res = {}
    for (name, grid), vals in cnt.items():
        for k in DECODE_KERNELS:
            if k in name and grid == step_grid_of.get(k):
                res[k] = (name, grid, vals)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("dir", help="directory holding the rocprofv3 outputs")
    ap.add_argument("--cmd-dir", default="/root/repo/gpurun_out/prof",
                    help="DIR as written in the recorded commands")
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args()
    d = args.dir
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)

    # ---- kernel trace: per-kernel durations of the step's launches ----
    trace = defaultdict(list)
    with open(os.path.join(d, "trace", "bench_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            trace[(r["Kernel_Name"], grid, int(r["Workgroup_Size_X"]), int(r["VGPR_Count"]),
                   int(r["Accum_VGPR_Count"]), int(r["SGPR_Count"]), int(r["LDS_Block_Size"]),
                   int(r["Scratch_Size"]))].append(dur)
    bench_trace = last_json(os.path.join(d, "trace.log"))
    digest = bench_trace["kernel_sources_sha256_16"]
    # The step's launches: the decode kernel's (kernel, grid) with the most
    # dispatches (warmup, timed and event-timed steps); fill-phase launches
    # are the cache writer's.
    step_grid = {}
    best = {}
    for key, durs in trace.items():
        for k in DECODE_KERNELS:
            if k in key[0] and len(durs) > best.get(k, 0):
                best[k] = len(durs)
                step_grid[k] = key[1]
    rows = []
    for key, durs in sorted(trace.items(), key=lambda kv: -sum(kv[1])):
        name, grid, wg, vgpr, agpr, sgpr, lds, scr = key
        is_step = any(k in name and grid == step_grid.get(k) for k in DECODE_KERNELS)
        rows.append((short(name), grid, wg, len(durs), statistics.mean(durs), statistics.median(durs),
                     min(durs), max(durs), vgpr, agpr, sgpr, lds, scr, is_step))

    split_us = mean_of(rows, "decode_split_kernel")
    eff = bench_trace["config"]["effective_kv_bytes"]
    lines = [
        "# rocprofv3 kernel trace of the decode step, Llama-3-8B-shaped batch",
        "# (S=64 H=32 Hkv=8 head_size=128 block_size=16, context lengths U[512,4096], seed 2)",
        "#",
        "# command (from any directory on the GPU machine):",
        "#   " + TRACE_CMD.format(d=args.cmd_dir),
        "# summarised with: python3 bench_profile.py <that -d directory's parent>",
        "#",
        "# kernel_sources_sha256_16: %s" % digest,
        "# durations in microseconds per dispatch; step = one launch of q8_decode_step (decode_split_kernel: "
        "appends the 64 new tokens, attends, and combines shared sequences)",
        "",
        "%-62s %9s %4s %5s %9s %9s %9s %9s %5s %5s %5s %6s %6s" % (
            "kernel", "grid", "wg", "calls", "mean_us", "median_us", "min_us", "max_us", "vgpr", "agpr", "sgpr",
            "lds", "scratch"),
    ]
    for r in rows:
        lines.append("%-62s %9d %4d %5d %9.2f %9.2f %9.2f %9.2f %5d %5d %5d %6d %6d%s" % (
            r[0][:62], r[1], r[2], r[3], r[4], r[5], r[6], r[7], r[8], r[9], r[10], r[11], r[12],
            "  <- step" if r[13] else ""))
    lines += [
        "",
        "step launch (decode_split_kernel mean): %.2f us" % split_us,
        "  effective int8 KV bytes per step: %d -> %.1f GB/s" % (eff, eff / (split_us * 1e-6) / 1e9),
        "bench.py in the same run (HIP events on the launch stream around the timed launches): %.2f us per "
        "launch, effective %.1f GB/s" % (bench_trace["step_launch"]["us_mean_back_to_back"],
                                         bench_trace["step_launch"]["effective_GBps"]),
        "",
        "rocprofv3 --stats table (all dispatches of each kernel, fill phase included):",
    ]
    with open(os.path.join(d, "trace", "bench_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            lines.append("  %-62s calls %4s avg_ns %12s min_ns %9s max_ns %9s" % (
                short(r["Name"])[:62], r["Calls"], r["AverageNs"], r["MinNs"], r["MaxNs"]))
    with open(os.path.join(ROOT, "profiles", "q8_paged_decode_llama_kernel_trace.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # ---- optional: every kernel of a run with the reference legs ----
    all_dir = os.path.join(d, "trace_all")
    if os.path.exists(os.path.join(all_dir, "bench_kernel_trace.csv")):
        per = defaultdict(list)
        with open(os.path.join(all_dir, "bench_kernel_trace.csv")) as f:
            for r in csv.DictReader(f):
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                per[(r["Kernel_Name"], grid, int(r["VGPR_Count"]), int(r["LDS_Block_Size"]))].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        allj = last_json(os.path.join(d, "trace_all.log"))
        out = [
            "# rocprofv3 kernel trace of every kernel the bench runs, Llama-3-8B-shaped batch",
            "# (step, two-launch reference, 4-row decode, f32- and bf16-cache steps, norm + rotary step, 16384-token bulk",
            "# writes, selected-token step: block selection + visible-list decode, long-context decode,",
            "# MHA head_size=256 decode and its 4096-token padded write, and the measurement kernels of the",
            "# practical HBM ceiling)",
            "#",
            "# command (from any directory on the GPU machine):",
            "#   " + TRACE_ALL_CMD.format(d=args.cmd_dir),
            "# summarised with: python3 bench_profile.py <that -d directory's parent>",
            "#",
            "# durations in microseconds per dispatch, grouped by kernel and grid",
            "",
            "%-60s %9s %5s %9s %9s %9s %5s %6s" % ("kernel", "grid", "calls", "mean_us", "median_us", "max_us",
                                                  "vgpr", "lds"),
        ]
        for (name, grid, vgpr, lds), durs in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            nm = kname(name)
            out.append("%-60s %9d %5d %9.2f %9.2f %9.2f %5d %6d" % (
                nm[:60], grid, len(durs), statistics.mean(durs), statistics.median(durs), max(durs), vgpr, lds))
        out += ["", "bench.py line of the same run (reference legs):"]
        for k in ("two_launch_reference", "multi_row_decode", "f32_cache_reference", "bf16_cache_reference",
                  "norm_rope_step",
                  "selected_step", "long_context", "mha256_decode", "mha256_write", "practical_ceiling"):
            out.append("  %s: %s" % (k, json.dumps(allj.get(k))))
        with open(os.path.join(ROOT, "profiles", "llama_step_all_kernels_trace.txt"), "w") as f:
            f.write("\n".join(out) + "\n")

    # ---- HBM traffic from FETCH_SIZE / WRITE_SIZE, calibrated by the copy ----
    mib = args.copy_mib
    copy_bytes = mib * (1 << 20)
    factor = {}
    raw_copy = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cc = counters(os.path.join(d, "copy_" + c, "copy_counter_collection.csv"))
        vals = [v for (name, _), vs in cc.items() if "copyBuffer" in name for v in vs]
        kib = statistics.median(vals)
        raw_copy[c] = kib
        factor[c] = copy_bytes / (kib * 1024.0)
    pmc = {}
    pmc_digest = set()
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        pmc[c] = step_dispatches(counters(os.path.join(d, "pmc_" + c, "bench_counter_collection.csv")), step_grid)
        pmc_digest.add(last_json(os.path.join(d, "pmc_%s.log" % c))["kernel_sources_sha256_16"])
    if pmc_digest != {digest}:
        raise SystemExit("counter runs and trace run were taken on different kernel sources: %s vs %s"
                         % (pmc_digest, digest))
    per_kernel = {}
    for k in DECODE_KERNELS:
        rd = statistics.median(pmc["FETCH_SIZE"][k][2]) * 1024.0 * factor["FETCH_SIZE"]
        wr = statistics.median(pmc["WRITE_SIZE"][k][2]) * 1024.0 * factor["WRITE_SIZE"]
        per_kernel[k] = (statistics.median(pmc["FETCH_SIZE"][k][2]), statistics.median(pmc["WRITE_SIZE"][k][2]),
                         rd, wr)
    dec_bytes = sum(per_kernel[k][2] + per_kernel[k][3] for k in DECODE_KERNELS)
    t = [
        "# HBM traffic of the step launch (append + decode), Llama-3-8B-shaped batch",
        "# (S=64 H=32 Hkv=8 head_size=128 block_size=16, context lengths U[512,4096], seed 2)",
        "#",
        "# commands (from any directory on the GPU machine), one counter per run:",
        "#   " + PMC_CMD.format(c="FETCH_SIZE", d=args.cmd_dir),
        "#   " + PMC_CMD.format(c="WRITE_SIZE", d=args.cmd_dir),
        "#   " + COPY_CMD.format(c="FETCH_SIZE", d=args.cmd_dir, mib=mib),
        "#   " + COPY_CMD.format(c="WRITE_SIZE", d=args.cmd_dir, mib=mib),
        "# summarised with: python3 bench_profile.py <that -d directory's parent>",
        "#",
        "# Calibration: a plain copy of %d bytes (rocclr copyBuffer, %d MiB) reads FETCH_SIZE %.1f KiB and" % (
            copy_bytes, mib, raw_copy["FETCH_SIZE"]),
        "# WRITE_SIZE %.1f KiB per dispatch, so HBM bytes = FETCH_SIZE KiB * 1024 * %.4f and" % (
            raw_copy["WRITE_SIZE"], factor["FETCH_SIZE"]),
        "# WRITE_SIZE KiB * 1024 * %.4f." % factor["WRITE_SIZE"],
        "#",
        "# per dispatch (median over the step's launches):",
    ]
    for k in DECODE_KERNELS:
        fk, wk, rd, wr = per_kernel[k]
        t.append("#   %-20s FETCH_SIZE %10.1f KiB -> %12.0f B read, WRITE_SIZE %9.1f KiB -> %11.0f B written" % (
            k, fk, rd, wk, wr))
    l2_line, l2_key = [], []
    l2_csv = os.path.join(d, "pmc_L2", "bench_counter_collection.csv")
    if os.path.exists(l2_csv):
        if last_json(os.path.join(d, "pmc_L2.log"))["kernel_sources_sha256_16"] != digest:
            raise SystemExit("L2 counter run was taken on different kernel sources")
        cb = counters_by_name(l2_csv)
        hit = [v for (name, grid, c), vs in cb.items()
               if "decode_split_kernel" in name and grid == step_grid.get("decode_split_kernel") and c.startswith("TCC_HIT")
               for v in vs]
        miss = [v for (name, grid, c), vs in cb.items()
                if "decode_split_kernel" in name and grid == step_grid.get("decode_split_kernel") and c.startswith("TCC_MISS")
                for v in vs]
        if hit and miss:
            h, m = statistics.median(hit), statistics.median(miss)
            l2_line = ["#", "# L2 (TCC) requests of the step launch, median per dispatch (command:",
                       "#   " + L2_CMD.format(d=args.cmd_dir) + "):",
                       "#   hits %.0f, misses %.0f -> hit rate %.4f (K/V tiles are read once per row group and"
                       " loaded nontemporal;" % (h, m, h / (h + m)),
                       "#   the hits are the shared q rows, block tables, lengths and the re-read partial records)"]
            l2_key = ["l2_hit_rate: %.4f" % (h / (h + m))]
    t += l2_line
    t += [
        "#   algorithmic bytes per step: int8 KV (codes + scale word of every attended row, K and V) %d"
        " + cache append %d" % (eff, bench_trace["roofline"]["algorithmic_bytes_per_launch"] - eff),
        "#   measured step traffic / algorithmic = %.4f" % (dec_bytes / bench_trace["roofline"]["algorithmic_bytes_per_launch"]),
        "",
        "kernel_sources_sha256_16: %s" % digest,
        "fetch_factor: %.6f" % factor["FETCH_SIZE"],
        "write_factor: %.6f" % factor["WRITE_SIZE"],
        "split_read_bytes: %.0f" % per_kernel["decode_split_kernel"][2],
        "split_write_bytes: %.0f" % per_kernel["decode_split_kernel"][3],
        "hbm_bytes_per_step: %.0f" % dec_bytes,
    ] + l2_key
    with open(os.path.join(ROOT, "profiles", "q8_paged_decode_llama_traffic.txt"), "w") as f:
        f.write("\n".join(t) + "\n")

    # ---- optional: SQ instruction and wait counters of the step launch ----
    sq_csv = [os.path.join(d, "pmc_sq%d" % i, "bench_counter_collection.csv") for i in (1, 2)]
    if all(os.path.exists(x) for x in sq_csv):
        vals = {}
        for i, x in enumerate(sq_csv, 1):
            if last_json(os.path.join(d, "pmc_sq%d.log" % i))["kernel_sources_sha256_16"] != digest:
                raise SystemExit("SQ counter runs were taken on different kernel sources")
            for (name, grid, c), vs in counters_by_name(x).items():
                if "decode_split_kernel" in name and grid == step_grid.get("decode_split_kernel"):
                    vals[c] = statistics.median(vs)
        q = [
            "# SQ counters of the step launch (append + decode), Llama-3-8B-shaped batch, median per dispatch",
            "# (S=64 H=32 Hkv=8 head_size=128 block_size=16, context lengths U[512,4096], seed 2)",
            "#",
            "# commands (from any directory on the GPU machine), eight SQ counters per run:",
        ] + ["#   " + SQ_CMD.format(cs=" ".join(cs), d=args.cmd_dir, i=i) for i, cs in enumerate(SQ_PASSES, 1)] + [
            "# summarised with: python3 bench_profile.py <that -d directory's parent>",
            "#",
            "# kernel_sources_sha256_16: %s" % digest,
            "",
        ]
        for c in [c for cs in SQ_PASSES for c in cs]:
            if c in vals:
                q.append("%-28s %16.0f" % (c, vals[c]))
        wc = vals.get("SQ_WAVE_CYCLES")
        if wc:
            q += ["", "fractions of wave cycles (SQ_WAVE_CYCLES):"]
            for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM",
                      "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_SCA"):
                if c in vals:
                    q.append("  %-26s %.3f" % (c, vals[c] / wc))
        if vals.get("SQ_VALU_MFMA_BUSY_CYCLES") is not None and split_us:
            # summed over the 256 CUs; the step's cycles from the trace's mean at the 2.4 GHz peak clock
            per_cu = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / 256
            q += ["", "MFMA busy cycles per CU %.0f over a %.2f us step (%.0f cycles at 2.4 GHz): %.3f"
                  % (per_cu, split_us, split_us * 2400, per_cu / (split_us * 2400))]
        with open(os.path.join(ROOT, "profiles", "q8_paged_decode_llama_sq_counters.txt"), "w") as f:
            f.write("\n".join(q) + "\n")

    # ---- optional: HBM traffic of every kernel of a run with the reference legs ----
    fa = os.path.join(d, "pmc_all_FETCH_SIZE", "bench_counter_collection.csv")
    wa = os.path.join(d, "pmc_all_WRITE_SIZE", "bench_counter_collection.csv")
    if os.path.exists(fa) and os.path.exists(wa):
        jf = last_json(os.path.join(d, "pmc_all_FETCH_SIZE.log"))
        if {jf["kernel_sources_sha256_16"], last_json(os.path.join(d, "pmc_all_WRITE_SIZE.log"))[
                "kernel_sources_sha256_16"]} != {digest}:
            raise SystemExit("all-legs counter runs were taken on different kernel sources")
        cf, cw = counters(fa), counters(wa)
        durs = {}
        if os.path.exists(os.path.join(all_dir, "bench_kernel_trace.csv")):
            acc = defaultdict(list)
            with open(os.path.join(all_dir, "bench_kernel_trace.csv")) as f:
                for r in csv.DictReader(f):
                    grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                    acc[(r["Kernel_Name"], grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            durs = {k: statistics.median(v) for k, v in acc.items()}
        out = [
            "# HBM traffic of every kernel the bench runs (step, two-launch reference, 4-row decode, f32- and",
            "# bf16-cache steps, norm + rotary step and 16384-token bulk writes, selected-token step, long-context and",
            "# MHA-256 decodes, the padded 4096-token write, ceiling kernels), median per dispatch",
            "# of each (kernel, grid), calibrated by the plain copy as in q8_paged_decode_llama_traffic.txt",
            "# (FETCH_SIZE x %.4f, WRITE_SIZE x %.4f)" % (factor["FETCH_SIZE"], factor["WRITE_SIZE"]),
            "#",
            "# commands (from any directory on the GPU machine), one counter per run:",
            "#   " + PMC_ALL_CMD.format(c="FETCH_SIZE", d=args.cmd_dir),
            "#   " + PMC_ALL_CMD.format(c="WRITE_SIZE", d=args.cmd_dir),
            "# durations: median of the same (kernel, grid) in llama_step_all_kernels_trace.txt's run",
            "# summarised with: python3 bench_profile.py <that -d directory's parent>",
            "#",
            "# kernel_sources_sha256_16: %s" % digest,
            "",
            "%-62s %9s %5s %14s %13s %9s %9s" % ("kernel", "grid", "calls", "read_B", "written_B", "median_us",
                                                 "HBM_GBps"),
        ]
        for key in sorted(cf, key=lambda k: -statistics.median(cf[k]) * len(cf[k])):
            if key not in cw:
                continue
            rd = statistics.median(cf[key]) * 1024.0 * factor["FETCH_SIZE"]
            wr = statistics.median(cw[key]) * 1024.0 * factor["WRITE_SIZE"]
            if rd + wr < 1e6:
                continue
            us = durs.get(key)
            nm = kname(key[0])
            out.append("%-62s %9d %5d %14.0f %13.0f %9s %9s" % (
                nm[:62], key[1], len(cf[key]), rd, wr, "%.2f" % us if us else "-",
                "%.0f" % ((rd + wr) / (us * 1e-6) / 1e9) if us else "-"))
        mr, f32, b16, nr, sel, lg, md, mw = (jf.get(k) or {} for k in (
            "multi_row_decode", "f32_cache_reference", "bf16_cache_reference", "norm_rope_step", "selected_step", "long_context",
            "mha256_decode", "mha256_write"))
        out += [
            "",
            "algorithmic bytes of the reference legs (bench.py line of the FETCH_SIZE run):",
            "  step decode: %d (int8 KV of every attended row, K and V)" % eff,
            "  4-row decode: the same prefixes, read once when the rows of a sequence share the reads: %d;"
            " counted per row: %s" % (eff, mr.get("per_row_kv_bytes")),
            "  f32-cache decode: %s" % f32.get("f32_kv_bytes"),
            "  bf16-cache decode: %s" % b16.get("bf16_kv_bytes"),
            "  bulk writes (16384 tokens): %s" % nr.get("bulk_algorithmic_bytes"),
            "  selected-token decode: %s" % sel.get("effective_kv_bytes"),
            "  long-context decode: %s" % lg.get("effective_kv_bytes"),
            "  MHA head_size=256 decode: %s" % md.get("effective_kv_bytes"),
            "  MHA head_size=256 4096-token write: %s" % mw.get("algorithmic_bytes"),
        ]
        with open(os.path.join(ROOT, "profiles", "llama_step_all_kernels_traffic.txt"), "w") as f:
            f.write("\n".join(out) + "\n")
        # the legs' kernels: the (kernel, grid) of the leg's instantiation launched most often
        legs = {"long_context": "decode_split_kernel<32, true, 2, false, true, 32, 64, false>",
                "mha256_decode": "decode_split_kernel<64, true, 1, false, true, 16, 64, false>",
                "mha256_write": "cache_write_kernel<false, 4, true>"}
        lt = [
            "# HBM bytes per launch of the long-context decode, the MHA head_size=256 decode and its padded",
            "# 4096-token write (bench.py legs long_context, mha256_decode, mha256_write), from the runs of",
            "# llama_step_all_kernels_traffic.txt; bench.py reads these while the sources match the digest.",
            "# Each leg's kernel is its instantiation's (kernel, grid) with the most dispatches.",
            "",
            "kernel_sources_sha256_16: %s" % digest,
        ]
        for leg, sig in legs.items():
            cands = [k for k in cf if sig in k[0] and k in cw]
            if not cands:
                continue
            key = max(cands, key=lambda k: len(cf[k]))
            rd = statistics.median(cf[key]) * 1024.0 * factor["FETCH_SIZE"]
            wr = statistics.median(cw[key]) * 1024.0 * factor["WRITE_SIZE"]
            lt += ["# %s: %s grid %d, %d dispatches: read %.0f B, written %.0f B" % (
                leg, sig, key[1], len(cf[key]), rd, wr),
                   "%s_hbm_bytes_per_launch: %.0f" % (leg, rd + wr)]
        with open(os.path.join(ROOT, "profiles", "bench_legs_traffic.txt"), "w") as f:
            f.write("\n".join(lt) + "\n")
    print("wrote profiles/q8_paged_decode_llama_kernel_trace.txt and profiles/q8_paged_decode_llama_traffic.txt")


def mean_of(rows, tag):
    sel = [r for r in rows if tag in r[0] and r[13]]
    return sel[0][4] if sel else float("nan")


if __name__ == "__main__":
    main()
