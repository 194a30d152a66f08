"""Build libq8kv.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every csrc/*.hip file is compiled to an object in parallel (the decode kernel
instantiations are spread over several files), then linked into one shared
library.  Objects live in a temporary directory, never in the tree.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libq8kv.so")
# measurement kernels of the benchmark (the practical HBM ceiling), a library of their own
BENCH_LIB = os.path.join(PKG, "libq8kv_bench.so")
# the same sources with the device-side content checks (Q8_DEBUG_BOUNDS)
DEBUG_LIB = os.path.join(PKG, "libq8kv_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed-FP32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources(sub: str = "csrc"):
    return sorted(glob.glob(os.path.join(PKG, sub, "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in l)
    return r.returncode, out


def build(verbose: bool = False, jobs: int = 0) -> str:
    _build_lib(sources("csrc"), LIB, verbose, jobs)
    _build_lib(sources("csrc"), DEBUG_LIB, verbose, jobs, ["-DQ8_DEBUG_BOUNDS"])
    _build_lib(sources("csrc_bench"), BENCH_LIB, verbose, jobs)
    return LIB


def _build_lib(srcs, lib_path: str, verbose: bool, jobs: int, defines=()) -> None:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="q8kv_build_") as tmpdir:
        cmds = []
        objs = []
        for src in srcs:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([HIPCC] + FLAGS + list(defines) + inc + ["-c", src, "-o", obj])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, out), c in zip(results, cmds):
            if rc != 0:
                raise RuntimeError("hipcc failed: %s\n%s" % (" ".join(c), out))
            if out.strip() and verbose:
                print(out)
        tmp = lib_path + ".tmp%d" % os.getpid()
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, out = _run(link)
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + out)
        os.replace(tmp, lib_path)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
