"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU touched).

tests/host_sanitize_check.cpp is linked with the library's api.hip, decode.hip
and baseline_cache.hip (argument validation, split planning, workspace sizing)
with the host pass instrumented (-Xarch_host before each -fsanitize, so no GPU
code is built with a sanitizer), and the other launchers stubbed.  It calls
every entry point with arguments that fail validation, up to 32-bit extremes,
and checks the workspace query against the launches' own plans over a grid of
shapes.  Its first run found record counts wrapping at 2^32 - 1 sequences."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int8_paged_kv_amd", "csrc")


def test_library_host_code_clean_under_asan_and_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc) and shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    exe = str(tmp_path / "host_sanitize_check")
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    cmd = ([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san +
           ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "decode.hip"), os.path.join(CSRC, "baseline_cache.hip"),
            "-x", "hip", os.path.join(ROOT, "tests", "host_sanitize_check.cpp"), "-o", exe])
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if build.returncode != 0 and "asan" in (build.stderr + build.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", HIP_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout[-2000:] + run.stderr[-3000:]
