"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle/sanitize_check.c calls every oracle entry point on small edge-case
inputs in exactly sized heap buffers; built with gcc -fsanitize=address,
undefined and no recovery, any out-of-bounds access, null dereference or
undefined arithmetic in the oracle aborts the run.  A wrong read in the oracle
would otherwise go unnoticed by the parity tests, which trust its output."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "sanitize_check")
    cmd = [gcc, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-fopenmp", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "sanitize_check.c"), "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr + build.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", OMP_NUM_THREADS="2")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
