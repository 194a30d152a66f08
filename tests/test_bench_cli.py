"""bench.py's command line and its kernel-source digest, without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_digest_ignores_comments_and_layout():
    import bench
    src = "int f(int a) { // note\n  return a /* c */ + 1;\n}\n"
    assert bench.code_only(src) == bench.code_only("int f(int a) {\n return a + 1; }")
    assert bench.code_only(src) != bench.code_only("int f(int a) { return a + 2; }")


def test_digest_covers_existing_sources():
    import bench
    d = bench.kernel_sources_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    for f in bench.DECODE_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "int8_paged_kv_amd", "csrc", f)), f
