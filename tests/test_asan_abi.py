"""The C ABI's host code under AddressSanitizer: the checked build with its
host code instrumented (libnvfp4kv_asan.so) runs the argument-check and
table-check tests (test_abi.py, test_checked_build.py) in a child process
with the clang ASan runtime preloaded; they must pass with no sanitizer
report.  No GPU: nothing is launched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_clean_under_host_asan():
    sys.path.insert(0, ROOT)
    from nvfp4_quantized_kv_amd import build as B
    from nvfp4_quantized_kv_amd import build_asan as A
    if B.stale(A.ASAN_LIB):
        A.build_asan()
    rt = A.asan_runtime()
    if not os.path.exists(rt):
        pytest.skip("clang ASan runtime not found")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               NVFP4KV_LIB=A.ASAN_LIB)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-W", "ignore",
                          os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_checked_build.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
