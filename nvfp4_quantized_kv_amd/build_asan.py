"""Host AddressSanitizer build of the C ABI (argument checks, planning, table
checks, RoPE table): libnvfp4kv_asan.so, the checked build with its host code
instrumented.  Load it into a Python process
with the clang ASan runtime preloaded (asan_runtime())."""
from __future__ import annotations

import os
import subprocess

from .build import CSRC, HIPCC_FLAGS, PKG, ROOT, SOURCES, hipcc

ASAN_LIB = os.path.join(PKG, "libnvfp4kv_asan.so")


def asan_runtime() -> str:
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    return out


def _run(cmd) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc (host ASan build) failed:\n{res.stdout}{res.stderr}")


def build_asan() -> str:
    """The whole library with the host code instrumented (device code as in
    the regular build), every source compiled in parallel, then linked."""
    import concurrent.futures
    import tempfile
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    # the sanitizer applies to the host code only (each -fsanitize= after -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [[hipcc(), *flags, *san, "-g", "-DNVFP4KV_DEBUG=1", "-I", os.path.join(ROOT, "include"), "-c",
                 "-o", os.path.join(tmp, s + ".o"), os.path.join(CSRC, s)] for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(len(jobs)) as ex:
            list(ex.map(_run, jobs))
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
              "-shared-libsan", "-o", ASAN_LIB + ".tmp", *[os.path.join(tmp, s + ".o") for s in SOURCES]])
    os.replace(ASAN_LIB + ".tmp", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build_asan())
