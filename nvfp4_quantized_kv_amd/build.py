"""Build libnvfp4kv.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4kv.so")

SOURCES = ["kv_append.hip", "decode_attn.hip", "decode_attn_gr.hip", "kv_spill.hip", "nvfp4kv_api.cpp"]
HEADERS = ["nvfp4kv_codec.hpp", "nvfp4kv_internal.hpp", "nvfp4kv_rowq.hpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep packed-fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-instruction accumulators in VGPRs: the softmax rescales them with
    # ordinary vector instructions, which cannot address AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


# the checked build: every entry point range-checks the device-side tables it
# trusts (copied back on the call's stream) before launching anything
DEBUG_LIB = os.path.join(PKG, "libnvfp4kv_debug.so")


def _run(cmd, verbose: bool) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out:
        print(out)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Build libnvfp4kv.so and, with `debug`, the checked libnvfp4kv_debug.so:
    every source compiled to an object (in parallel), then one link per
    library."""
    import concurrent.futures
    import tempfile
    variants = [(LIB, [])] + ([(DEBUG_LIB, ["-DNVFP4KV_DEBUG=1"])] if debug else [])
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory() as tmp:
        jobs = []
        for li, (_, extra) in enumerate(variants):
            for src in SOURCES:
                obj = os.path.join(tmp, f"{li}_{src}.o")
                jobs.append((obj, [hipcc(), *compile_flags, *extra, "-I", os.path.join(ROOT, "include"), "-c",
                                   "-o", obj, os.path.join(CSRC, src)]))
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda j: _run(j[1], verbose), jobs))
        for li, (out_path, _) in enumerate(variants):
            objs = [os.path.join(tmp, f"{li}_{src}.o") for src in SOURCES]
            _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_path + ".tmp", *objs], verbose)
            os.replace(out_path + ".tmp", out_path)
    return LIB


def stale(path: str = LIB) -> bool:
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    deps = [os.path.join(CSRC, s) for s in SOURCES + HEADERS] + [os.path.join(ROOT, "include", "nvfp4kv.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose=True))
