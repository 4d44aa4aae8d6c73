"""The append kernel's branch-free E4M3 block scale (e4m3_scale_fast in
the device codec) against the oracle's brute-force nearest-code search, on
the host: every binary32 near the places where the chosen code changes or
ties, the saturation and subnormal edges, and random magnitudes (release
post of the gzenz/ninfer fork, "NVFP4 KV cache (from scratch)", bullet 1).
The codec header is compiled for the host with hipcc; the oracle with gcc."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


def test_fast_scale_code_matches_oracle():
    if shutil.which("gcc") is None or not os.path.exists(HIPCC):
        pytest.skip("gcc or hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        obj = os.path.join(tmp, "oracle.o")
        subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-c",
                        "-o", obj, oracle.SRC], check=True)
        cobj = os.path.join(tmp, "check.o")
        subprocess.run([HIPCC, "-O1", "-std=c++17", "-ffp-contract=off", "-c",
                        "-I", os.path.join(ROOT, "nvfp4_quantized_kv_amd", "csrc"),
                        os.path.join(ROOT, "tests", "scale_fast_check.cpp"), "-o", cobj], check=True)
        exe = os.path.join(tmp, "check")
        subprocess.run([HIPCC, cobj, obj, "-fopenmp", "-o", exe, "-lm"], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout
