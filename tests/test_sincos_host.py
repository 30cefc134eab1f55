"""CPU check of the kernels' RoPE cos/sin evaluation (the library's
``sincos_angle``: Cody-Waite reduction by pi/2 and Taylor series in fp64,
rounded once to fp32), built for the host from the same header: every
angle of both RoPE configurations up to position 40000 and a million
random fp32 angles up to 2^31 must equal libm's fp64 cos / sin rounded to
fp32 (the oracle's evaluation).  About 6.4 million angles."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_sincos_matches_libm(tmp_path):
    exe = tmp_path / "sincos_check"
    src = os.path.join(ROOT, "tests", "native", "sincos_check.cpp")
    inc = os.path.join(ROOT, "full_kv_cache_amd", "csrc")
    subprocess.check_call([HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17",
                           "-I", inc, src, "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(" 0 mismatches") == 3
