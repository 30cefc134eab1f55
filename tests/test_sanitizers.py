"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The oracle (``oracle/oracle.c``) built with ``-fsanitize=address,undefined``
  runs the oracle's own pin tests in a child process (the sanitizer runtime
  preloaded into Python).
* The C-ABI entry points (``hda_api.cpp``: argument checks, plans, workspace
  layouts) built for the host with the same sanitizers, with stand-ins for
  the kernel launchers (``tests/native/host_stubs.cpp``), are driven over
  about 20,000 valid and invalid calls (``tests/native/host_driver.cpp``);
  the stand-ins check that every workspace pointer handed to a launcher lies
  inside the workspace the library asked for.

Any sanitizer report or overrun fails the test.  Nothing here uses a GPU.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(not shutil.which("gcc") or not _runtime("libasan.so"), reason="gcc with ASan not available")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", *SAN, "-o", str(lib),
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    env = dict(os.environ)
    env.update(HDA_ORACLE_LIB=str(lib), LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report


@pytest.mark.skipif(not shutil.which("g++") or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="g++ or the HIP headers not available")
def test_host_entry_points_under_asan_ubsan(tmp_path):
    exe = tmp_path / "hda_host_san"
    csrc = os.path.join(ROOT, "full_kv_cache_amd", "csrc")
    native = os.path.join(ROOT, "tests", "native")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           "-I", os.path.join(ROOT, "include"), "-I", csrc,
                           os.path.join(csrc, "hda_api.cpp"), os.path.join(native, "host_stubs.cpp"),
                           os.path.join(native, "host_driver.cpp"), "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"))
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "0 workspace overruns" in r.stdout
