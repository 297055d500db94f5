"""CPU builds of the host-side code under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU involved):

* the C oracle, driven by tests/sanitize/oracle_main.c over every 16-bit
  pattern and ragged flush / dequantize / attend shapes in exact-size
  buffers;
* the C ABI's validation and the decode-loop cache (abi.cpp, cache.cpp,
  plan.cpp), linked against tests/sanitize/launch_stubs.cpp, whose kernel
  stand-ins read the first and last byte of every range the real kernel
  would touch and copy the cache's ring rows for real; driven by
  tests/sanitize/host_main.cpp (valid calls, extreme and invalid arguments,
  and labelled-token decode loops with prompt chunks).

Both programs exit non-zero on the first sanitizer report
(-fno-sanitize-recover=all) or on a failed check."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_quantization_quantize_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    out = _build_and_run(["gcc", "-std=c11", "-ffp-contract=off", *FLAGS, "-I", os.path.join(ROOT, "oracle"),
                          os.path.join(ROOT, "oracle", "kivi_oracle.c"), os.path.join(SAN, "oracle_main.c"),
                          "-lm", "-o", exe], exe)
    assert "oracle checks passed" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="needs g++ and the HIP headers")
def test_abi_and_cache_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_checks")
    srcs = [os.path.join(CSRC, f) for f in ("abi.cpp", "cache.cpp", "plan.cpp")]
    srcs += [os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "host_main.cpp")]
    out = _build_and_run(["g++", "-std=c++17", *FLAGS, "-Wno-unused-parameter", "-D__HIP_PLATFORM_AMD__",
                          "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                          *srcs, "-o", exe], exe)
    assert "host checks passed" in out
