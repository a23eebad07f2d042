"""The host side of the C ABI (argument validation, the work planner and the C entry
points' argument marshalling in sigmoid_attention_amd/csrc/sigattn.cpp) built for the CPU
with AddressSanitizer and UndefinedBehaviorSanitizer, against host-only launchers that
touch no device (tests/host_san_stubs.cpp), and driven by the ABI and binding tests plus
valid calls of every entry point (tests/san_calls.py). Any out-of-bounds access, use of
freed memory, signed overflow, bad shift or misaligned access in that code aborts the
run."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libsigattn_san.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "sigmoid_attention_amd", "csrc", "sigattn.cpp"),
           os.path.join(ROOT, "tests", "host_san_stubs.cpp"), "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", SIGATTN_SANITIZED_STUBS="1")
    driver = (
        "import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "import sigmoid_attention_amd as S\n"
        "S._LIB_PATH = %r\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', %r, %r, %r]))\n"
    ) % (ROOT, os.path.join(ROOT, "tests"), str(lib), os.path.join(ROOT, "tests", "test_abi.py"),
         os.path.join(ROOT, "tests", "test_binding.py"), os.path.join(ROOT, "tests", "san_calls.py"))
    r = subprocess.run([sys.executable, "-c", driver], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "skipped" not in r.stdout.split("\n")[-2], tail
