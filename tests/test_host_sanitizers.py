"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU code built).

kvq_api.cpp and kvq_stream.cpp (argument checks, layouts, retention, stream
bookkeeping, workspace sizing) are built with g++ -fsanitize=address,undefined into
a host-only library whose device launches are stubs (tests/sanitize), and the host
test files run against it in a child process with the ASan runtime preloaded.  Any
sanitizer report stops the child and fails this test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_decode_attention_kv_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_TESTS = ["tests/test_abi_host.py", "tests/test_stream_host.py"]


def _runtime(name):
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    path = subprocess.run([gcc, "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    gxx, asan = shutil.which("g++"), _runtime("libasan.so")
    if not gxx or not asan or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++, libasan or the HIP headers are missing")
    out = str(tmp_path_factory.mktemp("asan") / "libkvq_host_asan.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(CSRC, "kvq_api.cpp"), os.path.join(CSRC, "kvq_stream.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out, asan


def test_host_tests_clean_under_asan_and_ubsan(sanitized_lib):
    lib, asan = sanitized_lib
    env = dict(os.environ)
    env.update(KVQ_LIBRARY=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *HOST_TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-6000:]
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
