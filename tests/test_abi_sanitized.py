"""The C ABI's host validation under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

seed_api.cpp (every argument check, the thread-local error text, the
status strings) is built with g++ -fsanitize=address,undefined together
with host-only stand-ins for the device launchers (tests/sanitize/
stub_launch.cpp), and tests/test_abi.py runs against that library in a
child process with the sanitizer runtime preloaded.  Any out-of-bounds
access, use after free, signed overflow, misaligned access or other
undefined behaviour in the validation code fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"


def _gcc_lib(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or _gcc_lib("libasan.so") is None
                    or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")),
                    reason="needs g++ with AddressSanitizer and the HIP headers")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libseed_host_sanitized.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "sink_rank_recurrent_amd", "csrc"),
           os.path.join(ROOT, "sink_rank_recurrent_amd", "csrc", "seed_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, SEED_LIBRARY=lib, LD_PRELOAD=_gcc_lib("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    probe = subprocess.run([sys.executable, "-c", "from sink_rank_recurrent_amd import binding; "
                            "print(binding.lib()._name, binding.lib().seed_abi_version())"],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.split()[0] == lib, probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
