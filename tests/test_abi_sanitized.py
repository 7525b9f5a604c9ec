"""The host side of libcsa (argument checks, workspace sizing, dispatch)
under AddressSanitizer and UndefinedBehaviorSanitizer: a sanitized build
(host code instrumented, device code as usual) runs the CPU ABI tests in a
child process with the ASan runtime preloaded.  Any report fails the test
(UBSan does not recover)."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_abi_tests_under_asan_and_ubsan(tmp_path):
    from compressed_sparse_attention_compressor_amd import build

    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.fail("the ASan runtime of the ROCm clang is missing")
    lib = build.build_host_sanitized(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rts[-1], CSA_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_cpu.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout
