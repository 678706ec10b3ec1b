"""The host side of the library (argument validation, workspace planning, status strings)
under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: a build of the same
sources with the sanitizers on the host code only (the device code is built as usual),
loaded by the C-ABI tests in a child process with the ASan runtime preloaded."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address,undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.slow
def test_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this ROCm install")
    from rejection_sampling_verify_specdec_amd import build
    lib = build.build(extra=SAN_FLAGS, out=str(tmp_path / "libspecdec_san.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, SPECDEC_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert "passed" in out
