"""The host side of the library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU): a
copy of libmla with the host code instrumented runs the C-ABI validation tests
(tests/test_host_abi.py: every entry point with null, misaligned and out-of-range arguments, the
workspace-size queries, the status strings) in a child process with the ASan runtime loaded
first.  Any memory error or undefined behaviour in the argument checks and size arithmetic ends
that process with a report, and this test fails."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_validation_paths_under_host_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or the ASan runtime is not installed")
    from mla_latent_kv_40_amd import build
    lib = build.build(host_sanitize=str(tmp_path / "libmla_san.so"))
    env = dict(os.environ, MLA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out
    assert r.returncode == 0
