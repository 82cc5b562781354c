"""The host ABI checks again, against a build of the library whose host code
carries AddressSanitizer and UndefinedBehaviorSanitizer (argument checks,
launch planning and set-up; device code built as usual, and no kernel is
launched here).  The sanitizer runtime is preloaded into a child Python;
any report fails the run."""

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(_asan_runtime() is None, reason="no clang AddressSanitizer runtime found")
def test_host_abi_checks_under_address_and_ub_sanitizers():
    from sparse_moe_layer_03_amd import build as Bld
    d = tempfile.mkdtemp(prefix="moe_san_")
    lib = Bld.build(sanitize_out=os.path.join(d, "libmoe_san.so"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "not instrumented"
    env = dict(os.environ, MOE_MI355X_LIB=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert " passed" in out
