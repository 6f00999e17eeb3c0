"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (g++ -fsanitize=address,undefined) runs its pin tests, and the
library's host side (hipcc with the sanitizers on the host code only) runs
the no-GPU library checks -- argument checks, workspace sizes, the plan --
each in a child process with the matching ASan runtime preloaded.  Any
sanitizer report aborts the child, which fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def _runtime(compiler, name):
    path = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not path or not os.path.exists(path):
        pytest.skip(f"{name} not found for {compiler}")
    return path


def _run_child(tests, extra_env):
    env = dict(os.environ)
    env.update(extra_env)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]


def test_oracle_under_asan_and_ubsan():
    import oracle
    lib = oracle.build(force=False, sanitize=True)
    tests = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py"))
    _run_child(tests, {"HTL_ORACLE_LIB": lib, "LD_PRELOAD": _runtime("gcc", "libasan.so")})


def test_library_host_code_under_asan_and_ubsan():
    from hash_table_lookup_amd import build as hb
    src = [os.path.join(hb.CSRC, f) for f in os.listdir(hb.CSRC)] + [os.path.join(ROOT, "include", "htl.h")]
    if not os.path.exists(hb.SAN_LIB_PATH) or os.path.getmtime(hb.SAN_LIB_PATH) < max(map(os.path.getmtime, src)):
        hb.build(verbose=False, sanitize=True)
    rt = "/opt/rocm/llvm/lib/clang"
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        pytest.skip("no ROCm clang for the ASan runtime")
    _run_child([os.path.join("tests", "test_library.py")],
               {"HTL_LIB": hb.SAN_LIB_PATH, "LD_PRELOAD": _runtime(clang, "libclang_rt.asan-x86_64.so")})
