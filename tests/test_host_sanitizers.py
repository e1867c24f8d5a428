"""Host sanitizer run (CPU only): the C oracle and librehyat's host code (argument
validation, workspace and state layouts, launch setup; the device code is unchanged) built
with AddressSanitizer and UndefinedBehaviorSanitizer, and the oracle and C-ABI test files
run in a child process that preloads the sanitizer runtime.  Any report fails the run
(no recovery; leaks are not checked, the interpreter itself holds memory to its end)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.mark.skipif(not RUNTIME, reason="clang sanitizer runtime not installed")
def test_oracle_and_api_tests_run_clean_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    import oracle
    from hybrid_softmax_linear_chunked_amd.build import SAN_DIR, build_sanitized

    lib = build_sanitized()
    olib = oracle.build_sanitized(SAN_DIR)
    env = dict(os.environ)
    env.update(LD_PRELOAD=RUNTIME[-1], REHYAT_LIB=lib, REHYAT_ORACLE_LIB=olib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child really runs the sanitized builds
    probe = ("import oracle, hybrid_softmax_linear_chunked_amd as rh; rh.lib(); oracle.lib(); "
             "print(open('/proc/self/maps').read())")
    maps = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=300).stdout
    for name in ("librehyat_san.so", "librehyat_oracle_san.so", "libclang_rt.asan"):
        assert name in maps, name
    files = ["tests/test_api.py", "tests/test_oracle.py", "tests/test_oracle_backward.py",
             "tests/test_oracle_distill.py", "tests/test_oracle_distill_grad.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
