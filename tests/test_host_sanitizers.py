"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

libpmx_san.so is the same library with its host-logic translation units
(argument validation, workspace carving, alias checks, the Shampoo plan's
tables) compiled with -fsanitize=address,undefined on their host pass only
(preconditioned_optimizer_matrix_amd/build.py, --sanitize).  The CPU ABI tests
run against it in a child process with the clang ASan runtime preloaded; any
sanitizer report fails the run (UBSan halts on the first error).
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_clean_under_host_sanitizers():
    from preconditioned_optimizer_matrix_amd import build
    srcs = [os.path.join(build.CSRC, f) for f in build.SAN_SOURCES] + [
        os.path.join(ROOT, "include", "pmx.h")]
    if (not os.path.exists(build.SAN_LIB)
            or os.path.getmtime(build.SAN_LIB) < max(os.path.getmtime(s) for s in srcs)):
        build.build_sanitized(verbose=False)
    env = dict(os.environ)
    env.update(PMX_LIBRARY=build.SAN_LIB, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
