"""The host-side argument validation under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with ASan and UBSan on its host code (device code as
usual), and the ABI tests (tests/test_abi.py: every rejection path, no GPU) run
against it in a child process with the ASan runtime preloaded.  Any
out-of-bounds access, use after free or undefined behaviour in the validation
layer aborts the child and fails this test.
"""
import os
import subprocess
import sys

import pytest

from protein_pair_representation_amd import build as b

HERE = os.path.dirname(os.path.abspath(__file__))
ASAN_LIB = os.path.join(os.path.dirname(b.LIB_PATH), "libtriattn_asan.so")
# every sanitizer flag goes to the host pass only; the device code is built as usual
HOST_ONLY = [f for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                            "-fno-omit-frame-pointer", "-g") for f in ("-Xarch_host", flag)]


def asan_runtime() -> str:
    """The clang ASan runtime, preloaded into the (uninstrumented) python of the child."""
    for clang in (os.path.join(os.path.dirname(os.path.realpath(b.hipcc())), "..", "lib", "llvm", "bin", "clang"),
                  "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(clang):
            path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                                  text=True).stdout.strip()
            if path and os.path.exists(path):
                return path
    raise RuntimeError("clang ASan runtime not found")


@pytest.mark.timeout(900)
def test_abi_under_asan_ubsan():
    lib = b.build(out=ASAN_LIB, extra_flags=HOST_ONLY)
    assert "__asan_report" in subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    env = dict(os.environ, TRIATTN_LIB=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")], cwd=os.path.dirname(HERE), env=env,
                       capture_output=True, text=True, timeout=800)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
