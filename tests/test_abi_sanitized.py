"""The host-side argument checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: a host-only sanitized build of the library
(``pixel_space_flow_amd/build.py host-asan``) runs every case of test_abi_host.py in a child
process with the ASan runtime preloaded.  Any sanitizer report fails the test.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "pixel_space_flow_amd"))


def test_abi_host_checks_under_asan_and_ubsan():
    import build as B
    lib = B.build_host_sanitized(verbose=False)
    clang = "/opt/rocm/llvm/bin/clang++"
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("clang's ASan runtime is not installed")
    env = dict(os.environ, PSF_GEN_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out
    assert r.returncode == 0
    assert " passed" in out
