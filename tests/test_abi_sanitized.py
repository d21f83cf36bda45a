"""The C ABI's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no kernel runs): m2ssd_api.cpp is
rebuilt with host ASan/UBSan (mamba_ssd_selective_amd.build.build_host_sanitized)
and tests/test_abi_host.py runs against that library in a child process with
clang's ASan runtime preloaded.  Any invalid access or undefined behaviour on
those paths aborts the child."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the sanitized library")
def test_abi_host_checks_under_asan_and_ubsan():
    from mamba_ssd_selective_amd import build as B
    lib = B.build_host_sanitized()
    env = dict(os.environ)
    env.update(M2SSD_LIB=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, pytest, mamba_ssd_selective_amd as m2; "
            "rc = pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi_host.py']); "
            "print('loaded', m2.LIB_PATH); sys.exit(rc)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    assert f"loaded {lib}" in out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
