"""The host planning code (validation, unit geometry, role split, workspace layout) under
AddressSanitizer and UndefinedBehaviorSanitizer: a C++ driver calls every planner on about a
million hand-picked and pseudo-random argument sets and checks the invariants the kernels rely on
for every plan it accepts.  Any overflow, out-of-bounds access or broken invariant aborts it.
CPU only."""
import shutil
import subprocess

import pytest


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planners_under_asan_and_ubsan():
    from communication_gemm_role_amd import build as B
    exe = B.build_host_plan_test()
    r = subprocess.run([exe, "200000"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300,
                       env={"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1",
                            "PATH": "/usr/bin:/bin"})
    assert r.returncode == 0, r.stdout[-4000:]
    assert r.stdout.strip().endswith("ok"), r.stdout[-2000:]
    calls, accepted = (int(x) for x in r.stdout.split()[0:4:3])
    assert calls > 1_000_000 and accepted > 100_000, r.stdout
