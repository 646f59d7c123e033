"""The C ABI's host code under AddressSanitizer (no GPU needed): api.cpp is rebuilt with ASan on
its host side only (the device code is the release code), and the host-side contract tests of
test_abi_cpu.py run against that build in a child process with the ASan runtime preloaded. Any
out-of-bounds access or use-after-free in argument validation, workspace carving or the entry
points' early returns makes ASan end the child with a report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

build = pytest.importorskip("gated_mla_kv_amd.build")


def test_abi_host_code_under_asan():
    try:
        lib = build.build_asan()
        runtime = build.asan_runtime()
    except RuntimeError as e:  # no hipcc or no ASan runtime on this host
        pytest.skip(str(e))
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    if out.returncode == 0:  # the library really is instrumented
        assert "__asan_report" in out.stdout
    env = dict(os.environ, LD_PRELOAD=runtime, GMLA_LIB=lib, PYTHONPATH=ROOT,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=66")
    env.pop("GMLA_LOG", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
