"""The C ABI's host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of the library whose host API layer (argument validation,
planning, index maps) is instrumented, preloads the ASan runtime into a fresh
Python, and runs tests/test_boundary.py against that copy. Any sanitizer
report fails the test. No GPU is used: every boundary test stops on the host.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the sanitized library")
def test_boundary_tests_run_clean_under_asan_and_ubsan(tmp_path):
    from scan_primitives_amd import build_lib
    lib = build_lib.build_asan()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": build_lib.asan_runtime(),
        "ASAN_OPTIONS": f"detect_leaks=0:halt_on_error=1:log_path={tmp_path}/asan",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan",
        "SX_SCAN_LIB": lib,
    })
    proc = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_boundary.py"), "-q",
                           "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)
    reports = sorted(glob.glob(str(tmp_path / "asan*")) + glob.glob(str(tmp_path / "ubsan*")))
    text = "".join(open(r).read() for r in reports)
    assert not reports, f"sanitizer reports:\n{text[:4000]}"
    assert proc.returncode == 0, proc.stdout[-3000:] + proc.stderr[-3000:]
    assert " passed" in proc.stdout
