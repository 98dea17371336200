"""The C-ABI's host code (argument validation, work plans, workspace layout)
under AddressSanitizer: the ABI tests run again, in a child process, against
a build of the library whose host pass is instrumented, and must pass with no
sanitizer report.  CPU only: every call in those tests returns before any HIP
call."""

import os
import subprocess
import sys

from recommender_ultra_long_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_pass_under_host_address_sanitizer():
    lib = build.build_host_asan()
    env = dict(os.environ)
    env.update(LD_PRELOAD=build.asan_runtime(), SA_LIBRARY_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86",
               PYTHONPATH=ROOT + os.pathsep + env.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
