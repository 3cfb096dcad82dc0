"""The host layer under AddressSanitizer.

libbrq_dryrun_asan.so is the dry-run build (validation, pass planning and
dispatch with an index walk in place of every launch) with the host code
instrumented by AddressSanitizer.  The whole dry-run test module runs against
it in a child process that loads the sanitizer runtime first; any heap or
stack overflow, use after free or double free in the host code aborts that
process with a report.  Leak checking is off: the interpreter itself is not
instrumented.
"""

import os
import subprocess
import sys

import pytest

import butterfly_rotation_quantization_amd as brq
from butterfly_rotation_quantization_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_dry_run_under_address_sanitizer():
    if not os.path.exists(B.DRYRUN_ASAN_LIB):
        B.build()
    rt = B.asan_runtime()
    assert rt, "no AddressSanitizer runtime found next to hipcc's clang"
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    env["BRQ_DRYRUN_LIB"] = B.DRYRUN_ASAN_LIB
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_dryrun.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stdout + r.stderr, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
