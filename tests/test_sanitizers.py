"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

Rebuilds the oracle and libsas.so's host side with the sanitizers
(tests/sanitize_build.py) and runs tests/test_oracle.py and tests/test_abi.py
against those builds in a child process with the sanitizer runtime
preloaded: every oracle entry point on small inputs, every argument check and
size query of the C ABI.  Any report (heap or stack overflow, use after
free, undefined behaviour) aborts the child and fails this test.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.timeout(900)
def test_oracle_and_abi_under_sanitizers(tmp_path):
    import sanitize_build as sb
    try:
        rt = sb.runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    oracle_lib = sb.build_oracle()
    sas_lib = sb.build_library()
    log = str(tmp_path / "san")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, SAS_LIBRARY=sas_lib, SAS_ORACLE_LIB=oracle_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:log_path=" + log,
               UBSAN_OPTIONS="print_stacktrace=1:log_path=" + log)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(HERE, "test_abi.py"),
                        os.path.join(HERE, "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    reports = sorted(glob.glob(log + "*"))
    text = "".join(open(p).read()[:4000] for p in reports)
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-3000:] + text)
