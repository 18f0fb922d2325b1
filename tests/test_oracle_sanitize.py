"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, host code only), driven over random tiny batches through every entry
point by tests/oracle_sanitize.cpp: any invalid access, leak or undefined
operation, or a violated invariant, fails the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_address_and_undefined_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitize")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               os.path.join(HERE, "oracle_sanitize.cpp"), os.path.join(ROOT, "oracle", "oracle.cpp"),
               "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
        # verify_asan_link_order=0: the environment may preload other libraries
        env = dict(os.environ,
                   ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, r.stderr[-4000:]
        assert r.stdout.strip() == "ok"
