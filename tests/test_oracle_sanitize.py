"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and driven through every entry point on small boxes
with solids, walls, open faces of every kind and one-cell axes: the run must
finish cleanly.  Skipped where the compiler lacks the sanitizer runtimes."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_is_clean_under_sanitizers():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitize")
        flags = ["-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off",
                 "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
        cmd = [gcc, *flags, "-o", exe, os.path.join(HERE, "oracle_sanitize_driver.c"),
               os.path.join(ROOT, "oracle", "lbm_oracle.c"), "-lm"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0 and "asan" in (r.stderr or "").lower():
            pytest.skip("sanitizer runtime not available: " + r.stderr[-200:])
        assert r.returncode == 0, r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert run.returncode == 0 and run.stdout.strip() == "ok", (run.stdout, run.stderr[-2000:])
