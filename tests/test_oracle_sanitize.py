"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a
driver (tests/c/oracle_sanitize.c) compiles the oracle's source into itself
and calls every entry point on small ragged, strided, grouped inputs; any
out-of-bounds access, use of freed memory or undefined operation aborts the
run.  Built without OpenMP so the sanitizers see every loop in one thread."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_is_clean_under_address_and_ub_sanitizers():
    src = os.path.join(HERE, "c", "oracle_sanitize.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitize")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                        "-Wno-unknown-pragmas", "-o", exe, src, "-lm"], check=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok"), r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
