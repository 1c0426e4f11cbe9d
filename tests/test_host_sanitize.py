"""Host sanitizers over the oracle: tests/host_sanitize/oracle_driver.c
compiles oracle/oracle.c into one translation unit with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, no OpenMP) and runs every oracle entry
point on small inputs that reach its edge cases; any out-of-bounds access,
use after free, leak or undefined behaviour aborts the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", os.path.join(HERE, "host_sanitize", "oracle_driver.c"), "-o", exe,
                    "-lm"], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "oracle driver: ok" in r.stdout
