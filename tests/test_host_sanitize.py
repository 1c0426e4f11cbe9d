"""Host sanitizers (AddressSanitizer and UndefinedBehaviorSanitizer, CPU
only).  tests/host_sanitize/oracle_driver.c compiles oracle/oracle.c into one
translation unit (gcc, no OpenMP) and runs every oracle entry point on small
inputs that reach its edge cases; tests/host_sanitize/abi_driver.c runs the
C-ABI's host validation and workspace-size code built with the sanitizers.
Any out-of-bounds access, use after free, leak, integer overflow or other
undefined behaviour aborts the driver."""
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


ROOT = os.path.dirname(HERE)
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    """The library's host code (validation, plans, workspace sizes) built with
    host AddressSanitizer and UndefinedBehaviorSanitizer, linked into
    tests/host_sanitize/abi_driver.c: every entry point refuses invalid
    arguments with its documented code before any launch (no GPU needed),
    and the workspace-size functions take extreme shapes without overflow."""
    csrc = os.path.join(ROOT, "compressed_sparse_attention_c4a_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".cpp")):
            continue
        obj = str(tmp_path / (f + ".o"))
        dev = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] \
            if f.endswith(".hip") else []
        cmd = [HIPCC, "-std=c++17", "-O1", "-g", "-fPIC"] + dev + SAN + inc + ["-c", os.path.join(csrc, f), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out[-3000:]
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([HIPCC] + SAN + ["-x", "c", os.path.join(HERE, "host_sanitize", "abi_driver.c"), "-x", "none"]
                       + objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "abi driver: ok" in r.stdout
