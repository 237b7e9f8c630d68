"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code
only) and driven through every function by oracle/sanitize_main.c, edge cases included:
no out-of-bounds access, leak or undefined operation.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           "-D_GNU_SOURCE", "-I", ORACLE, os.path.join(ORACLE, "oracle.c"),
           os.path.join(ORACLE, "sanitize_main.c"), "-o", exe, "-lm"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and "asan" in (b.stderr or "").lower() and "cannot find" in b.stderr:
        pytest.skip("the sanitizer runtime is not installed")
    assert b.returncode == 0, b.stderr
    # (other libraries preloaded into every process may precede the sanitizer runtime)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer run ok" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr
