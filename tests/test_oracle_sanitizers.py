"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize_oracle_driver.c calls every oracle entry point on small shapes and the edge cases
its definitions name, with every buffer allocated at exactly its documented size; built here
together with oracle/qspec_oracle.c with gcc -fsanitize=address,undefined (host code only) and run
as a separate process, so any out-of-bounds access, leak or undefined operation fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "qspec_oracle.c"), os.path.join(ROOT, "tests", "sanitize_oracle_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer driver: done" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr
