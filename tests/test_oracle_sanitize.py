"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a
small C driver (oracle_sanitize_main.c) calls every oracle routine -- grid
orders, pooling, selection, forward and backward with every flag, partial
row sets, transpose -- and any invalid access, leak or undefined operation
aborts it."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-I", os.path.join(ROOT, "oracle"), os.path.join(HERE, "oracle_sanitize_main.c"),
         os.path.join(ROOT, "oracle", "llsa_oracle.c"), "-lm", "-o", exe],
        capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "oracle sanitize run ok" in run.stdout
