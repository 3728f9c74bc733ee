"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/sanitize_oracle_driver.c calls every entry point of oracle/vbq_oracle.c
on small random shapes (one and several k-tiles, a scale-0 group, row subsets,
fp16 and bf16 x, residuals, an infinite residual) and checks its round trips;
built here with gcc and the sanitizers, any out-of-bounds access, leak or
undefined operation fails the run.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
           os.path.join(HERE, "sanitize_oracle_driver.c"), os.path.join(ROOT, "oracle", "vbq_oracle.c"), "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "oracle clean under the sanitizers" in run.stdout
