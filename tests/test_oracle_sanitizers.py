"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_main.c links oracle.c into one program and calls every
entry point on small shapes (threads included); gcc builds it with both
sanitizers set to abort on the first report.  A clean exit means no
out-of-bounds access, use after free, leak or undefined behaviour on those
paths.  Host code only: nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "oracle_sanitize_main.c"), "-o", str(exe), "-lm", "-lpthread"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    assert build.returncode == 0, build.stderr[-2000:]
    # the environment is passed on as it is; ASan is told not to insist on
    # being first in the library order, since the process may preload others
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=240, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    assert "oracle sanitizer driver ok" in run.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
