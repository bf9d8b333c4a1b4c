"""The host C of this repository (oracle/oracle.c, testgen/testgen.c) built
with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, CPU only) and run
through tests/sanitize_driver.c: any out-of-bounds access, leak or undefined
behaviour aborts the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_host_c_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
           os.path.join(HERE, "sanitize_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "testgen", "testgen.c"), "-lm", "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("the sanitizer runtimes are not installed: %s" % r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "0 failing cases" in run.stdout
