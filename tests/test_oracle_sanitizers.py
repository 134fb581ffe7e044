"""The CPU oracle under the host sanitizers: tests/native/oracle_sanitize_main.c
drives every filter kind and alphabet through oracle/sbf_oracle.c (edge
lengths, invalid bytes, threaded and sampled drivers, positions, the probe),
checks the Bloom property of the single-threaded insert and that the
threaded insert and query agree with it, and is built with gcc under
AddressSanitizer + UndefinedBehaviorSanitizer and, separately,
ThreadSanitizer.  Any report or failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "native", "oracle_sanitize_main.c")
ORACLE = os.path.join(ROOT, "oracle", "sbf_oracle.c")


@pytest.mark.parametrize("sanitizers", ["address,undefined", "thread"])
def test_oracle_under_sanitizer(tmp_path, sanitizers):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    flags = ["-fsanitize=" + sanitizers, "-fno-omit-frame-pointer"]
    if sanitizers != "thread":
        flags.append("-fno-sanitize-recover=all")
    build = subprocess.run(["gcc", "-O1", "-g", "-std=gnu99", "-pthread", "-Wall", "-Werror", *flags, "-o", exe,
                            DRIVER, ORACLE], capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot" in build.stderr:
        pytest.skip("this gcc cannot build with -fsanitize=%s" % sanitizers)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", TSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0 and "0 failures" in run.stdout, run.stdout[-2000:] + run.stderr[-4000:]
