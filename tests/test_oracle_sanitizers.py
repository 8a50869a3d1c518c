"""Host sanitizer build of the fp64 oracle (CPU only).

The oracle's C sources and tests/oracle_sanitize_driver.c are compiled with
gcc under AddressSanitizer and UndefinedBehaviorSanitizer (leak checks on),
and that C program exercises every option of the oracle's interface: packed
sequences with a zero-length one, NULL S0 / S_T / dS_T / dS0, a (sequence,
head) mask, decode run token by token against the forward (to 1e-12), and the
backward.  Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]


def _gcc():
    return shutil.which("gcc")


@pytest.mark.skipif(_gcc() is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "driver"
    srcs = [os.path.join(ROOT, "oracle", "gdr2_oracle.c"), os.path.join(ROOT, "oracle", "gdr2_oracle_bwd.c"),
            os.path.join(ROOT, "tests", "oracle_sanitize_driver.c")]
    r = subprocess.run([_gcc(), *FLAGS, *srcs, "-lm", "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("the sanitizer runtime is not available: " + r.stderr[:200])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    if run.returncode != 0 and "LeakSanitizer has encountered a fatal error" in run.stderr:
        # leak checking needs ptrace, which some containers forbid: run without it
        env["ASAN_OPTIONS"] = "detect_leaks=0"
        run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr
    assert "ok" in run.stdout
