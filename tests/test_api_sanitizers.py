"""Host sanitizer build of the C ABI's host code (CPU only).

gdr2_api.cpp (argument validation, workspace layout, size queries, error
strings) is compiled with hipcc under AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only, linked with the library's
other objects into tests/api_sanitize_driver.cpp, and run: every entry point is
called with arguments it must reject before any device call, the size queries
with valid, invalid and extreme sizes, and the string functions.  Any
sanitizer report, or a status other than the documented one, fails the test.
No GPU is used: the fake device addresses are never dereferenced.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_sequence_gdr_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# device code is never instrumented: each sanitizer flag applies to the host pass only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SAN]
KERNEL_OBJECTS = ["gdr2_intra.hip.o", "gdr2_state.hip.o", "gdr2_decode.hip.o", "gdr2_schedule.hip.o",
                  "gdr2_epilogue.hip.o", "gdr2_bwd.hip.o"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
@pytest.mark.skipif(not all(os.path.exists(os.path.join(BUILD, o)) for o in KERNEL_OBJECTS),
                    reason="library objects not built (python -m linear_attention_sequence_gdr_amd.build)")
def test_api_host_code_under_asan_ubsan(tmp_path):
    objs = []
    for src, name in ((os.path.join(CSRC, "gdr2_api.cpp"), "api.o"),
                      (os.path.join(ROOT, "tests", "api_sanitize_driver.cpp"), "driver.o")):
        obj = str(tmp_path / name)
        r = subprocess.run([HIPCC, "-x", "hip", *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "driver")
    link = [HIPCC, "-fno-gpu-sanitize", "-fsanitize=address", "-fsanitize=undefined", *objs,
            *(os.path.join(BUILD, o) for o in KERNEL_OBJECTS), "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    if run.returncode != 0 and "LeakSanitizer has encountered a fatal error" in run.stderr:
        env["ASAN_OPTIONS"] = "detect_leaks=0"
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-3000:]
    assert run.stdout.strip().endswith("ok"), run.stdout[-3000:]
