"""The CPU oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

* The oracle's C source with a driver (sanitize/oracle_harness.c) that calls
  every oracle entry point over seeded small problems and edge cases, each
  buffer at its exact size (gcc, -fsanitize=address,undefined).
* The library's host code (abi.cpp: validation, launch planning) with a driver
  (sanitize/abi_harness.cpp) that calls every entry point of the C header with
  rejected and extreme arguments, and the planning helpers over wide ranges;
  built host-only (no device code in this build: the kernel tables come from
  the built library it links against), sanitizers on the host pass only.

Leak detection is on.  A planted out-of-bounds read, built the same way, must
be reported, so that a clean run means the instrumentation was there.
Nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

import rl_post_loss_amd as rl
from rl_post_loss_amd import build as rl_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_C = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
# hipcc: every sanitizer option on the host pass only
SAN_HIP = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    return r.returncode, r.stdout + r.stderr


def need(tool):
    path = shutil.which(tool) or ("/opt/rocm/bin/" + tool if tool == "hipcc" else None)
    if not path or not os.path.exists(path):
        pytest.skip(f"{tool} not available")
    return path


def test_instrumentation_reports_a_planted_overflow(tmp_path):
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint main(int c, char** v) { int* p = malloc(4 * sizeof(int));\n"
                   "  int x = p[c + 3]; free(p); return x == 12345; }\n")
    exe = tmp_path / "planted"
    rc, out = run([need("gcc"), "-O0", "-g", *SAN_C, str(src), "-o", str(exe)])
    assert rc == 0, out
    rc, out = run([str(exe)], env=ENV)
    assert rc != 0 and "heap-buffer-overflow" in out


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_harness"
    rc, out = run([need("gcc"), "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", *SAN_C,
                   os.path.join(ROOT, "oracle", "rlpl_oracle.c"), os.path.join(HERE, "oracle_harness.c"),
                   "-lm", "-o", str(exe)])
    assert rc == 0, out
    rc, out = run([str(exe)], env=ENV)
    assert rc == 0 and out.startswith("ok "), out


def test_host_abi_under_sanitizers(tmp_path):
    hipcc = need("hipcc")
    lib = rl.library_path()
    if not os.path.exists(lib):
        rl_build.build()
    exe = tmp_path / "abi_harness"
    rc, out = run([hipcc, "--offload-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *SAN_HIP,
                   "-I", os.path.join(ROOT, "include"), "-I", rl_build.CSRC,
                   os.path.join(rl_build.CSRC, "abi.cpp"), os.path.join(HERE, "abi_harness.cpp"),
                   "-L", os.path.dirname(lib), "-lrl_post_loss", "-Wl,-rpath," + os.path.dirname(lib),
                   "-o", str(exe)])
    assert rc == 0, out
    # No GPU is used: hide any that the machine has, so that every valid call
    # stops at the device lookup.
    env = dict(ENV, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    rc, out = run([str(exe)], env=env)
    assert rc == 0 and out.startswith("ok "), out
