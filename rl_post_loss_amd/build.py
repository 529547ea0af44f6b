"""Build step of the HIP library: compiles csrc/ for gfx950 into librl_post_loss.so (in-tree)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librl_post_loss.so")
SOURCES = ["loss_kernels.hip", "vocab_kernels.hip", "logprob_kernels.hip", "abi.cpp"]
# Measurement helpers for bench.py (timing loops over the public entry points,
# reference kernels); linked against the loss library, found beside it.
BENCH_LIB = os.path.join(PKG, "librlpl_bench.so")
BENCH_SOURCES = ["bench_kernels.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def command(out: str, extra=(), sources=SOURCES) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-command-line-argument",
            # no packed-fp32 (v_pk_*_f32) instructions anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *extra,
            *[os.path.join(CSRC, s) for s in sources], "-o", out]


def _compile(cmd, target, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("HIP build failed:\n" + r.stdout + r.stderr)
    if verbose and (r.stdout or r.stderr):
        print(r.stdout + r.stderr)
    os.replace(target + ".tmp", target)


def build(verbose: bool = False) -> str:
    """Compile the library and the bench helpers (always; each result replaces any
    earlier build atomically)."""
    _compile(command(LIB + ".tmp"), LIB, verbose)
    _compile(command(BENCH_LIB + ".tmp", extra=("-L", PKG, "-lrl_post_loss", "-Wl,-rpath,$ORIGIN"),
                     sources=BENCH_SOURCES), BENCH_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
