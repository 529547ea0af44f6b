"""Build step of the HIP library: compiles csrc/ for gfx950 into librl_post_loss.so (in-tree)."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librl_post_loss.so")
SOURCES = ["loss_kernels_bf16.hip", "loss_kernels_f16.hip", "loss_kernels_f32.hip", "loss_kernels.hip",
           "vocab_kernels.hip", "logprob_kernels.hip", "abi.cpp"]
# Measurement helpers for bench.py (timing loops over the public entry points,
# reference kernels); linked against the loss library, found beside it.
BENCH_LIB = os.path.join(PKG, "librlpl_bench.so")
BENCH_SOURCES = ["bench_kernels.hip"]
# Object files of one build (not kept in the history).
OBJ_DIR = os.path.join(ROOT, "_build")


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
         # no packed-fp32 (v_pk_*_f32) instructions anywhere in the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("HIP build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r.stdout + r.stderr


def _objects(sources, csrc, obj_dir, verbose):
    """Compiles each source to an object, all at once (the policy-loss tables dominate)."""
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    for s in sources:
        obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [hipcc(), *FLAGS, "-I", INCLUDE, "-I", csrc, "-c", os.path.join(csrc, s), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o:
                print(o)
    return [j[0] for j in jobs]


def _link(objs, target, extra=()):
    _run([hipcc(), *FLAGS, "-shared", *objs, *extra, "-o", target + ".tmp"])
    os.replace(target + ".tmp", target)


def build(verbose: bool = False, csrc: str = CSRC, lib: str = LIB, bench_lib: str = BENCH_LIB) -> str:
    """Compile the library and the bench helpers (always; each result replaces any
    earlier build atomically)."""
    tag = os.path.basename(lib).replace(".so", "")
    objs = _objects(SOURCES, csrc, os.path.join(OBJ_DIR, tag), verbose)
    _link(objs, lib)
    bobjs = _objects(BENCH_SOURCES, csrc, os.path.join(OBJ_DIR, tag + "_bench"), verbose)
    libdir = os.path.dirname(lib)
    _link(bobjs, bench_lib, extra=("-L", libdir, "-l" + tag[3:], "-Wl,-rpath,$ORIGIN"))
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
