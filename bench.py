#!/usr/bin/env python3
"""Throughput of the fused PPO-family policy loss on one MI355X.

Default step = one fused forward+backward BNPO call (bs=64, seq_len=4096,
bf16 log-probs, int8 prefix mask with lengths U[256, 4096], beta=0.04,
eps=0.2, eps_high=0.28): the whole hot path (stream-in, per-token policy and
KL terms, local reduction, on-GPU global count, 1/N scaling, gradient store,
loss finalise) in one launch through the C ABI.

Inputs are generated once, copied into rotating sets totalling >= 1 GiB (so
each step reads from HBM rather than the 256 MB last-level cache) and are
resident before timing starts.  W warmup steps, then exactly K timed steps
between two stream synchronisations; the steps are issued by a C loop over
the public entry point (librlpl_bench.so), one call per step, so that the
interpreter's per-call cost does not set the pace.  HIP events recorded on
the launch stream at both ends of the timed region give the per-launch
kernel duration (span / K) used for the roofline: back-to-back launches keep
the GPU busy, so this agrees with rocprofv3's kernel durations.  `value`
counts every (row, position) slot of the batch per step (the mask is read
and the gradient written for all of them); the valid (completion) tokens per
second are reported beside it.

Options for context measurements (never the headline line's workload):
  --op bnpo|bnpo_fwd|grpo|grpo_fwd|rkl|rkl_fwd   another entry point
  --bs / --seq-len                               another size (inputs drawn on
                                                 the device above 2^24 slots)
  --copy-mib M [--copy-variant V] [--copy-grid G]
                                                 a streaming copy of M MiB by
                                                 every variant (or variant V,
                                                 grid G) of our own 128-bit
                                                 copy kernel, the best of them
                                                 the ceiling, and by the
                                                 runtime's copy (also the
                                                 reference for the traffic
                                                 counters)
  --read-mib M                                   a streaming read of M MiB
                                                 (the forward-only ceiling)
  --op rkl_logits|rkl_logits_fwd [--rows R --vocab V]
                                                 full-vocab reverse KL over
                                                 (R, V) logit slabs (default the
                                                 card's example, 1024 x 248320
                                                 bf16, rows valid with p = 0.8)
  --op logprob|logprob_fwd [--rows N --hidden H --vocab V]
                                                 selective log-probabilities from
                                                 hidden states and the output
                                                 projection on the matrix cores
                                                 (default one 1024-token group,
                                                 H = 4096, V = 128256, bf16)
  --op grpo_chain [--bs B]                       the chain policy + reference
                                                 log-probs -> GRPO loss -> backward
                                                 into the policy's hidden states,
                                                 projection and bias (B sequences
                                                 of 1024 tokens, default 1)
  --floor                                        back-to-back launches of an
                                                 empty kernel with the launch
                                                 shape of the workload (the
                                                 per-launch floor)
  --rotate-gib 0                                 two input sets only, which stay
                                                 in the last-level cache (a
                                                 warm-cache figure)

The CPU baseline is the oracle (double precision C) over the same host-side
batch, the batch's rows split over every host core (one oracle call per row
range, in parallel threads; ctypes releases the GIL) and the ranges' sums
combined into the batch's loss and gradient: 3 warmup steps, then the median
of at least 10 steps.  Beside it: one whole batch on one thread, and whole
batches on every core at once (throughput of independent batches).

Prints one JSON line.  --gpus above 1 is not supported.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix-core peak
METRIC = "tokens/s and achieved HBM GB/s (% of peak) for fused loss fwd+bwd"


def algorithmic_bytes(op: str, slots: int, valid: int, bs: int, elem: int, has_kl: bool, fused: bool) -> int:
    """Bytes the method must move: the mask and (fused) the dense gradient for every slot;
    the input planes only for valid tokens; the advantages and the 4-byte loss."""
    planes = 2 if op.startswith("rkl") else (3 if has_kl else 2)
    b = slots * 1 + valid * planes * elem + 4
    if fused:
        b += slots * elem
    if not op.startswith("rkl"):
        b += bs * elem
    return b


# The sources the per-token loss kernels and their launch are built from (the
# full-vocab and log-prob kernels live in files of their own).
LOSS_KERNEL_SOURCES = ("abi.cpp", "device_common.h", "loss_kernels.h", "loss_kernels.hip", "loss_kernels_impl.h",
                       "loss_kernels_bf16.hip", "loss_kernels_f16.hip", "loss_kernels_f32.hip", "row_divisor.h")


def kernel_source_hash() -> str:
    """sha256 over the per-token loss kernel sources (sorted; each file's name, then its bytes)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(LOSS_KERNEL_SOURCES):
        h.update(name.encode())
        with open(os.path.join(ROOT, "rl_post_loss_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per launch (read + written) recorded from rocprofv3 counters for this
    workload, or None when none is recorded for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = kernel_source_hash()
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 4 and not line.startswith("#") and parts[0] == workload and parts[1] == digest:
                return int(parts[2]) + int(parts[3])
    return None


def timed(fn, calls, K, W, stream, torch):
    """W warmup calls, then K timed back-to-back calls from Python (long kernels only);
    returns (ms per step wall, ms per launch GPU)."""
    n = len(calls)
    for i in range(W):
        rc = fn(*calls[i % n])
        if rc != 0:
            raise RuntimeError(f"{getattr(fn, '__name__', 'call')} returned status {rc}")
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bad = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        bad |= fn(*calls[(W + i) % n])
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if bad:
        raise RuntimeError("a timed call returned an error status")
    return (t1 - t0) * 1e3 / K, ev0.elapsed_time(ev1) / K


def timed_loop(run, K, W, stream, torch):
    """run(first, iters) enqueues `iters` steps from rotating index `first` with one C call
    (returns a status).  W untimed steps, then exactly K timed steps between two
    synchronisations; returns (ms per step wall, ms per launch GPU from HIP events)."""
    if W:
        rc = run(0, W)
        if rc != 0:
            raise RuntimeError(f"warmup returned status {rc}")
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    rc = run(W, K)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if rc != 0:
        raise RuntimeError(f"a timed step returned status {rc}")
    return (t1 - t0) * 1e3 / K, ev0.elapsed_time(ev1) / K


def bench_lib():
    """The measurement helpers (librlpl_bench.so, beside the loss library)."""
    import ctypes
    import rl_post_loss_amd as rl
    from rl_post_loss_amd import build as b
    rl.library()
    if not os.path.exists(b.BENCH_LIB):
        b.build()
    lib = ctypes.CDLL(b.BENCH_LIB)
    vp, i32, i64, f32, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_uint64
    sz, u32 = ctypes.c_size_t, ctypes.c_uint32
    lib.rlpl_bench_empty.argtypes = [i32, i32, vp]
    lib.rlpl_bench_copy.argtypes = [i32, vp, u64, i32, i32, i32, i32, vp]
    lib.rlpl_bench_read.argtypes = [i32, vp, u64, i32, i32, vp, i32, i32, vp]
    lib.rlpl_bench_policy.argtypes = [i32, u32, i32, vp, i64, i64, i32, i32, f32, f32, f32, vp, sz, i32, i32, vp]
    lib.rlpl_bench_rkl.argtypes = [i32, i32, vp, i64, i64, i32, i32, vp, sz, i32, i32, vp]
    lib.rlpl_bench_noalloc.argtypes = [i32, vp, i64, i64, i32, i32, f32, f32, f32, i32, i32, vp]
    for f in (lib.rlpl_bench_empty, lib.rlpl_bench_copy, lib.rlpl_bench_read, lib.rlpl_bench_policy,
              lib.rlpl_bench_rkl, lib.rlpl_bench_noalloc):
        f.restype = ctypes.c_int
    return lib


def pointer_table(rows):
    """A contiguous uint64 array of device pointers (rows x columns) for the C loops."""
    import numpy as np
    return np.ascontiguousarray(np.array(rows, dtype=np.uint64))


COPY_VARIANTS = {0: "grid-stride x4", 1: "grid-stride x4 nt", 2: "grid-stride x8", 3: "grid-stride x8 nt",
                 4: "chunked x4", 5: "chunked x4 nt", 6: "chunked x8", 7: "chunked x8 nt"}


def copy_ceiling(args, torch):
    """Streaming copies of M MiB on rotating buffers (>= 1 GiB in all): every variant of our
    own 128-bit copy kernel at several grids (the best is the ceiling), and the runtime's copy
    for comparison."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lib = bench_lib()
    nbytes = int(args.copy_mib * (1 << 20)) // 16 * 16
    nsets = max(2, math.ceil((1 << 30) / (2 * nbytes)))
    pairs = [(torch.empty(nbytes, dtype=torch.uint8, device=dev),
              torch.empty(nbytes, dtype=torch.uint8, device=dev)) for _ in range(nsets)]
    table = pointer_table([[d.data_ptr(), s.data_ptr()] for s, d in pairs])
    out = {"metric": "streaming copy (read + write) of the same bytes", "bytes_read": nbytes,
           "bytes_written": nbytes, "steps": args.steps, "rotating_sets": nsets, "own_kernel": {}}
    best = None
    variants = COPY_VARIANTS if args.copy_variant is None else {args.copy_variant: COPY_VARIANTS[args.copy_variant]}
    grids = (1024, 2048, 4096, 8192) if args.copy_grid is None else (args.copy_grid,)
    for variant, name in variants.items():
        for grid in grids:
            _, ms = timed_loop(lambda first, k: lib.rlpl_bench_copy(nsets, table.ctypes.data, nbytes, grid, variant,
                                                                     k, first, stream.cuda_stream),
                               args.steps, args.warmup, stream, torch)
            gbs = 2 * nbytes / (ms * 1e-3) / 1e9
            out["own_kernel"][f"{name} grid {grid}"] = round(gbs, 1)
            if best is None or gbs > best[0]:
                best = (gbs, ms, f"{name} grid {grid}")
    out["own_kernel_best"] = {"variant": best[2], "us_per_launch": round(best[1] * 1e3, 3), "GBs": round(best[0], 1),
                              "frac_of_peak": round(best[0] / PEAK_HBM_GBS, 4)}

    def fn(d, s):
        d.copy_(s)
        return 0
    _, ms = timed(fn, [(d, s) for s, d in pairs], args.steps, args.warmup, stream, torch)
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    out["runtime_copy"] = {"us_per_launch": round(ms * 1e3, 3), "GBs": round(gbs, 1),
                           "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    print(json.dumps(out), flush=True)
    return 0


def read_ceiling(args, torch):
    """Streaming reads of M MiB (our own 128-bit kernel, plain and non-temporal)."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lib = bench_lib()
    nbytes = int(args.read_mib * (1 << 20)) // 16 * 16
    nsets = max(2, math.ceil((1 << 30) / nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nsets)]
    table = pointer_table([b.data_ptr() for b in bufs])
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    out = {"metric": "streaming read of the same bytes", "bytes_read": nbytes, "steps": args.steps,
           "rotating_sets": nsets}
    for nt in (0, 1):
        _, ms = timed_loop(lambda first, k: lib.rlpl_bench_read(nsets, table.ctypes.data, nbytes, 0, nt,
                                                                 sink.data_ptr(), k, first, stream.cuda_stream),
                           args.steps, args.warmup, stream, torch)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["own_kernel_nt" if nt else "own_kernel"] = {"us_per_launch": round(ms * 1e3, 3), "GBs": round(gbs, 1),
                                                        "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    print(json.dumps(out), flush=True)
    return 0


def launch_floor(args, torch):
    """Back-to-back launches of an empty kernel with the workload's grid (x 256 threads)."""
    import rl_post_loss_amd as rl
    import synthetic
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lib = bench_lib()
    w = synthetic.WORKLOADS[args.workload]
    grid, vec, tiles = rl.launch_shape(args.bs or w.bs, args.seq_len or w.seq_len, synthetic.DTYPES[w.dtype],
                                       args.op or w.op)
    ms_wall, ms_gpu = timed_loop(lambda first, k: lib.rlpl_bench_empty(grid, k, stream.cuda_stream), args.steps,
                                 args.warmup, stream, torch)
    print(json.dumps({"metric": "per-launch floor: empty kernel, back to back",
                      "grid": grid, "threads_per_workgroup": 256,
                      "us_per_launch": round(ms_gpu * 1e3, 3), "us_per_step_wall": round(ms_wall * 1e3, 3),
                      "steps": args.steps}), flush=True)
    return 0


def cpu_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(env))) if env.isdigit() else n


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rate(run_once, seconds: float, threads: int):
    """Batches per second of run_once() with `threads` threads each running whole batches."""
    import threading
    counts = [0] * threads
    stop = time.perf_counter() + seconds

    def worker(i):
        while True:
            run_once()
            counts[i] += 1
            if time.perf_counter() >= stop:
                break
    t0 = time.perf_counter()
    ts = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return sum(counts) / (time.perf_counter() - t0), sum(counts)


def oracle_rows_step(op, x, w, fused, threads):
    """One batch of the oracle (double precision C), its rows split into `threads`
    contiguous ranges computed in parallel (one oracle call per range; ctypes releases
    the GIL), then combined into the batch's loss and gradient: for the global-mean
    losses each range's sum is loss_c * max(n_c, 1) and its gradient is rescaled by
    max(n_c, 1) / max(N, 1) (reverse-KL: n_c / N, unclamped); for GRPO, whose rows are
    independent, by rows_c / bs.  Returns step() -> (loss, grad, N) and the range count."""
    import ctypes
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    lib = oracle._load()
    is_rkl = op.startswith("rkl")
    if is_rkl:
        lp, rf = oracle.to_f64(x["student"]), oracle.to_f64(x["teacher"])
        od = adv = None
    else:
        lp, od = oracle.to_f64(x["policy"]), oracle.to_f64(x["old"])
        rf = oracle.to_f64(x["ref"]) if w.beta != 0 else None
        adv = oracle.to_f64(x["advantages"])
    m = oracle.to_mask_u8(x["mask"])
    bs, T = lp.shape
    bounds = np.linspace(0, bs, threads + 1).astype(int)
    ranges = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    grad = np.empty((bs, T), dtype=np.float64) if fused else None
    dp = ctypes.POINTER(ctypes.c_double)

    def ptr(a, r0):
        return None if a is None else ctypes.cast(a.ctypes.data + r0 * a.strides[0], dp)

    def chunk(r):
        r0, r1 = r
        loss = ctypes.c_double(0.0)
        n = np.zeros(r1 - r0 if op.startswith("grpo") else 1, dtype=np.int64)
        g = ptr(grad, r0) if fused else None
        mp = ctypes.cast(m.ctypes.data + r0 * m.strides[0], ctypes.POINTER(ctypes.c_uint8))
        if is_rkl:
            lib.rlpl_oracle_rkl(r1 - r0, T, ptr(lp, r0), ptr(rf, r0), mp, ctypes.byref(loss), g,
                                n.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        else:
            fn = lib.rlpl_oracle_grpo if op.startswith("grpo") else lib.rlpl_oracle_bnpo
            fn(r1 - r0, T, ptr(lp, r0), ptr(od, r0), ptr(rf, r0), ctypes.cast(adv.ctypes.data + r0 * 8, dp), mp,
               float(np.float32(w.beta)), float(np.float32(w.epsilon)), float(np.float32(w.epsilon_high)),
               ctypes.byref(loss), g, n.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        return loss.value, int(n.sum())

    pool = ThreadPoolExecutor(max_workers=len(ranges))

    def rescale(args):
        (r0, r1), f = args
        if fused:
            grad[r0:r1] *= f

    def step():
        res = list(pool.map(chunk, ranges))
        N = sum(n for _, n in res)
        if op.startswith("grpo"):
            loss = sum(l * (r1 - r0) for (l, _), (r0, r1) in zip(res, ranges)) / bs
            f = [(r1 - r0) / bs for r0, r1 in ranges]
        elif is_rkl:
            loss = sum(l * n for l, n in res if n) / N if N else float("nan")
            f = [n / N if N else 0.0 for _, n in res]
        else:
            loss = sum(l * max(n, 1) for l, n in res) / max(N, 1)
            f = [max(n, 1) / max(N, 1) for _, n in res]
        list(pool.map(rescale, zip(ranges, f)))
        return loss, grad, N
    return step, len(ranges)


def cpu_baseline(op, x, w, fused, args):
    """The oracle timed on the host: one batch with its rows over every core (median of at
    least 10 steps after 3 warmups, the reported value), one whole batch on one thread, and
    independent whole batches on every core at once (throughput)."""
    import numpy as np
    import oracle
    threads = cpu_threads()
    step, n_ranges = oracle_rows_step(op, x, w, fused, threads)
    for _ in range(3):
        step()
    times = []
    t_end = time.perf_counter() + args.cpu_seconds
    while len(times) < 10 or (time.perf_counter() < t_end and len(times) < 1000):
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    # the row-split result is the batch's result (checked once, outside the timed steps)
    loss_rows, grad_rows, n_rows = step()
    whole = (oracle.rkl(x["student"], x["teacher"], x["mask"], grad=fused) if op.startswith("rkl") else
             (oracle.grpo if op.startswith("grpo") else oracle.bnpo)(
                 x["policy"], x["old"], x.get("ref") if w.beta != 0 else None, x["advantages"], x["mask"],
                 float(np.float32(w.beta)), float(np.float32(w.epsilon)), float(np.float32(w.epsilon_high)),
                 grad=fused))
    if abs(loss_rows - whole.loss) > 1e-9 * max(1.0, abs(whole.loss)) or (
            fused and float(np.max(np.abs(grad_rows - whole.grad))) > 1e-12):
        raise RuntimeError("row-split oracle disagrees with the whole-batch oracle")
    xs = {k: oracle.to_f64(v) for k, v in x.items() if k in ("policy", "old", "ref", "advantages", "student",
                                                               "teacher")}
    m8 = oracle.to_mask_u8(x["mask"])

    def run_once():
        if op.startswith("rkl"):
            oracle.rkl(xs["student"], xs["teacher"], m8, grad=fused)
        else:
            fo = oracle.bnpo if op.startswith("bnpo") else oracle.grpo
            fo(xs["policy"], xs["old"], xs.get("ref") if w.beta != 0 else None, xs["advantages"], m8,
               float(np.float32(w.beta)), float(np.float32(w.epsilon)), float(np.float32(w.epsilon_high)),
               grad=fused)
    rate1, runs1 = oracle_rate(run_once, 2.0, 1)
    rate_n, runs_n = oracle_rate(run_once, 3.0, threads) if threads > 1 else (rate1, runs1)
    return {"value": round(w.slots / med, 1), "unit": "tokens/s", "cores": n_ranges, "kind": "oracle",
            "sample": f"one full {w.name} batch (loss + gradient, double precision) per step, its rows split "
                      f"over {n_ranges} threads and combined; median of {len(times)} steps after 3 warmups, "
                      f"{med * 1e3:.3f} ms per batch",
            "cpu_model": cpu_model(),
            "single_thread_value": round(w.slots * rate1, 1),
            "independent_batches_value": round(w.slots * rate_n, 1),
            "independent_batches_sample": f"{runs_n} whole batches on {threads} threads at once, one per thread"}


def vocab_bench(args, torch):
    """Full-vocab reverse KL: logits drawn on the device, rotating sets >= 1 GiB."""
    import rl_post_loss_amd as rl
    import synthetic
    rows, V = args.rows or 1024, args.vocab or 248320
    dtype = "bf16"
    fused = args.op == "rkl_logits"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    lib = rl.library()
    x = synthetic.device_vocab_inputs(rows, V, dtype, "bool", 0, "cuda:0")
    valid = int(torch.count_nonzero(x["mask"]))
    elem = 2
    set_bytes = 2 * rows * V * elem + (rows * V * elem if fused else 0)
    nsets = max(1, math.ceil(args.rotate_gib * (1 << 30) / set_bytes))
    nsets = max(nsets, 2) if set_bytes < (1 << 30) else nsets
    ws = rl.workspace_for(dev, sptr, "rkl_logits")
    fn = lib.reverse_kl_logits if fused else lib.reverse_kl_logits_fwd
    sets, calls = [], []
    for i in range(nsets):
        st = x if i == 0 else {k: v.clone() for k, v in x.items()}
        st = dict(st)
        st["grad"] = torch.empty(rows, V, dtype=torch.bfloat16, device=dev) if fused else None
        st["loss"] = torch.empty((), dtype=torch.float32, device=dev)
        st["n"] = torch.empty(1, dtype=torch.int32, device=dev)
        sets.append(st)
        a = [st["student"].data_ptr(), st["teacher"].data_ptr(), st["mask"].data_ptr(), rows, V,
             rl.DTYPE[torch.bfloat16], rl.MASK_DTYPE[torch.bool], st["loss"].data_ptr()]
        if fused:
            a.append(st["grad"].data_ptr())
        calls.append(tuple(a + [st["n"].data_ptr(), ws.data_ptr(), ws.numel(), sptr]))
    torch.cuda.synchronize()
    ms_per_step, ms_gpu = timed(fn, calls, args.steps, args.warmup, stream, torch)
    n0 = int(sets[(args.warmup + args.steps - 1) % nsets]["n"][0].cpu())
    if n0 != valid:
        raise RuntimeError(f"valid rows {n0} != {valid}")
    # The method must read each valid row's two logit planes once and (fwd+bwd)
    # write every gradient element; the mask and the loss are negligible.
    alg = 2 * valid * V * elem + rows + 4 + (rows * V * elem if fused else 0)
    grid, vec, tiles = rl.launch_shape(rows, V, torch.bfloat16, args.op)
    # The fused kernel keeps a piece of up to 1024 32-byte blocks in registers
    # between its two passes; longer pieces are read a second time.
    blocks = V // vec if V % vec == 0 else V // vec + 2
    piece = -(-blocks // (tiles // rows))
    moved = alg + (2 * valid * V * elem if fused and piece > 1024 else 0)
    achieved = alg / (ms_gpu * 1e-3) / 1e9
    print(json.dumps({
        "metric": "full-vocab reverse KL: logit elements/s and achieved HBM GB/s (% of peak)",
        "value": round(rows * V / (ms_per_step * 1e-3), 1), "unit": "logits/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": f"rkl_logits_{dtype}_{rows}x{V}", "op": "fwd+bwd" if fused else "fwd-only",
                   "rows": rows, "vocab": V, "valid_rows": valid, "mask": "bool, U(0,1) > 0.2",
                   "inputs": "device-generated, independent N(0,1) logits", "rotating_sets": nsets,
                   "grid": grid, "piece_blocks": piece, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 5), "traffic": None},
        "kernel_us_per_launch": round(ms_gpu * 1e3, 3), "algorithmic_bytes_per_launch": alg,
        "bytes_read_and_written_by_design": moved,
        "design_GBs": round(moved / (ms_gpu * 1e-3) / 1e9, 2),
        "context_only": True}), flush=True)
    return 0


def logprob_bench(args, torch):
    """Selective log-probabilities: one group of tokens, weights resident (1 GB at the default size)."""
    import rl_post_loss_amd as rl
    import synthetic
    n, H, V = args.rows or 1024, args.hidden or 4096, args.vocab or 128256
    fused = args.op == "logprob"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    lib = rl.library()
    x = synthetic.device_logprob_inputs(n, H, V, "bf16", 0, "cuda:0")
    align = lambda t: t.data_ptr() + (-t.data_ptr()) % 256
    ws_f = torch.empty(lib.selective_logprob_workspace_bytes(n, H, V, 0) + 256, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(lib.selective_logprob_workspace_bytes(n, H, V, 1) + 256, dtype=torch.uint8, device=dev)
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    dh = torch.empty(n, H, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(V, H, dtype=torch.float32, device=dev)
    db = torch.empty(V, dtype=torch.float32, device=dev)
    bf16 = rl.DTYPE[torch.bfloat16]
    common = (x["hidden"].data_ptr(), x["weight"].data_ptr(), x["bias"].data_ptr(), x["targets"].data_ptr())

    def fwd():
        return lib.selective_logprob_fwd(*common, n, H, V, bf16, logp.data_ptr(), lse.data_ptr(), align(ws_f),
                                         ws_f.numel() - 256, sptr)

    def step():
        rc = fwd()
        return rc or lib.selective_logprob_bwd(*common, lse.data_ptr(), x["grad_logp"].data_ptr(), n, H, V, bf16,
                                               dh.data_ptr(), dw.data_ptr(), db.data_ptr(), 0, align(ws_b),
                                               ws_b.numel() - 256, sptr)
    torch.cuda.synchronize()
    ms_per_step, ms_gpu = timed(step if fused else fwd, [()], args.steps, args.warmup, stream, torch)
    _, ms_fwd = timed(fwd, [()], args.steps, args.warmup, stream, torch)
    if not bool(torch.isfinite(logp).all()):
        raise RuntimeError("non-finite log-probabilities")
    # The method's contractions: logits (2nVH) forward; hidden and weight gradients (2nVH each) backward.
    # The backward here also recomputes the logits (another 2nVH) instead of storing them.
    alg = 2 * n * V * H * (3 if fused else 1)
    done = 2 * n * V * H * (4 if fused else 1)
    tflops = alg / (ms_gpu * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        xh, xw, xb = (oracle.to_f64(x[k][:2] if k == "hidden" else x[k]) for k in ("hidden", "weight", "bias"))
        y = x["targets"][:2].cpu().numpy()
        g = oracle.to_f64(x["grad_logp"][:2])
        t0 = time.perf_counter()
        oracle.selective_logprob(xh, xw, xb, y, g if fused else None)
        sec = time.perf_counter() - t0
        cpu = {"value": round(2 / sec, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"2 tokens of the same problem (H = {H}, V = {V}), {'forward + backward' if fused else 'forward'}, "
                         f"double precision, one thread: {sec:.2f} s"}
    print(json.dumps({
        "metric": "selective log-probs: tokens/s and achieved matrix-core TFLOP/s (% of dense bf16 peak)",
        "value": round(n / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"logprob_bf16_{n}x{H}x{V}", "op": "fwd+bwd" if fused else "fwd-only",
                   "tokens": n, "hidden": H, "vocab": V, "bias": True,
                   "inputs": "device-generated: hidden N(0,1), weight N(0,4/H), bias N(0,1/4), uniform targets",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 5), "traffic": None},
        "cpu_baseline": cpu,
        "gpu_ms_per_step": round(ms_gpu, 4), "gpu_ms_forward": round(ms_fwd, 4),
        "forward_TFLOPs": round(2 * n * V * H / (ms_fwd * 1e-3) / 1e12, 2),
        "algorithmic_flops_per_step": alg, "executed_matrix_flops_per_step": done,
        "executed_TFLOPs": round(done / (ms_gpu * 1e-3) / 1e12, 2),
        "context_only": True}), flush=True)
    return 0


def chain_bench(args, torch):
    """Policy and reference log-probs -> GRPO loss -> policy backward, B sequences of 1024 tokens."""
    import rl_post_loss_amd as rl
    import synthetic
    bs, T, H, V = args.bs or 1, 1024, args.hidden or 4096, args.vocab or 128256
    n = bs * T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    lib = rl.library()
    pol = synthetic.device_logprob_inputs(n, H, V, "bf16", 0, "cuda:0")
    refm = synthetic.device_logprob_inputs(n, H, V, "bf16", 1, "cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    adv = torch.randn(bs, generator=g, device=dev)
    lengths = torch.randint(T // 4, T + 1, (bs,), generator=g, device=dev)
    mask = (torch.arange(T, device=dev)[None, :] < lengths[:, None]).to(torch.int8)
    align = lambda t: t.data_ptr() + (-t.data_ptr()) % 256
    ws_f = torch.empty(lib.selective_logprob_workspace_bytes(n, H, V, 0) + 256, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(lib.selective_logprob_workspace_bytes(n, H, V, 1) + 256, dtype=torch.uint8, device=dev)
    ws_l = rl.workspace_for(dev, sptr, "grpo")
    lp, lse = torch.empty(n, device=dev), torch.empty(n, device=dev)
    ref, ref_lse = torch.empty(n, device=dev), torch.empty(n, device=dev)
    loss, grad = torch.empty((), device=dev), torch.empty(n, device=dev)
    dh = torch.empty(n, H, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(V, H, dtype=torch.float32, device=dev)
    db = torch.empty(V, dtype=torch.float32, device=dev)
    bf16, f32, i8 = rl.DTYPE[torch.bfloat16], rl.DTYPE[torch.float32], rl.MASK_DTYPE[torch.int8]
    P = lambda d: (d["hidden"].data_ptr(), d["weight"].data_ptr(), d["bias"].data_ptr(), pol["targets"].data_ptr())

    def fwd(d, out, out_lse):
        return lib.selective_logprob_fwd(*P(d), n, H, V, bf16, out.data_ptr(), out_lse.data_ptr(), align(ws_f),
                                         ws_f.numel() - 256, sptr)
    # behaviour log-probs: the policy's own, slightly perturbed (inputs only, outside the timed region)
    fwd(pol, lp, lse)
    torch.cuda.synchronize()
    old = (lp + 0.05 * torch.randn(n, generator=g, device=dev)).contiguous()

    def step():
        rc = fwd(pol, lp, lse) or fwd(refm, ref, ref_lse)
        rc = rc or lib.grpo_loss(lp.data_ptr(), old.data_ptr(), ref.data_ptr(), adv.data_ptr(), mask.data_ptr(),
                                 bs, T, f32, i8, 0.04, 0.2, 0.28, loss.data_ptr(), grad.data_ptr(), None,
                                 ws_l.data_ptr(), ws_l.numel(), sptr)
        return rc or lib.selective_logprob_bwd(*P(pol), lse.data_ptr(), grad.data_ptr(), n, H, V, bf16,
                                               dh.data_ptr(), dw.data_ptr(), db.data_ptr(), 0, align(ws_b),
                                               ws_b.numel() - 256, sptr)
    torch.cuda.synchronize()
    ms_per_step, ms_gpu = timed(step, [()], args.steps, args.warmup, stream, torch)
    if not bool(torch.isfinite(loss)):
        raise RuntimeError("non-finite loss")
    alg = 2 * n * V * H * 4          # policy and reference logits, hidden and weight gradients
    done = 2 * n * V * H * 5         # plus the logits recomputed in the backward
    tflops = alg / (ms_gpu * 1e-3) / 1e12
    print(json.dumps({
        "metric": "log-prob -> GRPO chain (policy + reference log-probs, loss, backward): tokens/s and "
                  "achieved matrix-core TFLOP/s",
        "value": round(n / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"grpo_chain_bf16_{bs}x{T}_H{H}_V{V}", "sequences": bs, "tokens": n, "hidden": H,
                   "vocab": V, "beta": 0.04, "epsilon": 0.2, "epsilon_high": 0.28,
                   "mask": f"int8 prefix U[{T // 4},{T}]", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 5), "traffic": None},
        "cpu_baseline": None,
        "gpu_ms_per_step": round(ms_gpu, 4), "algorithmic_flops_per_step": alg,
        "executed_matrix_flops_per_step": done, "executed_TFLOPs": round(done / (ms_gpu * 1e-3) / 1e12, 2),
        "context_only": True}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bnpo_bf16_64x4096")
    ap.add_argument("--op", default=None, choices=["bnpo", "bnpo_fwd", "grpo", "grpo_fwd", "rkl", "rkl_fwd",
                                                   "rkl_logits", "rkl_logits_fwd", "logprob", "logprob_fwd",
                                                   "grpo_chain"])
    ap.add_argument("--rows", type=int, default=None)
    ap.add_argument("--vocab", type=int, default=None)
    ap.add_argument("--hidden", type=int, default=None)
    ap.add_argument("--bs", type=int, default=None)
    ap.add_argument("--seq-len", type=int, default=None)
    ap.add_argument("--beta", type=float, default=None)
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=float, default=None)
    ap.add_argument("--copy-variant", type=int, default=None, choices=sorted(COPY_VARIANTS))
    ap.add_argument("--copy-grid", type=int, default=None)
    ap.add_argument("--read-mib", type=float, default=None)
    ap.add_argument("--noalloc", action="store_true")
    ap.add_argument("--floor", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library is measured on one GPU only "
              f"(the loss shards by rows across GPUs)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_mib is not None:
        return copy_ceiling(args, torch)
    if args.read_mib is not None:
        return read_ceiling(args, torch)
    if args.floor:
        return launch_floor(args, torch)
    if args.op in ("rkl_logits", "rkl_logits_fwd"):
        return vocab_bench(args, torch)
    if args.op in ("logprob", "logprob_fwd"):
        return logprob_bench(args, torch)
    if args.op == "grpo_chain":
        return chain_bench(args, torch)

    import rl_post_loss_amd as rl
    import synthetic

    w = synthetic.WORKLOADS[args.workload]
    headline = args.op is None and args.bs is None and args.seq_len is None and args.beta is None and not args.noalloc
    op = args.op or w.op
    if args.bs or args.seq_len:
        w = w.with_(bs=args.bs or w.bs, seq_len=args.seq_len or w.seq_len,
                    len_lo=min(w.len_lo, args.seq_len or w.seq_len), len_hi=args.seq_len or w.len_hi,
                    name=f"{w.name}@{args.bs or w.bs}x{args.seq_len or w.seq_len}")
    if args.beta is not None:
        w = w.with_(beta=args.beta)
    fused = not op.endswith("_fwd")
    is_rkl = op.startswith("rkl")
    if is_rkl and not w.op == "rkl":
        w = w.with_(op="rkl")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    lib = rl.library()

    on_device = w.slots > (1 << 24)
    if on_device:
        d = synthetic.device_policy_inputs(w, "cuda:0")
        x = {"student": d["policy"], "teacher": d["ref"], "mask": d["mask"]} if is_rkl else d
    else:
        x = synthetic.inputs(w)
    valid = int(torch.count_nonzero(x["mask"]))
    planes = ["student", "teacher"] if is_rkl else (["policy", "old", "ref"] if w.beta != 0 else ["policy", "old"])
    dt = x[planes[0]].dtype
    elem = x[planes[0]].element_size()
    base = {k: x[k].to(dev) for k in planes + ["mask"] + ([] if is_rkl else ["advantages"])}
    set_bytes = sum(t.numel() * t.element_size() for t in base.values()) + (w.slots * elem if fused else 0)
    nsets = max(1, math.ceil(args.rotate_gib * (1 << 30) / set_bytes)) if set_bytes < (1 << 29) else 1
    if nsets == 1 and not on_device:
        nsets = 2
    ws = rl.workspace_for(dev, sptr, w.op)
    blib = bench_lib()
    sets, rows = [], []
    for i in range(nsets):
        s = base if i == 0 else {k: v.clone() for k, v in base.items()}
        s = dict(s)
        s["grad"] = torch.empty(w.bs, w.seq_len, dtype=dt, device=dev) if fused else None
        s["loss"] = torch.empty((), dtype=torch.float32, device=dev)
        s["n"] = torch.empty(w.bs, dtype=torch.int32, device=dev)
        sets.append(s)
        g = s["grad"].data_ptr() if fused else 0
        if is_rkl:
            rows.append([s["student"].data_ptr(), s["teacher"].data_ptr(), s["mask"].data_ptr(),
                         s["loss"].data_ptr(), g, s["n"].data_ptr()])
        else:
            rows.append([s["policy"].data_ptr(), s["old"].data_ptr(), s["ref"].data_ptr() if "ref" in s else 0,
                         s["advantages"].data_ptr(), s["mask"].data_ptr(), s["loss"].data_ptr(), g,
                         s["n"].data_ptr()])
    table = pointer_table(rows)
    dtc, mdc = rl.DTYPE[dt], rl.MASK_DTYPE[base["mask"].dtype]
    if is_rkl:
        run = lambda first, k: blib.rlpl_bench_rkl(int(fused), nsets, table.ctypes.data, w.bs, w.seq_len, dtc, mdc,
                                                   ws.data_ptr(), ws.numel(), k, first, sptr)
    elif args.noalloc:
        if op != "bnpo":
            raise SystemExit("--noalloc measures the fused BNPO loss only")
        run = lambda first, k: blib.rlpl_bench_noalloc(nsets, table.ctypes.data, w.bs, w.seq_len, dtc, mdc, w.beta,
                                                       w.epsilon, w.epsilon_high, k, first, sptr)
    else:
        run = lambda first, k: blib.rlpl_bench_policy(rl.OP[op], 0, nsets, table.ctypes.data, w.bs, w.seq_len, dtc,
                                                      mdc, w.beta, w.epsilon, w.epsilon_high, ws.data_ptr(),
                                                      ws.numel(), k, first, sptr)
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    ms_per_step, ms_gpu = timed_loop(run, K, W, stream, torch)
    tokens_per_s = w.slots / (ms_per_step * 1e-3)

    if not op.startswith("grpo"):
        n0 = int(sets[(W + K - 1) % nsets]["n"][0].cpu())
        if n0 != valid:
            raise RuntimeError(f"valid count {n0} != {valid}")

    alg = algorithmic_bytes(op, w.slots, valid, w.bs, elem, is_rkl or w.beta != 0, fused)
    achieved = alg / (ms_gpu * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 5),
                "traffic": recorded_traffic(w.name) if headline else None,
                "traffic_unit": "HBM bytes per launch (read + written), calibrated rocprofv3 counters"}

    cpu = None
    if headline and not args.no_cpu_baseline:
        cpu = cpu_baseline(op, x, w, fused, args)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[dt],
        "data": "synthetic",
        "config": {"workload": w.name, "op": op.replace("_fwd", " fwd-only") + ("" if op.endswith("_fwd") else " fwd+bwd"),
                   "bs": w.bs, "seq_len": w.seq_len, "beta": 1.0 if is_rkl else w.beta,
                   "epsilon": w.epsilon, "epsilon_high": w.epsilon_high,
                   "mask": f"{w.mask_dtype} prefix U[{w.len_lo},{w.len_hi}]", "valid_tokens": valid,
                   "tokens_counted": "bs * seq_len (row, position) slots per step",
                   "inputs": "device-generated" if on_device else "host-generated",
                   "rotating_sets": nsets, "entry_point": "bnpo_loss_noalloc" if args.noalloc else "C ABI",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "valid_tokens_per_s": round(valid / (ms_per_step * 1e-3), 1),
        "kernel_us_per_launch": round(ms_gpu * 1e3, 3),
        "algorithmic_bytes_per_launch": alg,
    }
    if not headline:
        out["context_only"] = True
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
