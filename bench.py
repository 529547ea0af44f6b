#!/usr/bin/env python3
"""Throughput of the fused PPO-family policy loss on one MI355X.

One step = one fused forward+backward BNPO call (bs=64, seq_len=4096, bf16
log-probs, int8 prefix mask with lengths U[256, 4096], beta=0.04, eps=0.2,
eps_high=0.28): the whole hot path (stream-in, per-token policy and KL terms,
local reduction, on-GPU global count, 1/N scaling, gradient store, loss
finalise) in one launch through the C ABI.

Inputs are generated once, copied into rotating sets totalling >= 1 GiB (so
each step reads from HBM rather than the 256 MB last-level cache) and are
resident before timing starts.  W warmup steps, then exactly K timed steps
between two stream synchronisations.  HIP events are recorded
on the stream it runs on at both ends of the timed region: their span / K is
the per-launch kernel duration used for the roofline (back-to-back launches
keep the GPU busy, so this agrees with rocprofv3's kernel durations).

Prints one JSON line (see the keys below).  --gpus above 1 is not supported.
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


def algorithmic_bytes(op: str, slots: int, valid: int, bs: int, elem: int, has_kl: bool, fused: bool) -> int:
    """Bytes the method must move: the mask and (fused) the dense gradient for every slot;
    the input planes only for valid tokens; the advantages and the 4-byte loss."""
    planes = 2 if op == "rkl" else (3 if has_kl else 2)
    b = slots * 1 + valid * planes * elem + 4
    if fused:
        b += slots * elem
    if op != "rkl":
        b += bs * elem
    return b


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bnpo_bf16_64x4096")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build measures one GPU only "
              f"(the loss shards by rows; see the design notes)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import rl_post_loss_amd as rl
    import synthetic

    w = synthetic.WORKLOADS[args.workload]
    if w.op not in ("bnpo", "grpo", "rkl"):
        raise SystemExit(f"unknown op {w.op}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    lib = rl.library()

    x = synthetic.inputs(w)
    mask_cpu = x["mask"]
    valid = int(torch.count_nonzero(mask_cpu))
    planes = ["student", "teacher"] if w.op == "rkl" else (["policy", "old", "ref"] if w.beta != 0
                                                            else ["policy", "old"])
    dt = x[planes[0]].dtype
    elem = x[planes[0]].element_size()
    base = {k: x[k].to(dev) for k in planes + ["mask"] + ([] if w.op == "rkl" else ["advantages"])}
    set_bytes = sum(t.numel() * t.element_size() for t in base.values()) + w.slots * elem
    nsets = max(2, math.ceil(args.rotate_gib * (1 << 30) / set_bytes))
    ws = rl.workspace_for(dev, sptr, w.op)
    sets, calls = [], []
    fn = {"bnpo": lib.bnpo_loss, "grpo": lib.grpo_loss, "rkl": lib.reverse_kl}[w.op]
    for _ in range(nsets):
        s = {k: v.clone() for k, v in base.items()}
        s["grad"] = torch.empty(w.bs, w.seq_len, dtype=dt, device=dev)
        s["loss"] = torch.empty((), dtype=torch.float32, device=dev)
        s["n"] = torch.empty(w.bs, dtype=torch.int32, device=dev)
        sets.append(s)
        if w.op == "rkl":
            a = (s["student"].data_ptr(), s["teacher"].data_ptr(), s["mask"].data_ptr(), w.bs,
                 w.seq_len, rl.DTYPE[dt], rl.MASK_DTYPE[s["mask"].dtype], s["loss"].data_ptr(),
                 s["grad"].data_ptr(), s["n"].data_ptr(), ws.data_ptr(), ws.numel(), sptr)
        else:
            a = (s["policy"].data_ptr(), s["old"].data_ptr(),
                 s["ref"].data_ptr() if "ref" in s else None, s["advantages"].data_ptr(),
                 s["mask"].data_ptr(), w.bs, w.seq_len, rl.DTYPE[dt], rl.MASK_DTYPE[s["mask"].dtype],
                 w.beta, w.epsilon, w.epsilon_high, s["loss"].data_ptr(), s["grad"].data_ptr(),
                 s["n"].data_ptr(), ws.data_ptr(), ws.numel(), sptr)
        calls.append(a)
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    for i in range(W):
        rc = fn(*calls[i % nsets])
        if rc != 0:
            raise rl.RlplError(fn.__name__, rc)
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches between two stream synchronisations, with
    # HIP events recorded on the launch stream at both ends of it.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bad = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        bad |= fn(*calls[(W + i) % nsets])
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if bad:
        raise RuntimeError("a timed call returned an error status")
    k_mean = ev0.elapsed_time(ev1) / K          # ms per launch on the GPU timeline
    ms_per_step = (t1 - t0) * 1e3 / K
    tokens_per_s = w.slots / (ms_per_step * 1e-3)

    # Check one timed result against the oracle-free invariants the kernel must keep.
    n0 = int(sets[(W + K - 1) % nsets]["n"][0].cpu()) if w.op != "grpo" else None
    if n0 is not None and n0 != valid:
        raise RuntimeError(f"valid count {n0} != {valid}")

    alg = algorithmic_bytes(w.op, w.slots, valid, w.bs, elem, w.op == "rkl" or w.beta != 0, True)
    achieved = alg / (k_mean * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 5), "traffic": None}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        xs = {k: oracle.to_f64(v) for k, v in x.items() if k in planes or k == "advantages"}
        m8 = oracle.to_mask_u8(mask_cpu)
        f32 = lambda v: float(np.float32(v))
        runs, tc0 = 0, time.perf_counter()
        while True:
            if w.op == "rkl":
                oracle.rkl(xs["student"], xs["teacher"], m8)
            else:
                fo = oracle.bnpo if w.op == "bnpo" else oracle.grpo
                fo(xs["policy"], xs["old"], xs.get("ref"), xs["advantages"], m8, f32(w.beta),
                   f32(w.epsilon), f32(w.epsilon_high))
            runs += 1
            if time.perf_counter() - tc0 >= args.cpu_seconds:
                break
        tc = (time.perf_counter() - tc0) / runs
        cpu = {"value": round(w.slots / tc, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{runs} full {w.name} batches (loss + grad, double precision, one thread), "
                         f"{tc * 1e3:.1f} ms each"}

    out = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak) for fused loss fwd+bwd",
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
        "config": {"workload": w.name, "op": w.op + " fwd+bwd", "bs": w.bs, "seq_len": w.seq_len,
                   "beta": w.beta, "epsilon": w.epsilon, "epsilon_high": w.epsilon_high,
                   "mask": f"{w.mask_dtype} prefix U[{w.len_lo},{w.len_hi}]", "valid_tokens": valid,
                   "rotating_sets": nsets, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_us_per_launch": round(k_mean * 1e3, 3),
        "algorithmic_bytes_per_launch": alg,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
