"""Parity of the HIP kernels (through the C ABI binding) with the CPU oracle.

Every workload runs at its full size (the oracle finishes each in well under a
second), element by element, at the tolerances in parity.py.  Edge cases
cover empty and ragged inputs, tails shorter than a lane, seq_len not a
multiple of 16, one-slot rows, odd int8 mask bytes, grids where every
workgroup owns several tiles, and rows longer than a tile.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import rl_post_loss_amd as rl
import synthetic
from parity import (check_grad, check_loss, check_masked_zero, f32, kink_alternative, kink_tokens,
                    policy_grad_magnitude, rkl_grad_magnitude, sign_aware_kinks)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def gpu_policy(op, fused, g, beta, eps, eps_high, ref=True, clip="literal"):
    fn = {("bnpo", True): rl.bnpo_loss, ("bnpo", False): rl.bnpo_loss_fwd,
          ("grpo", True): rl.grpo_loss, ("grpo", False): rl.grpo_loss_fwd}[(op, fused)]
    out = fn(g["policy"], g["old"], g["ref"] if ref else None, g["advantages"], g["mask"],
             epsilon=eps, epsilon_high=eps_high, beta=beta, return_n_valid=True, clip=clip)
    torch.cuda.synchronize()
    return out


def oracle_policy(op, x, beta, eps, eps_high, clip="literal"):
    fn = oracle.bnpo if op == "bnpo" else oracle.grpo
    return fn(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], f32(beta), f32(eps),
              f32(eps_high), sign_aware=clip == "sign_aware")


def assert_policy_parity(op, x, beta, eps, eps_high, what, fused=True, clip="literal"):
    g = dev(x)
    ref = oracle_policy(op, x, beta, eps, eps_high, clip)
    out = gpu_policy(op, fused, g, beta, eps, eps_high, ref=beta != 0.0, clip=clip)
    loss, n = (out[0], out[-1])
    dt = x["policy"].dtype
    check_loss(float(loss.cpu()), ref.loss, dt, what)
    if op == "bnpo":
        assert int(n.cpu()[0]) == ref.n_valid, what
    else:
        np.testing.assert_array_equal(n.cpu().numpy().astype(np.int64), ref.n_valid, err_msg=what)
    if fused:
        grad = out[1]
        assert grad.dtype == dt and grad.shape == x["policy"].shape
        if op == "bnpo":
            scale = 1.0 / max(ref.n_valid, 1)
        else:
            scale = (1.0 / (np.maximum(ref.n_valid, 1) * x["policy"].shape[0]))[:, None]
        if clip == "literal":
            kinks = kink_tokens(x["policy"], x["old"], x["mask"], eps_high)
            alt = kink_alternative(ref.grad, x["policy"], x["old"], x["advantages"], x["mask"],
                                   eps_high, scale)
        else:
            kinks, alt = sign_aware_kinks(ref.grad, x, eps, eps_high, scale)
        mag = policy_grad_magnitude(x["policy"], x["old"], x["ref"], x["advantages"], f32(beta), scale)
        check_grad(grad, ref.grad, dt, what, alt, kinks, mag)
        check_masked_zero(grad, x["mask"], what)
    return out


def assert_rkl_parity(x, what, fused=True):
    g = dev(x)
    ref = oracle.rkl(x["student"], x["teacher"], x["mask"])
    fn = rl.reverse_kl if fused else rl.reverse_kl_fwd
    out = fn(g["student"], g["teacher"], g["mask"], return_n_valid=True)
    torch.cuda.synchronize()
    dt = x["student"].dtype
    check_loss(float(out[0].cpu()), ref.loss, dt, what)
    assert int(out[-1].cpu()[0]) == ref.n_valid, what
    if fused:
        mag = rkl_grad_magnitude(x["student"], x["teacher"], 1.0 / max(ref.n_valid, 1))
        check_grad(out[1], ref.grad, dt, what, mag=mag)
        check_masked_zero(out[1], x["mask"], what)
    return out


# --------------------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["bnpo_fp32_4x64", "bnpo_bf16_16x1024", "bnpo_bf16_64x4096",
                                  "grpo_fp16_128x2048"])
def test_workload_parity(name):
    w = synthetic.WORKLOADS[name]
    x = synthetic.inputs(w)
    print(f"[parity] {name} beta={w.beta}", flush=True)
    assert_policy_parity(w.op, x, w.beta, w.epsilon, w.epsilon_high, name)
    assert_policy_parity(w.op, x, w.beta, w.epsilon, w.epsilon_high, name + " fwd", fused=False)


def test_bnpo_64x4096_beta0_kl_compiled_out():
    w = synthetic.WORKLOADS["bnpo_bf16_64x4096"].with_(beta=0.0)
    x = synthetic.inputs(w)
    assert_policy_parity("bnpo", x, 0.0, w.epsilon, w.epsilon_high, "beta0")
    assert_policy_parity("bnpo", x, 0.0, w.epsilon, w.epsilon_high, "beta0 fwd", fused=False)


def test_rkl_workload_parity():
    w = synthetic.WORKLOADS["rkl_bf16_256x8192"]
    x = synthetic.inputs(w)
    print("[parity] rkl_bf16_256x8192", flush=True)
    assert_rkl_parity(x, "rkl")
    assert_rkl_parity(x, "rkl fwd", fused=False)


# --------------------------------------------------------------------------- exactness properties

@pytest.mark.parametrize("op", ["bnpo", "grpo", "rkl"])
def test_forward_only_loss_equals_fused_loss_bitwise(op):
    if op == "rkl":
        x = dev(synthetic.inputs(synthetic.WORKLOADS["rkl_bf16_256x8192"]))
        a = rl.reverse_kl(x["student"], x["teacher"], x["mask"])[0]
        b = rl.reverse_kl_fwd(x["student"], x["teacher"], x["mask"])
    else:
        w = synthetic.WORKLOADS["bnpo_bf16_64x4096" if op == "bnpo" else "grpo_fp16_128x2048"]
        x = dev(synthetic.inputs(w))
        kw = dict(epsilon=w.epsilon, epsilon_high=w.epsilon_high, beta=w.beta)
        fused, fwd = (rl.bnpo_loss, rl.bnpo_loss_fwd) if op == "bnpo" else (rl.grpo_loss, rl.grpo_loss_fwd)
        a = fused(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], **kw)[0]
        b = fwd(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], **kw)
    assert a.cpu().view(torch.int32).item() == b.cpu().view(torch.int32).item()


def test_repeated_calls_are_bitwise_identical_and_leave_tagged_entries():
    """Every call publishes its values as entries carrying its launch's two tags (workspace
    header: flags at byte 128, release entry at 384; per-worker count entries from byte 512,
    16 bytes each: value, t0, value, t1); the next call carries other tags."""
    w = synthetic.WORKLOADS["bnpo_bf16_64x4096"]
    x = dev(synthetic.inputs(w))
    kw = dict(epsilon=w.epsilon, epsilon_high=w.epsilon_high, beta=w.beta)
    l0, g0 = rl.bnpo_loss(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], **kw)
    for _ in range(50):
        l1, g1 = rl.bnpo_loss(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], **kw)
        assert torch.equal(l1.view(torch.int32), l0.view(torch.int32))
        assert torch.equal(g1.view(torch.int16), g0.view(torch.int16))
    torch.cuda.synchronize()
    ws = rl.workspace_for(DEV, torch.cuda.current_stream(DEV).cuda_stream, "bnpo")
    n_valid = int(torch.count_nonzero(x["mask"]))
    grid, vec, tiles = rl.launch_shape(64, 4096, torch.bfloat16, "bnpo")
    assert grid == tiles + 1                              # one coordinator plus one worker per tile

    def head():
        return ws[:512 + 16 * tiles].cpu().view(torch.int32).numpy().view(np.uint32)
    h = head()
    assert h[128 // 4] == 0                               # no timeout flag
    rel = h[384 // 4:384 // 4 + 4]
    assert rel[0] == rel[2] == n_valid and rel[1] != 0 and rel[3] != 0
    cnt = h[512 // 4:].reshape(tiles, 4)
    assert (cnt[:, 1] == rel[1]).all() and (cnt[:, 3] == rel[3]).all()   # the same launch's tags
    assert (cnt[:, 0] == cnt[:, 2]).all() and int(cnt[:, 0].sum()) == n_valid
    rl.bnpo_loss(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], **kw)
    torch.cuda.synchronize()
    rel2 = head()[384 // 4:384 // 4 + 4]
    assert rel2[0] == n_valid and rel2[1] != rel[1] and rel2[3] != rel[3]
    import ctypes
    flags = ctypes.c_uint32(7)
    assert rl.library().rlpl_workspace_flags(ws.data_ptr(), ctypes.byref(flags),
                                             torch.cuda.current_stream(DEV).cuda_stream) == 0
    assert flags.value == 0


def test_lower_clip_bound_has_no_effect():
    w = synthetic.WORKLOADS["bnpo_bf16_16x1024"]
    x = dev(synthetic.inputs(w))
    base = rl.bnpo_loss(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"],
                        epsilon=0.2, epsilon_high=0.28, beta=0.04)
    for eps in (0.0, 0.5, 0.9):
        o = rl.bnpo_loss(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"],
                         epsilon=eps, epsilon_high=0.28, beta=0.04)
        assert torch.equal(o[0], base[0]) and torch.equal(o[1], base[1])


# --------------------------------------------------------------------------- edge cases

def _custom(op, dtype, bs, T, mask_kind="prefix", seed=5, mask_dtype="int8", lo=0, hi=None):
    w = synthetic.Workload("edge", op, dtype, mask_dtype, bs, T, lo, T if hi is None else hi, seed=seed)
    x = synthetic.inputs(w)
    rng = np.random.default_rng(seed + 100)
    if mask_kind == "random":
        m = rng.random((bs, T)) < 0.6
        x["mask"] = torch.from_numpy(m).to(synthetic.MASK_DTYPES[mask_dtype])
    elif mask_kind == "none":
        x["mask"] = torch.zeros(bs, T, dtype=synthetic.MASK_DTYPES[mask_dtype])
    elif mask_kind == "odd_bytes":
        v = rng.integers(-128, 128, size=(bs, T)).astype(np.int8)
        v[rng.random((bs, T)) < 0.4] = 0
        x["mask"] = torch.from_numpy(v)
    return x


SHAPES = [(1, 1), (1, 5), (3, 37), (2, 17), (5, 3), (7, 1), (4, 1000), (2, 4097), (1, 4096),
          (3, 16), (9, 4095)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("bs,T", SHAPES)
def test_edge_shapes_bnpo_grpo(dtype, bs, T):
    x = _custom("bnpo", dtype, bs, T, "random", seed=bs * 131 + T)
    what = f"{dtype} {bs}x{T}"
    assert_policy_parity("bnpo", x, 0.04, 0.2, 0.28, "bnpo " + what)
    assert_policy_parity("grpo", x, 0.04, 0.2, 0.28, "grpo " + what)
    assert_policy_parity("bnpo", x, 0.0, 0.2, 0.28, "bnpo beta0 " + what)


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("bs,T", [(1, 1), (3, 37), (4, 1000), (2, 4097)])
def test_edge_shapes_rkl(dtype, bs, T):
    w = synthetic.Workload("edge", "rkl", dtype, "bool", bs, T, 1, T, seed=bs + T)
    x = synthetic.inputs(w)
    assert_rkl_parity(x, f"rkl {dtype} {bs}x{T}")


@pytest.mark.parametrize("op", ["bnpo", "grpo"])
def test_all_masked_policy(op):
    x = _custom(op, "bf16", 4, 300, "none")
    out = assert_policy_parity(op, x, 0.04, 0.2, 0.28, f"{op} all masked")
    assert float(out[0].cpu()) == 0.0
    assert torch.all(out[1] == 0)


def test_all_masked_rkl_gives_nan_loss_and_zero_grad():
    w = synthetic.Workload("edge", "rkl", "bf16", "bool", 3, 100, 1, 100)
    x = synthetic.inputs(w)
    x["mask"] = torch.zeros(3, 100, dtype=torch.bool)
    out = assert_rkl_parity(x, "rkl all masked")
    assert math.isnan(float(out[0].cpu()))
    assert torch.all(out[1] == 0)


def test_single_valid_token():
    x = _custom("bnpo", "fp32", 3, 50, "none")
    x["mask"][1, 17] = 1
    assert_policy_parity("bnpo", x, 0.04, 0.2, 0.28, "single token bnpo")
    assert_policy_parity("grpo", x, 0.04, 0.2, 0.28, "single token grpo")


def test_int8_mask_nonzero_bytes_are_valid():
    x = _custom("bnpo", "bf16", 6, 333, "odd_bytes")
    assert_policy_parity("bnpo", x, 0.04, 0.2, 0.28, "odd bytes bnpo")
    assert_policy_parity("grpo", x, 0.04, 0.2, 0.28, "odd bytes grpo")


def test_bool_and_int8_masks_agree():
    x = _custom("bnpo", "bf16", 8, 512, "random", mask_dtype="bool")
    a = dev(x)
    o1 = rl.bnpo_loss(a["policy"], a["old"], a["ref"], a["advantages"], a["mask"], beta=0.04)
    o2 = rl.bnpo_loss(a["policy"], a["old"], a["ref"], a["advantages"], a["mask"].to(torch.int8), beta=0.04)
    assert torch.equal(o1[0], o2[0]) and torch.equal(o1[1], o2[1])


def test_multi_tile_grid_bnpo_and_rkl():
    # 8M slots: more tiles than co-resident workgroups, so each workgroup counts
    # several masks before the exchange and then streams its tiles.
    x = _custom("bnpo", "bf16", 1024, 8192, "prefix", lo=0)
    print("[parity] multi-tile bnpo 1024x8192", flush=True)
    assert_policy_parity("bnpo", x, 0.04, 0.2, 0.28, "multi-tile bnpo")
    assert_policy_parity("bnpo", x, 0.04, 0.2, 0.28, "multi-tile bnpo fwd", fused=False)
    w = synthetic.Workload("edge", "rkl", "bf16", "bool", 1024, 8192, 1, 8192)
    assert_rkl_parity(synthetic.inputs(w), "multi-tile rkl")


def _shape_kind(grid, vec, tiles):
    if tiles >= grid:
        return "stream"
    return "one-tile vec%d" % vec


@pytest.mark.parametrize("op", ["bnpo", "grpo", "rkl"])
def test_every_kernel_shape(op):
    # The three kernel shapes (one tile per worker with the narrow or the wide
    # lane, and the wide lane striding over several tiles per worker), each in
    # its fused and forward-only form, reached through problem size alone.
    kinds = set()
    # (GRPO's one-tile kernels hold fewer workgroups per compute unit, so its
    # wide one-tile case is a smaller problem.)
    for bs, T in [(64, 4096), (512 if op == "grpo" else 1024, 4096), (1024, 8192)]:
        grid, vec, tiles = rl.launch_shape(bs, T, torch.bfloat16, op)
        kind = _shape_kind(grid, vec, tiles)
        kinds.add(kind)
        what = f"{op} {bs}x{T} {kind} grid={grid} tiles={tiles}"
        print("[parity]", what, flush=True)
        if op == "rkl":
            w = synthetic.Workload("edge", "rkl", "bf16", "bool", bs, T, 1, T, seed=bs + T)
            x = synthetic.inputs(w)
            assert_rkl_parity(x, what)
            assert_rkl_parity(x, what + " fwd", fused=False)
        else:
            x = _custom(op, "bf16", bs, T, "prefix", seed=bs + T, lo=0)
            assert_policy_parity(op, x, 0.04, 0.2, 0.28, what)
            assert_policy_parity(op, x, 0.04, 0.2, 0.28, what + " fwd", fused=False)
    assert kinds == {"one-tile vec4", "one-tile vec16", "stream"}, kinds


# 16-slot lanes take their slots as chunks of 16 bytes of a plane (two of 8
# slots for fp16/bf16, four of 4 for fp32), a wavefront access apart.  Odd
# seq_len puts row ends inside chunks (the per-slot path), random masks leave
# some chunks of a lane valid and others not (planes loaded per chunk), in
# the wide one-tile kernel (257 x 4093) and the striding one (1000 x 8191).
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("bs,T", [(257, 4093), (1000, 8191)])
def test_chunked_lanes_rows_ending_inside_chunks(dtype, bs, T):
    kinds = set()
    for op in ("bnpo", "grpo"):
        grid, vec, tiles = rl.launch_shape(bs, T, TORCH_DT[dtype], op)
        assert vec == 16, (op, grid, vec, tiles)
        kinds.add(_shape_kind(grid, vec, tiles))
        for mask in ("random", "prefix"):
            x = _custom(op, dtype, bs, T, mask, seed=bs + T, lo=0)
            what = f"chunked {op} {dtype} {bs}x{T} {mask} grid={grid} tiles={tiles}"
            print("[parity]", what, flush=True)
            first = assert_policy_parity(op, x, 0.04, 0.2, 0.28, what)
            fwd = assert_policy_parity(op, x, 0.04, 0.2, 0.28, what + " fwd", fused=False)
            assert torch.equal(fwd[0], first[0]), what
    w = synthetic.Workload("edge", "rkl", dtype, "bool", bs, T, 1, T, seed=bs + T)
    x = synthetic.inputs(w)
    x["mask"] = torch.from_numpy(np.random.default_rng(bs + T).random((bs, T)) < 0.6)
    what = f"chunked rkl {dtype} {bs}x{T} random"
    print("[parity]", what, flush=True)
    first = assert_rkl_parity(x, what)
    fwd = assert_rkl_parity(x, what + " fwd", fused=False)
    assert torch.equal(fwd[0], first[0]), what
    assert kinds <= {"one-tile vec16", "stream"}, kinds


# Rows of a few slots in 16-slot lanes: nearly every chunk holds a row end
# (the per-slot path of every lane), in the wide one-tile kernel and the
# striding one; GRPO's tiles then touch hundreds of rows each.
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("bs,T", [(300_000, 7), (2_100_000, 3)])
def test_chunked_lanes_tiny_rows(dtype, bs, T):
    for op in ("bnpo", "grpo"):
        grid, vec, tiles = rl.launch_shape(bs, T, TORCH_DT[dtype], op)
        assert vec == 16, (op, grid, vec, tiles)
        x = _custom(op, dtype, bs, T, "random", seed=bs + T, lo=0)
        what = f"tiny rows {op} {dtype} {bs}x{T} grid={grid} tiles={tiles}"
        print("[parity]", what, flush=True)
        first = assert_policy_parity(op, x, 0.04, 0.2, 0.28, what)
        fwd = assert_policy_parity(op, x, 0.04, 0.2, 0.28, what + " fwd", fused=False)
        assert torch.equal(fwd[0], first[0]), what


def test_striding_sweep_full_rounds_and_remainder():
    # The striding BNPO and reverse-KL workers take groups of eight tiles side
    # by side, then split what is left into one contiguous piece each: 8300 x
    # 4099 has more tiles than eight per worker and a remainder, and rows that
    # cross tiles.
    bs, T = 8300, 4099
    grid, vec, tiles = rl.launch_shape(bs, T, torch.bfloat16, "bnpo")
    assert vec == 16 and tiles >= 8 * grid and tiles % (8 * grid) != 0, (grid, tiles)
    x = _custom("bnpo", "bf16", bs, T, "prefix", seed=7, lo=0)
    what = f"sweep bnpo {bs}x{T} grid={grid} tiles={tiles}"
    print("[parity]", what, flush=True)
    first = assert_policy_parity("bnpo", x, 0.04, 0.2, 0.28, what)
    fwd = assert_policy_parity("bnpo", x, 0.04, 0.2, 0.28, what + " fwd", fused=False)
    assert torch.equal(fwd[0], first[0]), what
    r = {"student": x["policy"], "teacher": x["ref"], "mask": x["mask"] != 0}
    print("[parity] sweep rkl", flush=True)
    assert_rkl_parity(r, "sweep rkl")


# From this many bytes of mask, planes and gradient (whole arrays) on, a
# striding fwd+bwd launch stores its gradient non-temporally (the library's
# kNtGradBytes, 1.25 GiB): these launches take that kernel.
NT_GRAD_BYTES = 5 << 28


def _sample_rows(bs, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, bs - 1], rng.integers(0, bs, 10)]))


@pytest.mark.parametrize("op,name,bs,T", [("bnpo", "bnpo_bf16_64x4096", 40960, 4096),
                                          ("grpo", "grpo_fp16_128x2048", 40960, 4096),
                                          ("rkl", "rkl_bf16_256x8192", 24576, 8192)])
def test_streaming_sizes_non_temporal_gradient(op, name, bs, T):
    # At these sizes the oracle runs on sampled rows alone: each row's gradient
    # depends on the other rows only through the normaliser (the global count
    # for BNPO and reverse KL, the row count for GRPO), so the oracle's rows are
    # rescaled from their own to the launch's.  The loss is checked against the
    # forward-only kernel (the same partition, so bit-equal), the count exactly,
    # and every masked slot's gradient is +0.
    w = synthetic.WORKLOADS[name]
    w = w.with_(bs=bs, seq_len=T, len_lo=min(w.len_lo, T), len_hi=T, name=f"{name}@{bs}x{T}")
    g = synthetic.device_policy_inputs(w, "cuda:0")
    e = g["policy"].element_size()
    planes = 2 if op == "rkl" else 3
    assert bs * T * (1 + planes * e + e) >= NT_GRAD_BYTES
    what = f"non-temporal gradient {op} {bs}x{T}"
    print("[parity]", what, flush=True)
    rows = _sample_rows(bs, bs + T)
    dt = g["policy"].dtype
    if op == "rkl":
        mask = g["mask"] != 0
        loss, grad, n = rl.reverse_kl(g["policy"], g["ref"], mask, return_n_valid=True)
        loss_f, n_f = rl.reverse_kl_fwd(g["policy"], g["ref"], mask, return_n_valid=True)
        torch.cuda.synchronize()
        N = int(torch.count_nonzero(mask))
        assert int(n.cpu()[0]) == N and int(n_f.cpu()[0]) == N, what
        assert torch.equal(loss, loss_f), what
        sub = {"student": g["policy"][rows].cpu(), "teacher": g["ref"][rows].cpu(), "mask": mask[rows].cpu()}
        ref = oracle.rkl(sub["student"], sub["teacher"], sub["mask"])
        want = ref.grad * (max(ref.n_valid, 1) / max(N, 1))
        mag = rkl_grad_magnitude(sub["student"], sub["teacher"], 1.0 / max(N, 1))
        check_grad(grad[rows].cpu(), want, dt, what, mag=mag)
    else:
        out = gpu_policy(op, True, g, w.beta, w.epsilon, w.epsilon_high)
        out_f = gpu_policy(op, False, g, w.beta, w.epsilon, w.epsilon_high)
        loss, grad, n = out
        assert torch.equal(loss, out_f[0]), what
        sub = {k: g[k][rows].cpu() for k in ("policy", "old", "ref", "advantages", "mask")}
        ref = oracle_policy(op, sub, w.beta, w.epsilon, w.epsilon_high)
        if op == "bnpo":
            N = int(torch.count_nonzero(g["mask"]))
            assert int(n.cpu()[0]) == N and int(out_f[-1].cpu()[0]) == N, what
            want = ref.grad * (max(ref.n_valid, 1) / max(N, 1))
            scale = 1.0 / max(N, 1)
        else:
            counts = torch.count_nonzero(g["mask"], dim=1).cpu().numpy().astype(np.int64)
            np.testing.assert_array_equal(n.cpu().numpy().astype(np.int64), counts, err_msg=what)
            np.testing.assert_array_equal(counts[rows], ref.n_valid, err_msg=what)
            want = ref.grad * (len(rows) / bs)
            scale = (1.0 / (np.maximum(ref.n_valid, 1) * bs))[:, None]
        kinks = kink_tokens(sub["policy"], sub["old"], sub["mask"], w.epsilon_high)
        alt = kink_alternative(want, sub["policy"], sub["old"], sub["advantages"], sub["mask"], w.epsilon_high,
                               scale)
        mag = policy_grad_magnitude(sub["policy"], sub["old"], sub["ref"], sub["advantages"], f32(w.beta), scale)
        check_grad(grad[rows].cpu(), want, dt, what, alt, kinks, mag)
        mask = g["mask"] != 0
    bits = grad.view(torch.int16 if e == 2 else torch.int32)
    assert not bool(torch.any(bits[~mask] != 0)), what + ": a masked slot is not +0"


@pytest.mark.parametrize("bs,T", [(2048, 4096), (8192, 1024)])
def test_grpo_striding_kernel_repeats_bitwise(bs, T):
    # Each worker streams several tiles and rebuilds the per-row scales in LDS
    # for every tile: the results must match the oracle and repeat bit for bit.
    grid, vec, tiles = rl.launch_shape(bs, T, torch.bfloat16, "grpo")
    assert tiles >= grid, (grid, tiles)
    x = _custom("grpo", "bf16", bs, T, "prefix", seed=bs + T, lo=0)
    what = f"grpo striding {bs}x{T} grid={grid} tiles={tiles}"
    print("[parity]", what, flush=True)
    first = assert_policy_parity("grpo", x, 0.04, 0.2, 0.28, what)
    g = dev(x)
    for _ in range(3):
        again = gpu_policy("grpo", True, g, 0.04, 0.2, 0.28)
        assert torch.equal(again[0], first[0]) and torch.equal(again[1], first[1]), what


@pytest.mark.parametrize("op", ["bnpo", "grpo"])
@pytest.mark.parametrize("name", ["bnpo_bf16_64x4096", "bnpo_fp32_4x64", "grpo_fp16_128x2048"])
def test_sign_aware_clip(op, name):
    # Standard PPO -min(A*ratio, A*clipped): where A < 0 the lower bound 1-eps clips.
    # old = policy + N(0, 0.3) here, so that ratios fall outside the clip range on both sides.
    w = synthetic.WORKLOADS[name]
    x = synthetic.inputs(w)
    rng = np.random.default_rng(17)
    x["old"] = (x["policy"].double() + 0.3 * torch.from_numpy(rng.standard_normal(tuple(x["policy"].shape)))
                ).to(x["policy"].dtype)
    what = f"sign-aware {op} {name}"
    print("[parity]", what, flush=True)
    assert_policy_parity(op, x, w.beta, w.epsilon, w.epsilon_high, what, clip="sign_aware")
    assert_policy_parity(op, x, w.beta, w.epsilon, w.epsilon_high, what + " fwd", fused=False, clip="sign_aware")
    # eps now changes the result (it never does in the literal form)
    g = dev(x)
    a = gpu_policy(op, True, g, w.beta, 0.1, w.epsilon_high, clip="sign_aware")
    b = gpu_policy(op, True, g, w.beta, 0.3, w.epsilon_high, clip="sign_aware")
    assert not torch.equal(a[0], b[0])
    # and where every advantage is >= 0 it equals the literal form bit for bit
    g["advantages"] = g["advantages"].abs()
    c = gpu_policy(op, True, g, w.beta, w.epsilon, w.epsilon_high, clip="sign_aware")
    d = gpu_policy(op, True, g, w.beta, w.epsilon, w.epsilon_high)
    assert torch.equal(c[0], d[0]) and torch.equal(c[1], d[1])


@pytest.mark.parametrize("bs,T", [(3, 37), (9, 4095), (2, 4097), (40, 1)])
def test_sign_aware_clip_row_crossing_lanes(bs, T):
    x = _custom("bnpo", "bf16", bs, T, "random", seed=bs + T)
    rng = np.random.default_rng(bs)
    x["old"] = (x["policy"].double() + 0.3 * torch.from_numpy(rng.standard_normal((bs, T)))).to(torch.bfloat16)
    x["advantages"] = torch.from_numpy(rng.standard_normal(bs)).to(torch.bfloat16)
    for op in ("bnpo", "grpo"):
        assert_policy_parity(op, x, 0.04, 0.2, 0.28, f"sign-aware {op} {bs}x{T}", clip="sign_aware")


def test_grpo_rows_longer_than_a_tile():
    x = _custom("grpo", "fp16", 6, 50000, "prefix", lo=0)
    assert_policy_parity("grpo", x, 0.04, 0.2, 0.2, "grpo long rows")


# GRPO row counts across tile and worker-run boundaries: rows spanning many
# tiles, rows that do not divide a tile, a single row over the whole launch,
# in the one-tile and the striding kernels (each worker owning a run of tiles),
# with 2 to 5 workers per thread of the workgroup that closes the rows (3 x
# 1,500,000: 1,099 one-tile workers).
GRPO_ROWS = [(16, 131072, "prefix"), (64, 32768, "random"), (1, 1 << 21, "random"), (5, 4099, "random"),
             (64, 100000, "prefix"), (2000, 3000, "random"), (1, 6_000_000, "prefix"), (700, 8192, "random"),
             (3, 1_500_000, "random")]


@pytest.mark.parametrize("bs,T,mask", GRPO_ROWS)
def test_grpo_rows_across_tiles_and_runs(bs, T, mask):
    grid, vec, tiles = rl.launch_shape(bs, T, torch.float16, "grpo")
    x = _custom("grpo", "fp16", bs, T, mask, seed=bs + T, lo=0)
    what = f"grpo rows {bs}x{T} grid={grid} tiles={tiles}"
    print("[parity]", what, flush=True)
    first = assert_policy_parity("grpo", x, 0.04, 0.2, 0.28, what)
    fwd = assert_policy_parity("grpo", x, 0.04, 0.2, 0.28, what + " fwd", fused=False)
    assert torch.equal(fwd[0], first[0]), what
    g = dev(x)
    again = gpu_policy("grpo", True, g, 0.04, 0.2, 0.28)
    assert all(torch.equal(a, b) for a, b in zip(again, first)), what


def test_grpo_one_slot_rows():
    x = _custom("grpo", "bf16", 9000, 1, "random")
    assert_policy_parity("grpo", x, 0.04, 0.2, 0.28, "grpo T=1")


def _all_ops(x_bnpo, x_rkl, ws):
    kw = dict(epsilon=0.2, epsilon_high=0.28, beta=0.04, workspace=ws)
    b = x_bnpo
    out = []
    out += list(rl.bnpo_loss(b["policy"], b["old"], b["ref"], b["advantages"], b["mask"], **kw))
    out += [rl.bnpo_loss_fwd(b["policy"], b["old"], b["ref"], b["advantages"], b["mask"], **kw)]
    out += list(rl.grpo_loss(b["policy"], b["old"], b["ref"], b["advantages"], b["mask"], **kw))
    out += [rl.grpo_loss_fwd(b["policy"], b["old"], b["ref"], b["advantages"], b["mask"], **kw)]
    out += list(rl.reverse_kl(x_rkl["student"], x_rkl["teacher"], x_rkl["mask"], workspace=ws))
    out += [rl.reverse_kl_fwd(x_rkl["student"], x_rkl["teacher"], x_rkl["mask"], workspace=ws)]
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("start_gen", [0, 1, 2**31, 2**32 - 2])
def test_fresh_workspace_first_calls_and_generation_wraparound(start_gen):
    # Every op's first use of a zero-filled workspace, and launches across the 32-bit
    # generation wrap, give bit-identical results to calls on a long-used workspace.
    xb = dev(synthetic.inputs(synthetic.WORKLOADS["bnpo_bf16_64x4096"]))
    xr = dev(synthetic.inputs(synthetic.Workload("w", "rkl", "bf16", "bool", 64, 4096, 1, 4096)))
    ref = _all_ops(xb, xr, None)
    nbytes = rl.library().rlpl_workspace_bytes(64, 4096, 0)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    ws[0:4].view(torch.int32)[0] = start_gen - 2**32 if start_gen >= 2**31 else start_gen
    for _ in range(3):
        got = _all_ops(xb, xr, ws)
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
    assert int(ws[256:260].cpu().view(torch.int32)[0]) == 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_non_finite_values_in_masked_slots_change_nothing(dtype):
    # Masked slots are computed with everything else and selected away: NaN or inf
    # there must not reach the loss, the gradient or the counts.
    x = _custom("bnpo", dtype, 7, 1000, "random", seed=77)
    xr = {"student": x["policy"].clone(), "teacher": x["ref"].clone(), "mask": x["mask"]}
    poisoned = {k: v.clone() for k, v in x.items() if isinstance(v, torch.Tensor)}
    masked = x["mask"] == 0
    for k, val in (("policy", float("nan")), ("old", float("inf")), ("ref", float("-inf"))):
        poisoned[k][masked] = val
    a, b = dev(x), dev(poisoned)
    kw = dict(epsilon=0.2, epsilon_high=0.28, beta=0.04)
    for fn in (rl.bnpo_loss, rl.grpo_loss):
        o1 = fn(a["policy"], a["old"], a["ref"], a["advantages"], a["mask"], **kw)
        o2 = fn(b["policy"], b["old"], b["ref"], b["advantages"], b["mask"], **kw)
        assert torch.equal(o1[0], o2[0]) and torch.equal(o1[1], o2[1])
    pr = dev(xr)
    pp = {"student": b["policy"], "teacher": b["ref"], "mask": b["mask"]}
    o1 = rl.reverse_kl(pr["student"], pr["teacher"], pr["mask"])
    o2 = rl.reverse_kl(pp["student"], pp["teacher"], pp["mask"])
    assert torch.equal(o1[0], o2[0]) and torch.equal(o1[1], o2[1])
