"""Parity of the full-vocab reverse-KL kernels (through the C ABI binding) with
the CPU oracle (model card "Geometric-AI Kernels", section "Reverse KL").

Tolerances, from the kernels' float32 arithmetic:

* loss: relative 1e-5 for fp32 logits, 1e-3 for fp16/bf16 (as for the
  per-token losses);
* gradient, per element: 2 ulp of the output dtype at the oracle's value,
  plus p_v * (R_r * |d_v - E_p[d]| + 8 * 2^-24 * (|d_v| + |E_p[d]|)) / N, where
  d = s - t.  R_r bounds the relative error of p_v = exp(s_v - lse_s) that
  comes from the float32 row sums behind lse_s (a lane adds about V/1024
  terms per accumulator, then 10 merges) and from rounding lse_s:
  R_r = (V/1024 + 16 + 4 * |lse_s|) * 2^-24.  The second term is the
  evaluation bound of d_v - E_p[d] where the two cancel.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import rl_post_loss_amd as rl
import synthetic
from parity import check_loss, ulp

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
EPS32 = 2.0 ** -24


def _row_terms(s, t):
    """(p, d, E_p[d], lse_s) of each row, float64 (test-side, to size the allowance)."""
    m = s.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
    p = np.exp(s - lse)
    d = s - t
    ed = (p * d).sum(axis=1, keepdims=True)
    return p, d, ed, lse


def check_vocab_grad(got_t, want, s, t, n_valid, dtype, what):
    got = got_t.detach().cpu().to(torch.float64).numpy().reshape(want.shape)
    V = s.shape[1]
    p, d, ed, lse = _row_terms(s, t)
    R = (V / 1024.0 + 16.0 + 4.0 * np.abs(lse)) * EPS32
    inv = 1.0 / n_valid
    allow = 2.0 * ulp(want, dtype) + inv * p * (R * np.abs(d - ed) + 8.0 * EPS32 * (np.abs(d) + np.abs(ed)))
    err = np.abs(got - want)
    bad = err > allow
    if bad.any():
        i = np.unravel_index(np.argmax(err / allow), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} gradient elements out of tolerance; "
                             f"worst at {i}: got {got[i]!r} oracle {want[i]!r} (allowed {allow[i]:.3e})")


def assert_vocab_parity(x, what, fused=True):
    s64, t64 = oracle.to_f64(x["student"]), oracle.to_f64(x["teacher"])
    m = oracle.to_mask_u8(x["mask"])
    ref = oracle.rkl_logits(s64, t64, m, grad=fused)
    g = {k: v.to(DEV) for k, v in x.items()}
    dt = x["student"].dtype
    if fused:
        loss, grad, n = rl.reverse_kl_logits(g["student"], g["teacher"], g["mask"], return_n_valid=True)
    else:
        loss, n = rl.reverse_kl_logits_fwd(g["student"], g["teacher"], g["mask"], return_n_valid=True)
    torch.cuda.synchronize()
    assert int(n.cpu()[0]) == ref.n_valid, what
    check_loss(float(loss.cpu()), ref.loss, dt, what)
    if fused:
        assert grad.dtype == dt and grad.shape == x["student"].shape
        valid = m.reshape(-1) != 0
        s2, t2 = s64.reshape(-1, s64.shape[-1]), t64.reshape(-1, t64.shape[-1])
        gw = ref.grad.reshape(s2.shape)
        gg = grad.reshape(s2.shape)
        if valid.any():
            check_vocab_grad(gg[torch.from_numpy(valid).to(DEV)], gw[valid], s2[valid], t2[valid],
                             ref.n_valid, dt, what)
        z = gg[torch.from_numpy(~valid).to(DEV)].float().cpu()
        assert torch.all(z == 0) and not torch.any(torch.signbit(z)), f"{what}: masked rows not +0"
    return loss, (grad if fused else None)


SHAPES = [(1, 1), (1, 7), (3, 8), (5, 9), (4, 1000), (7, 4097), (3, 32000), (9, 50257), (2, 65536)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("rows,V", SHAPES)
def test_vocab_shapes(dtype, rows, V):
    x = synthetic.vocab_inputs(rows, V, dtype, "int8" if rows % 2 else "bool", seed=rows * 7 + V,
                               p_valid=0.8 if rows > 2 else 1.0)
    what = f"rkl_logits {dtype} {rows}x{V}"
    print("[parity]", what, flush=True)
    a, _ = assert_vocab_parity(x, what)
    b, _ = assert_vocab_parity(x, what + " fwd", fused=False)
    assert a.cpu().view(torch.int32).item() == b.cpu().view(torch.int32).item()


def test_vocab_many_rows_per_workgroup():
    x = synthetic.vocab_inputs(6000, 384, "bf16", "bool", seed=3)
    grid, vec, tiles = rl.launch_shape(6000, 384, torch.bfloat16, "rkl_logits")
    assert tiles == 6000 and grid < tiles
    print(f"[parity] rkl_logits 6000x384 grid={grid}", flush=True)
    assert_vocab_parity(x, "rkl_logits 6000x384")


@pytest.mark.parametrize("dtype,rows,V", [("bf16", 1, 248320), ("bf16", 3, 100000), ("fp16", 5, 50257),
                                          ("fp32", 2, 70001), ("bf16", 64, 40000)])
def test_vocab_rows_split_across_workgroups(dtype, rows, V):
    # Few rows: each row is split among several workgroups that exchange their
    # softmax sums (misaligned rows and a ragged last piece included).
    grid, vec, tiles = rl.launch_shape(rows, V, synthetic.DTYPES[dtype], "rkl_logits")
    assert tiles > rows, (grid, tiles)
    x = synthetic.vocab_inputs(rows, V, dtype, "bool", seed=rows + V, p_valid=1.0 if rows < 3 else 0.8)
    what = f"rkl_logits split {dtype} {rows}x{V} grid={grid} pieces={tiles // rows}"
    print("[parity]", what, flush=True)
    a, ga = assert_vocab_parity(x, what)
    b, _ = assert_vocab_parity(x, what + " fwd", fused=False)
    assert a.cpu().view(torch.int32).item() == b.cpu().view(torch.int32).item()
    g = {k: v.to(DEV) for k, v in x.items()}
    for _ in range(2):
        c = rl.reverse_kl_logits(g["student"], g["teacher"], g["mask"])
        assert torch.equal(c[0], a) and torch.equal(c[1], ga)


@pytest.mark.parametrize("dtype,rows,V", [("bf16", 2, 4_300_000), ("fp32", 1, 2_200_001)])
def test_vocab_long_pieces_read_twice(dtype, rows, V):
    # Rows so long that, at the largest number of pieces per row, a piece is
    # longer than the 1024 32-byte blocks a workgroup keeps in registers: the
    # fused kernel then reads its piece a second time for the gradient.
    grid, vec, tiles = rl.launch_shape(rows, V, synthetic.DTYPES[dtype], "rkl_logits")
    chunks = tiles // rows
    blocks = V // vec if V % vec == 0 else V // vec + 2
    assert -(-blocks // chunks) > 1024, (chunks, blocks)
    x = synthetic.vocab_inputs(rows, V, dtype, "bool", seed=V % 1000, p_valid=1.0)
    what = f"rkl_logits long pieces {dtype} {rows}x{V} pieces={chunks}"
    print("[parity]", what, flush=True)
    a, _ = assert_vocab_parity(x, what)
    b, _ = assert_vocab_parity(x, what + " fwd", fused=False)
    assert a.cpu().view(torch.int32).item() == b.cpu().view(torch.int32).item()


def test_vocab_leading_dims_and_shifted_logits():
    x = synthetic.vocab_inputs(24, 3000, "fp32", "bool", seed=4)
    x = {"student": (x["student"] + 40.0).reshape(2, 3, 4, 3000),
         "teacher": (x["teacher"] - 25.0).reshape(2, 3, 4, 3000),
         "mask": x["mask"].reshape(2, 3, 4)}
    assert_vocab_parity(x, "rkl_logits (2,3,4,3000) shifted")


def test_vocab_all_rows_masked():
    x = synthetic.vocab_inputs(5, 700, "bf16", "bool", seed=5)
    x["mask"] = torch.zeros(5, dtype=torch.bool)
    g = {k: v.to(DEV) for k, v in x.items()}
    loss, grad, n = rl.reverse_kl_logits(g["student"], g["teacher"], g["mask"], return_n_valid=True)
    torch.cuda.synchronize()
    assert math.isnan(float(loss.cpu())) and int(n.cpu()[0]) == 0
    z = grad.float().cpu()
    assert torch.all(z == 0) and not torch.any(torch.signbit(z))


def test_vocab_masked_rows_are_never_read():
    x = synthetic.vocab_inputs(8, 2049, "fp16", "int8", seed=6)
    x["mask"] = torch.tensor([1, 0, 1, 1, 0, 1, 0, 1], dtype=torch.int8)
    ref = assert_vocab_parity(x, "rkl_logits masked rows")
    y = dict(x)
    y["student"], y["teacher"] = x["student"].clone(), x["teacher"].clone()
    for r in (1, 4, 6):
        y["student"][r] = float("nan")
        y["teacher"][r] = float("inf")
    g = {k: v.to(DEV) for k, v in y.items()}
    loss, grad = rl.reverse_kl_logits(g["student"], g["teacher"], g["mask"])
    torch.cuda.synchronize()
    assert torch.equal(loss, ref[0]) and torch.equal(grad, ref[1])


def test_vocab_repeats_bitwise():
    x = {k: v.to(DEV) for k, v in synthetic.vocab_inputs(300, 4096, "bf16", "bool", seed=7).items()}
    a = rl.reverse_kl_logits(x["student"], x["teacher"], x["mask"])
    for _ in range(3):
        b = rl.reverse_kl_logits(x["student"], x["teacher"], x["mask"])
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_vocab_card_example_size_sampled_rows():
    # The card's example shape: (4, 256, 248320) bf16 logits, mask = rand > 0.2.
    # The loss is checked against the oracle over the whole slab, the gradient
    # element by element on sampled rows (the oracle on each row alone, rescaled
    # by 1/N).
    rows, V = 4 * 256, 248320
    x = synthetic.vocab_inputs(rows, V, "bf16", "bool", seed=11)
    print("[parity] rkl_logits card example 4x256x248320 bf16", flush=True)
    g = {k: v.to(DEV) for k, v in x.items()}
    loss, grad, n = rl.reverse_kl_logits(g["student"].view(4, 256, V), g["teacher"].view(4, 256, V),
                                         g["mask"].view(4, 256), return_n_valid=True)
    fwd = rl.reverse_kl_logits_fwd(g["student"], g["teacher"], g["mask"])
    torch.cuda.synchronize()
    # Here the fused kernel splits each row into pieces of ~1024 blocks and the
    # forward-only kernel reads whole rows, so their float32 sums differ in
    # order: each is within about (V/1024 + 64) * 2^-24 (relative, per row, of
    # the row's softmax sums and so of kl_r) of the exact loss; doubled for the
    # difference of the two, and again as margin.
    bound = 4 * (V / 1024 + 64) * 2.0 ** -24
    assert abs(float(loss) - float(fwd)) <= bound * abs(float(loss)), (float(loss), float(fwd), bound)
    m = oracle.to_mask_u8(x["mask"])
    ref = oracle.rkl_logits(x["student"], x["teacher"], m, grad=False)
    assert int(n.cpu()[0]) == ref.n_valid
    check_loss(float(loss.cpu()), ref.loss, torch.bfloat16, "card example")
    grad = grad.view(rows, V)
    rng = np.random.default_rng(12)
    valid_rows = np.flatnonzero(m)
    masked_rows = np.flatnonzero(m == 0)
    for r in list(rng.choice(valid_rows, 6, replace=False)) + [int(valid_rows[-1])]:
        s64, t64 = oracle.to_f64(x["student"][r:r + 1]), oracle.to_f64(x["teacher"][r:r + 1])
        one = oracle.rkl_logits(s64, t64, np.ones(1, dtype=np.uint8))
        check_vocab_grad(grad[r:r + 1], one.grad / ref.n_valid, s64, t64, ref.n_valid, torch.bfloat16,
                         f"card example row {r}")
    for r in rng.choice(masked_rows, 3, replace=False):
        z = grad[int(r)].float().cpu()
        assert torch.all(z == 0) and not torch.any(torch.signbit(z))
