"""Pins of the CPU oracle against what the model card and the mathematics fix.

None of these re-types the oracle's formula: each checks a closed form, an
invariant, a hand-worked example, central finite differences, or an exact
count.  A dropped term, a wrong sign or row index, a swapped operand
(lp - old vs old - lp, ref - lp vs lp - ref), the wrong clip bound or the wrong
normaliser each fails at least one test below.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def ev(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"ln": math.log, "nan": float("nan")}))


def small(op="bnpo", bs=5, T=13, seed=3, **kw):
    w = synthetic.Workload("tiny", op, "fp32", "int8", bs, T, 0, T, seed=seed, **kw)
    return synthetic.inputs(w)


# --------------------------------------------------------------------------- hand-worked example

def test_golden_policy_example_bnpo_and_grpo():
    g = json.load(open(GOLDEN))["policy"]
    lp = np.array([[ev(v) for v in row] for row in g["lp"]])
    delta = np.array([[ev(v) for v in row] for row in g["delta"]])
    x = np.array([[ev(v) for v in row] for row in g["x"]])
    old, ref = lp - delta, lp + x
    adv = np.array([ev(v) for v in g["advantages"]])
    mask = np.array(g["mask"], dtype=np.uint8)
    args = (lp, old, ref, adv, mask, g["beta"], g["epsilon"], g["epsilon_high"])
    for name, fn in (("bnpo", oracle.bnpo), ("grpo", oracle.grpo)):
        exp_ = g[name]
        assert ev(exp_["loss"]) == pytest.approx(exp_["loss_value"], rel=1e-15)
        r = fn(*args)
        assert r.loss == pytest.approx(ev(exp_["loss"]), rel=1e-12, abs=1e-14), name
        want = np.array([[ev(v) for v in row] for row in exp_["grad"]])
        np.testing.assert_allclose(r.grad, want, rtol=1e-12, atol=1e-14, err_msg=name)
        assert np.all(np.isfinite(r.grad))
        np.testing.assert_array_equal(np.atleast_1d(r.n_valid), np.atleast_1d(exp_["n_valid"]))


def test_golden_rkl_example():
    g = json.load(open(GOLDEN))["rkl"]
    s = np.array([[ev(v) for v in row] for row in g["student"]])
    t = s + np.array([[ev(v) for v in row] for row in g["x"]])
    m = np.array(g["mask"], dtype=np.uint8)
    r = oracle.rkl(s, t, m)
    assert r.loss == pytest.approx(ev(g["loss"]), rel=1e-12)
    want = np.array([[ev(v) for v in row] for row in g["grad"]])
    np.testing.assert_allclose(r.grad, want, rtol=1e-12, atol=1e-15)
    assert r.n_valid == g["n_valid"]


# --------------------------------------------------------------------------- closed forms

def _ratio_one_inputs(bs=6, T=11, seed=7):
    rng = np.random.default_rng(seed)
    lp = -np.abs(rng.standard_normal((bs, T)))
    adv = rng.standard_normal(bs)
    lengths = np.array([0, 1, T, 4, 7, 2])[:bs]
    mask = (np.arange(T)[None, :] < lengths[:, None]).astype(np.uint8)
    return lp, adv, lengths, mask


def test_ratio_one_bnpo_closed_form():
    # old == lp gives ratio 1 inside [1-eps, 1+eps_high], so per_token = -A_r.
    lp, adv, n, mask = _ratio_one_inputs()
    r = oracle.bnpo(lp, lp.copy(), None, adv, mask, 0.0, 0.2, 0.28)
    N = n.sum()
    assert r.loss == pytest.approx(-(adv * n).sum() / max(N, 1), rel=1e-13)
    np.testing.assert_allclose(r.grad, -adv[:, None] * mask / max(N, 1), rtol=1e-13, atol=0)
    assert r.n_valid == N


def test_ratio_one_grpo_closed_form():
    lp, adv, n, mask = _ratio_one_inputs()
    bs = len(adv)
    r = oracle.grpo(lp, lp.copy(), None, adv, mask, 0.0, 0.2, 0.28)
    # mean over all bs rows; a fully-masked row (n=0) adds 0 but still counts.
    assert r.loss == pytest.approx(-(adv[n > 0]).sum() / bs, rel=1e-13)
    D = np.maximum(n, 1)
    np.testing.assert_allclose(r.grad, -adv[:, None] * mask / (D[:, None] * bs), rtol=1e-13, atol=0)
    np.testing.assert_array_equal(r.n_valid, n)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_clip_branches(sign):
    # ratio 2 (> 1+eps_high) is clipped to 1+eps_high with zero slope; ratio 1/2 and 1.1
    # stay unclipped with slope -A*ratio.  eps != eps_high so the bounds cannot be confused.
    eps, eps_high = 0.15, 0.3
    A = sign * 1.75
    lp = np.array([[-0.4, -1.1, -0.9]])
    delta = np.array([[math.log(2.0), math.log(0.5), math.log(1.1)]])
    mask = np.ones((1, 3), np.uint8)
    r = oracle.bnpo(lp, lp - delta, None, np.array([A]), mask, 0.0, eps, eps_high)
    pt = np.array([-A * (1 + eps_high), -A * 0.5, -A * 1.1])
    slope = np.array([0.0, -A * 0.5, -A * 1.1])
    assert r.loss == pytest.approx(pt.sum() / 3, rel=1e-13)
    np.testing.assert_allclose(r.grad[0], slope / 3, rtol=1e-13, atol=1e-16)


def test_lower_clip_bound_has_no_effect_literal_reading():
    # min(ratio, clip(ratio, 1-eps, 1+eps_high)) == min(ratio, 1+eps_high): eps never matters.
    d = small(bs=4, T=9)
    old = d["old"].double() - 0.5 * torch.sign(torch.randn(4, 9, generator=torch.Generator().manual_seed(1)))
    base = oracle.bnpo(d["policy"], old, d["ref"], d["advantages"], d["mask"], 0.04, 0.2, 0.28)
    for eps in (0.0, 0.05, 0.5, 0.9):
        r = oracle.bnpo(d["policy"], old, d["ref"], d["advantages"], d["mask"], 0.04, eps, 0.28)
        assert r.loss == base.loss
        np.testing.assert_array_equal(r.grad, base.grad)


def test_kl_single_token_closed_form():
    # One valid token, ratio 1, A = 0: loss = beta*(e^x - x - 1), grad = beta*(1 - e^x).
    beta = 0.5
    for x, kl, g in ((math.log(3.0), 2 - math.log(3.0), 1 - 3.0),
                     (-math.log(3.0), 1 / 3 + math.log(3.0) - 1, 1 - 1 / 3)):
        lp = np.array([[-0.7, -0.2]])
        mask = np.array([[1, 0]], np.uint8)
        r = oracle.bnpo(lp, lp.copy(), lp + x, np.array([0.0]), mask, beta, 0.2, 0.28)
        assert r.loss == pytest.approx(beta * kl, rel=1e-13)
        assert r.grad[0, 0] == pytest.approx(beta * g, rel=1e-13)
        assert r.grad[0, 1] == 0.0


def test_kl_vanishes_when_ref_equals_policy_and_is_nonnegative():
    d = small(bs=4, T=10)
    lp = d["policy"].double()
    for fn in (oracle.bnpo, oracle.grpo):
        r0 = fn(lp, d["old"], None, d["advantages"], d["mask"], 0.0, 0.2, 0.28)
        rb = fn(lp, d["old"], lp.clone(), d["advantages"], d["mask"], 0.3, 0.2, 0.28)
        assert rb.loss == pytest.approx(r0.loss, rel=1e-14, abs=1e-15)
        np.testing.assert_allclose(rb.grad, r0.grad, rtol=1e-14, atol=1e-16)
        rk = fn(lp, d["old"], d["ref"], d["advantages"], d["mask"], 0.3, 0.2, 0.28)
        assert rk.loss >= r0.loss  # kl >= 0 per token


def test_beta_linearity():
    d = small(bs=5, T=12)
    for fn in (oracle.bnpo, oracle.grpo):
        a = [fn(d["policy"], d["old"], d["ref"], d["advantages"], d["mask"], b, 0.2, 0.28)
             for b in (0.0, 1.0, 0.37)]
        assert a[2].loss == pytest.approx(a[0].loss + 0.37 * (a[1].loss - a[0].loss), rel=1e-12)
        np.testing.assert_allclose(a[2].grad, a[0].grad + 0.37 * (a[1].grad - a[0].grad),
                                   rtol=1e-11, atol=1e-15)


def test_all_masked():
    d = small(bs=3, T=7)
    z = torch.zeros(3, 7, dtype=torch.int8)
    for fn in (oracle.bnpo, oracle.grpo):
        r = fn(d["policy"], d["old"], d["ref"], d["advantages"], z, 0.04, 0.2, 0.28)
        assert r.loss == 0.0
        assert np.all(r.grad == 0.0) and not np.any(np.signbit(r.grad))
        assert np.all(np.atleast_1d(r.n_valid) == 0)
    e = synthetic.rkl_inputs(synthetic.Workload("t", "rkl", "fp32", "bool", 3, 7, 1, 7))
    r = oracle.rkl(e["student"], e["teacher"], torch.zeros(3, 7, dtype=torch.bool))
    assert math.isnan(r.loss)      # unclamped 1/sum(mask): 0/0
    assert np.all(r.grad == 0.0) and not np.any(np.signbit(r.grad))


def test_bnpo_equals_grpo_when_rows_have_equal_counts():
    d = small(bs=4, T=9)
    mask = torch.zeros(4, 9, dtype=torch.int8)
    for r_, cols in enumerate(([0, 1, 2, 3], [1, 3, 5, 7], [5, 6, 7, 8], [0, 2, 4, 8])):
        mask[r_, cols] = 1
    a = oracle.bnpo(d["policy"], d["old"], d["ref"], d["advantages"], mask, 0.04, 0.2, 0.28)
    b = oracle.grpo(d["policy"], d["old"], d["ref"], d["advantages"], mask, 0.04, 0.2, 0.28)
    assert a.loss == pytest.approx(b.loss, rel=1e-13)
    np.testing.assert_allclose(a.grad, b.grad, rtol=1e-13, atol=1e-17)


def test_bnpo_differs_from_grpo_when_counts_differ():
    d = small(bs=2, T=8)
    mask = torch.tensor([[1, 0, 0, 0, 0, 0, 0, 0], [1, 1, 1, 1, 1, 1, 1, 1]], dtype=torch.int8)
    a = oracle.bnpo(d["policy"], d["old"], d["ref"], d["advantages"], mask, 0.04, 0.2, 0.28)
    b = oracle.grpo(d["policy"], d["old"], d["ref"], d["advantages"], mask, 0.04, 0.2, 0.28)
    assert abs(a.loss - b.loss) > 1e-3


def test_row_permutation_invariance():
    d = small(bs=6, T=8)
    perm = torch.tensor([3, 0, 5, 1, 4, 2])
    for fn in (oracle.bnpo, oracle.grpo):
        a = fn(d["policy"], d["old"], d["ref"], d["advantages"], d["mask"], 0.04, 0.2, 0.28)
        b = fn(d["policy"][perm], d["old"][perm], d["ref"][perm], d["advantages"][perm],
               d["mask"][perm], 0.04, 0.2, 0.28)
        assert b.loss == pytest.approx(a.loss, rel=1e-13, abs=1e-16)
        np.testing.assert_allclose(b.grad, a.grad[perm.numpy()], rtol=1e-13, atol=1e-17)
    e = synthetic.rkl_inputs(synthetic.Workload("t", "rkl", "fp32", "bool", 6, 8, 1, 8))
    a = oracle.rkl(e["student"], e["teacher"], e["mask"])
    b = oracle.rkl(e["student"][perm], e["teacher"][perm], e["mask"][perm])
    assert b.loss == pytest.approx(a.loss, rel=1e-13)


def test_sum_of_grad_equals_loss_without_clipping():
    # beta = 0 and no ratio above 1+eps_high: d per_token / d lp = per_token (d ratio = ratio),
    # so sum(grad) == loss for BNPO and for GRPO.
    d = small(bs=4, T=10)
    for fn in (oracle.bnpo, oracle.grpo):
        r = fn(d["policy"], d["old"], None, d["advantages"], d["mask"], 0.0, 0.2, 10.0)
        assert r.grad.sum() == pytest.approx(r.loss, rel=1e-12, abs=1e-15)


# --------------------------------------------------------------------------- finite differences

def _fd_check(loss_fn, lp, skip, h=1e-6, rtol=1e-6):
    base_grad = loss_fn(lp)[1]
    checked = 0
    for idx in np.ndindex(lp.shape):
        if skip[idx]:
            continue
        p, m = lp.copy(), lp.copy()
        p[idx] += h
        m[idx] -= h
        fd = (loss_fn(p)[0] - loss_fn(m)[0]) / (2 * h)
        assert fd == pytest.approx(base_grad[idx], rel=rtol, abs=1e-9), idx
        checked += 1
    return checked


@pytest.mark.parametrize("which", ["bnpo", "grpo"])
def test_policy_grad_matches_central_differences(which):
    fn = oracle.bnpo if which == "bnpo" else oracle.grpo
    rng = np.random.default_rng(11)
    bs, T = 3, 8
    lp = -np.abs(rng.standard_normal((bs, T)))
    old = lp - rng.normal(0, 0.25, (bs, T))        # some ratios above 1+eps_high
    ref = lp + rng.normal(0, 0.3, (bs, T))
    adv = rng.standard_normal(bs)
    mask = (rng.random((bs, T)) > 0.3).astype(np.uint8)
    hi = 1.28
    near_kink = np.abs(np.exp(lp - old) - hi) < 1e-3
    f = lambda x: (lambda r: (r.loss, r.grad))(fn(x, old, ref, adv, mask, 0.07, 0.2, 0.28))
    assert _fd_check(f, lp, near_kink) >= bs * T - 2
    assert np.any(np.exp(lp - old) > hi) and np.any(np.exp(lp - old) < hi)


def test_rkl_grad_matches_central_differences():
    rng = np.random.default_rng(12)
    s = -np.abs(rng.standard_normal((3, 8)))
    t = s + rng.normal(0, 0.3, (3, 8))
    mask = (rng.random((3, 8)) > 0.3).astype(np.uint8)
    f = lambda x: (lambda r: (r.loss, r.grad))(oracle.rkl(x, t, mask))
    assert _fd_check(f, s, np.zeros_like(mask, dtype=bool)) == 24


# --------------------------------------------------------------------------- counts and masks

def test_counts_exact_and_int8_nonzero_is_valid():
    d = small(bs=6, T=16)
    m = d["mask"].clone()
    m[0, 0] = -3
    m[1, 5] = 7          # any nonzero byte is a valid token
    r = oracle.bnpo(d["policy"], d["old"], d["ref"], d["advantages"], m, 0.04, 0.2, 0.28)
    assert r.n_valid == int(np.count_nonzero(m.numpy()))
    g = oracle.grpo(d["policy"], d["old"], d["ref"], d["advantages"], m, 0.04, 0.2, 0.28)
    np.testing.assert_array_equal(g.n_valid, np.count_nonzero(m.numpy(), axis=1))
    r1 = oracle.bnpo(d["policy"], d["old"], d["ref"], d["advantages"], (m != 0).to(torch.int8),
                     0.04, 0.2, 0.28)
    assert r1.loss == r.loss
    np.testing.assert_array_equal(r1.grad, r.grad)


def test_masked_slots_never_read():
    d = small(bs=3, T=6)
    lp, old, ref = d["policy"].double(), d["old"].double(), d["ref"].double()
    m = d["mask"]
    for a in (lp, old, ref):
        a[m == 0] = float("nan")
    r = oracle.bnpo(lp, old, ref, d["advantages"], m, 0.04, 0.2, 0.28)
    assert math.isfinite(r.loss) and np.all(np.isfinite(r.grad))


# --------------------------------------------------------------------------- generator

def test_generator_is_deterministic_and_matches_recipe():
    w = synthetic.WORKLOADS["grpo_fp16_128x2048"]
    a, b = synthetic.inputs(w), synthetic.inputs(w)
    for k in ("policy", "old", "ref", "advantages", "mask"):
        assert torch.equal(a[k], b[k])
    assert a["policy"].dtype == torch.float16 and a["mask"].dtype == torch.int8
    assert (a["policy"] <= 0).all()
    n = a["mask"].sum(1)
    assert int((n == 0).sum()) == 6                      # round(0.05 * 128) fully masked rows
    c = synthetic.inputs(w.with_(seed=1))
    assert not torch.equal(a["policy"], c["policy"])
    w3 = synthetic.WORKLOADS["bnpo_bf16_64x4096"]
    l3 = synthetic.inputs(w3)["lengths"]
    assert l3.min() >= 256 and l3.max() <= 4096
    e = synthetic.inputs(synthetic.WORKLOADS["rkl_bf16_256x8192"])
    assert e["mask"].dtype == torch.bool and e["student"].dtype == torch.bfloat16
    assert int(e["mask"].sum(1).min()) >= 1024
