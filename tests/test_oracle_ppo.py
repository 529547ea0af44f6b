"""Pins of the sign-aware PPO form of per_token in the oracle:
per_token = -min(A*ratio, A*clip(ratio, 1-eps, 1+eps_high)), the standard PPO
clipped objective that the model card ("Geometric-AI Kernels", section "BNPO
Loss") calls PPO-clipped, with the card's BNPO and GRPO normalisations.

Checked against the hand-worked example (tests/golden), the literal form
(identical wherever A >= 0), single-token closed forms of both clip branches
for A < 0, the dependence on eps that only this form has, and central finite
differences.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def ev(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"ln": math.log, "nan": float("nan")}))


def small(op="bnpo", bs=6, T=11, seed=4):
    w = synthetic.Workload("tiny", op, "fp32", "int8", bs, T, 0, T, seed=seed)
    x = synthetic.inputs(w)
    return {k: oracle.to_f64(v) if k != "mask" else oracle.to_mask_u8(v) for k, v in x.items() if k != "lengths"}


def test_golden_sign_aware_example():
    g = json.load(open(GOLDEN))["policy"]
    lp = np.array([[ev(v) for v in row] for row in g["lp"]])
    delta = np.array([[ev(v) for v in row] for row in g["delta"]])
    x = np.array([[ev(v) for v in row] for row in g["x"]])
    adv = np.array([ev(v) for v in g["advantages"]])
    mask = np.array(g["mask"], dtype=np.uint8)
    args = (lp, lp - delta, lp + x, adv, mask, g["beta"], g["epsilon"], g["epsilon_high"])
    for name, fn in (("bnpo_sign_aware", oracle.bnpo), ("grpo_sign_aware", oracle.grpo)):
        exp_ = g[name]
        assert ev(exp_["loss"]) == pytest.approx(exp_["loss_value"], rel=1e-15)
        r = fn(*args, sign_aware=True)
        assert r.loss == pytest.approx(exp_["loss_value"], rel=1e-12, abs=1e-14), name
        want = np.array([[ev(v) for v in row] for row in exp_["grad"]])
        np.testing.assert_allclose(r.grad, want, rtol=1e-12, atol=1e-14, err_msg=name)
        np.testing.assert_array_equal(np.atleast_1d(r.n_valid), np.atleast_1d(exp_["n_valid"]))


@pytest.mark.parametrize("fn", [oracle.bnpo, oracle.grpo])
def test_equals_the_literal_form_where_advantages_are_non_negative(fn):
    x = small()
    adv = np.abs(x["advantages"])
    a = fn(x["policy"], x["old"], x["ref"], adv, x["mask"], 0.04, 0.2, 0.28)
    b = fn(x["policy"], x["old"], x["ref"], adv, x["mask"], 0.04, 0.2, 0.28, sign_aware=True)
    assert a.loss == b.loss and np.array_equal(a.grad, b.grad)


@pytest.mark.parametrize("delta,term,slope", [
    (math.log(0.5), 0.8, 0.0),      # ratio below 1-eps: the clipped objective, a constant
    (math.log(2.0), 2.0, 2.0),      # ratio above 1+eps_high: unclipped for A < 0
    (math.log(1.1), 1.1, 1.1),      # inside the clip range
])
def test_single_token_closed_forms_for_negative_advantage(delta, term, slope):
    lp = np.array([[-0.3]])
    old = lp - delta
    r = oracle.bnpo(lp, old, None, np.array([-1.0]), np.array([[1]], dtype=np.uint8), 0.0, 0.2, 0.28,
                    sign_aware=True)
    assert r.loss == pytest.approx(term, rel=1e-13)
    assert r.grad[0, 0] == pytest.approx(slope, rel=1e-13, abs=0)
    lit = oracle.bnpo(lp, old, None, np.array([-1.0]), np.array([[1]], dtype=np.uint8), 0.0, 0.2, 0.28)
    assert lit.loss == pytest.approx(min(math.exp(delta), 1.28), rel=1e-13)


def test_eps_matters_only_in_the_sign_aware_form():
    x = small(bs=8, T=40, seed=9)
    # widen the ratios so that some fall below 1 - eps
    old = x["policy"] - 0.5 * np.random.default_rng(1).standard_normal(x["policy"].shape)
    adv = -np.abs(x["advantages"])
    args = (x["policy"], old, x["ref"], adv, x["mask"], 0.04)
    lit = [oracle.bnpo(*args, e, 0.28).loss for e in (0.1, 0.3)]
    sa = [oracle.bnpo(*args, e, 0.28, sign_aware=True).loss for e in (0.1, 0.3)]
    assert lit[0] == lit[1]
    assert sa[0] != sa[1]


@pytest.mark.parametrize("op", ["bnpo", "grpo"])
def test_sign_aware_gradient_matches_finite_differences(op):
    x = small(op, bs=3, T=5, seed=5)
    fn = oracle.bnpo if op == "bnpo" else oracle.grpo
    old = x["policy"] - 0.4 * np.random.default_rng(2).standard_normal(x["policy"].shape)
    adv = np.array([-1.5, 0.7, -0.4])
    args = lambda lp: (lp, old, x["ref"], adv, x["mask"], 0.04, 0.2, 0.28)
    r = fn(*args(x["policy"]), sign_aware=True)
    h = 1e-6
    fd = np.zeros_like(x["policy"])
    for i in np.ndindex(fd.shape):
        lp_p, lp_m = x["policy"].copy(), x["policy"].copy()
        lp_p[i] += h
        lp_m[i] -= h
        fd[i] = (fn(*args(lp_p), grad=False, sign_aware=True).loss
                 - fn(*args(lp_m), grad=False, sign_aware=True).loss) / (2 * h)
    np.testing.assert_allclose(r.grad, fd, rtol=1e-5, atol=1e-8)
