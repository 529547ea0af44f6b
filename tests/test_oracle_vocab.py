"""Pins of the full-vocab reverse-KL oracle (model card "Geometric-AI Kernels",
section "Reverse KL"): p = softmax(student), q = softmax(teacher) per row,
kl_row = sum_v p_v (log p_v - log q_v), loss = (mask * kl_row).sum() / mask.sum()
unclamped, grad_v = mask[r] / mask.sum() * p_v (log p_v - log q_v - kl_row).

Each pin checks the oracle against something other than its own formula: a
hand-worked example, closed forms (two classes, identical rows, a uniform
teacher), scipy's softmax / relative entropy, invariances of softmax, and
central finite differences of the loss.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sp

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vocab_worked_example.json")


def _ev(expr, env=None):
    return float(eval(expr, {"ln": math.log, "nan": float("nan"), **(env or {})}))


def _case(rows, V, seed, scale=2.0, masked=()):
    rng = np.random.default_rng(seed)
    s = scale * rng.standard_normal((rows, V))
    t = s + 1.5 * rng.standard_normal((rows, V))
    m = np.ones(rows, dtype=np.int8)
    for r in masked:
        m[r] = 0
    return s, t, m


def test_worked_example_from_the_card():
    g = json.load(open(GOLDEN))
    s = np.array([[_ev(e) for e in row] for row in g["student"]])
    t = np.array([[_ev(e) for e in row] for row in g["teacher"]])
    m = np.array(g["mask"], dtype=np.int8)
    r = oracle.rkl_logits(s, t, m)
    assert r.n_valid == g["n_valid"]
    assert r.loss == pytest.approx(_ev(g["loss"]), rel=1e-13, abs=0)
    assert r.loss == pytest.approx(g["loss_value"], rel=1e-13, abs=0)
    kl = [_ev(e) for e in g["kl_rows"]]
    np.testing.assert_allclose(r.kl_rows, kl, rtol=1e-13, atol=1e-15)
    env = {"kl0": kl[0], "kl1": kl[1]}
    want = np.array([[_ev(e, env) for e in row] for row in g["grad"]])
    np.testing.assert_allclose(r.grad, want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r.grad, np.array(g["grad_values"]), rtol=1e-12, atol=1e-15)
    assert not np.any(np.signbit(r.grad[2]))


def test_identical_logits_give_zero():
    s, _, m = _case(4, 33, 1)
    r = oracle.rkl_logits(s, s.copy(), m)
    assert r.loss == 0.0
    assert np.all(r.grad == 0.0)


def test_two_classes_match_the_bernoulli_closed_form():
    # V = 2: p = sigmoid(s1 - s0), q = sigmoid(t1 - t0),
    # KL = p ln(p/q) + (1-p) ln((1-p)/(1-q)); dKL/ds1 = p(1-p)(logit p - logit q) = -dKL/ds0.
    s, t, m = _case(6, 2, 2, masked=(4,))
    r = oracle.rkl_logits(s, t, m)
    p = 1.0 / (1.0 + np.exp(-(s[:, 1] - s[:, 0])))
    q = 1.0 / (1.0 + np.exp(-(t[:, 1] - t[:, 0])))
    kl = p * np.log(p / q) + (1 - p) * np.log((1 - p) / (1 - q))
    valid = m != 0
    n = valid.sum()
    assert r.loss == pytest.approx(kl[valid].sum() / n, rel=1e-12)
    d1 = p * (1 - p) * ((s[:, 1] - s[:, 0]) - (t[:, 1] - t[:, 0])) / n
    np.testing.assert_allclose(r.grad[valid, 1], d1[valid], rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(r.grad[valid, 0], -d1[valid], rtol=1e-10, atol=1e-15)


def test_uniform_teacher_gives_log_v_minus_entropy():
    s, _, m = _case(5, 40, 3)
    t = np.full_like(s, 0.7)
    r = oracle.rkl_logits(s, t, m)
    H = sp.entr(sp.softmax(s, axis=1)).sum(axis=1)
    np.testing.assert_allclose(r.kl_rows, np.log(40) - H, rtol=1e-12, atol=1e-14)


def test_rows_match_scipy_relative_entropy():
    s, t, m = _case(7, 129, 4, masked=(2, 5))
    r = oracle.rkl_logits(s, t, m)
    kl = sp.rel_entr(sp.softmax(s, axis=1), sp.softmax(t, axis=1)).sum(axis=1)
    valid = m != 0
    np.testing.assert_allclose(r.kl_rows[valid], kl[valid], rtol=1e-11, atol=1e-14)
    assert r.loss == pytest.approx(kl[valid].mean(), rel=1e-11)
    assert np.all(r.kl_rows >= 0.0)


def test_row_constants_change_nothing():
    s, t, m = _case(4, 50, 5, masked=(1,))
    rng = np.random.default_rng(9)
    r0 = oracle.rkl_logits(s, t, m)
    r1 = oracle.rkl_logits(s + 30.0 * rng.standard_normal((4, 1)), t - 20.0 * rng.standard_normal((4, 1)), m)
    assert r1.loss == pytest.approx(r0.loss, rel=1e-12)
    np.testing.assert_allclose(r1.grad, r0.grad, rtol=1e-9, atol=1e-15)


def test_gradient_matches_finite_differences():
    s, t, m = _case(3, 5, 6, scale=1.0, masked=(1,))
    r = oracle.rkl_logits(s, t, m)
    h = 1e-6
    fd = np.zeros_like(s)
    for i in range(s.shape[0]):
        for v in range(s.shape[1]):
            sp_, sm_ = s.copy(), s.copy()
            sp_[i, v] += h
            sm_[i, v] -= h
            fd[i, v] = (oracle.rkl_logits(sp_, t, m, grad=False).loss
                        - oracle.rkl_logits(sm_, t, m, grad=False).loss) / (2 * h)
    np.testing.assert_allclose(r.grad, fd, rtol=1e-6, atol=1e-9)


def test_gradient_rows_sum_to_zero():
    s, t, m = _case(6, 77, 7, masked=(0,))
    r = oracle.rkl_logits(s, t, m)
    np.testing.assert_allclose(r.grad.sum(axis=1), 0.0, atol=1e-15)


def test_masked_rows_are_never_read():
    s, t, m = _case(6, 20, 8, masked=(1, 4))
    s2, t2 = s.copy(), t.copy()
    s2[[1, 4]] = np.nan
    t2[[1, 4]] = np.inf
    a, b = oracle.rkl_logits(s, t, m), oracle.rkl_logits(s2, t2, m)
    assert a.loss == b.loss
    assert np.array_equal(a.grad, b.grad)
    keep = m != 0
    c = oracle.rkl_logits(s[keep], t[keep], m[keep])
    assert c.loss == pytest.approx(a.loss, rel=1e-15)
    assert np.all(a.grad[~keep] == 0.0) and not np.any(np.signbit(a.grad[~keep]))


def test_all_rows_masked_give_nan_loss_and_zero_gradient():
    s, t, _ = _case(3, 9, 10)
    r = oracle.rkl_logits(s, t, np.zeros(3, dtype=np.int8))
    assert math.isnan(r.loss) and r.n_valid == 0
    assert np.all(r.grad == 0.0)


def test_row_order_does_not_matter():
    s, t, m = _case(8, 31, 11, masked=(3,))
    perm = np.random.default_rng(12).permutation(8)
    a, b = oracle.rkl_logits(s, t, m), oracle.rkl_logits(s[perm], t[perm], m[perm])
    assert b.loss == pytest.approx(a.loss, rel=1e-13)
    np.testing.assert_allclose(b.grad, a.grad[perm], rtol=0, atol=0)


def test_leading_dimensions_and_counts():
    s, t, _ = _case(12, 16, 13)
    m = (np.arange(12) % 3 != 0).astype(np.int8)
    a = oracle.rkl_logits(s, t, m)
    b = oracle.rkl_logits(s.reshape(3, 4, 16), t.reshape(3, 4, 16), m.reshape(3, 4))
    assert a.n_valid == b.n_valid == 8
    assert a.loss == b.loss and np.array_equal(a.grad, b.grad.reshape(12, 16))
