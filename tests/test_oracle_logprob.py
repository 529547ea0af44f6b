"""Pins of the selective log-probability oracle (page "Add SM100 CuTe DSL GRPO
fast path": per-token log-probability of the target under
softmax(hidden . weight^T + bias), temperature 1, and its backward).

Checked against scipy's log-softmax on independently formed logits, the
two-class closed form, probabilities summing to one over all targets, bias
shift invariance, central finite differences of every gradient, and the
zero-sum structure of the logits' gradient.
"""
import numpy as np
import pytest
import scipy.special as sp

import oracle


def _case(n=4, h=6, V=9, seed=0, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, h))
    w = 0.7 * rng.standard_normal((V, h))
    b = rng.standard_normal(V) if bias else None
    y = rng.integers(0, V, size=n)
    g = rng.standard_normal(n)
    return x, w, b, y, g


def test_matches_scipy_log_softmax():
    x, w, b, y, _ = _case(n=7, h=11, V=23, seed=1)
    r = oracle.selective_logprob(x, w, b, y)
    z = np.einsum("ik,vk->iv", x, w) + b
    np.testing.assert_allclose(r.logp, sp.log_softmax(z, axis=1)[np.arange(7), y], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r.lse, sp.logsumexp(z, axis=1), rtol=1e-13)


def test_two_classes_closed_form():
    x = np.array([[0.5, -1.0], [2.0, 0.25]])
    w = np.array([[1.0, 0.5], [-0.5, 2.0]])
    y = np.array([0, 1])
    r = oracle.selective_logprob(x, w, None, y)
    z = x @ w.T
    want = [-np.log1p(np.exp(z[0, 1] - z[0, 0])), -np.log1p(np.exp(z[1, 0] - z[1, 1]))]
    np.testing.assert_allclose(r.logp, want, rtol=1e-13)


def test_probabilities_over_all_targets_sum_to_one():
    x, w, b, _, _ = _case(n=3, h=5, V=8, seed=2)
    total = np.zeros(3)
    for v in range(8):
        total += np.exp(oracle.selective_logprob(x, w, b, np.full(3, v)).logp)
    np.testing.assert_allclose(total, 1.0, rtol=1e-13)


def test_bias_shift_changes_nothing():
    x, w, b, y, g = _case(seed=3)
    a = oracle.selective_logprob(x, w, b, y, g)
    c = oracle.selective_logprob(x, w, b + 17.5, y, g)
    np.testing.assert_allclose(c.logp, a.logp, rtol=1e-12)
    np.testing.assert_allclose(c.d_hidden, a.d_hidden, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("which", ["hidden", "weight", "bias"])
def test_gradients_match_finite_differences(which):
    x, w, b, y, g = _case(n=3, h=4, V=5, seed=4)
    r = oracle.selective_logprob(x, w, b, y, g)
    arr = {"hidden": x, "weight": w, "bias": b}[which]
    got = {"hidden": r.d_hidden, "weight": r.d_weight, "bias": r.d_bias}[which]
    eps = 1e-6
    fd = np.zeros_like(arr)
    for idx in np.ndindex(arr.shape):
        p, m = arr.copy(), arr.copy()
        p[idx] += eps
        m[idx] -= eps
        args_p = {"hidden": x, "weight": w, "bias": b, which: p}
        args_m = {"hidden": x, "weight": w, "bias": b, which: m}
        lp = oracle.selective_logprob(args_p["hidden"], args_p["weight"], args_p["bias"], y).logp
        lm = oracle.selective_logprob(args_m["hidden"], args_m["weight"], args_m["bias"], y).logp
        fd[idx] = (np.dot(g, lp) - np.dot(g, lm)) / (2 * eps)
    np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8)


def test_logit_gradient_sums_to_zero_and_is_linear_in_g():
    x, w, b, y, g = _case(n=5, h=3, V=12, seed=5)
    r = oracle.selective_logprob(x, w, b, y, g)
    assert abs(r.d_bias.sum()) < 1e-13
    r2 = oracle.selective_logprob(x, w, b, y, 2.0 * g)
    np.testing.assert_allclose(r2.d_weight, 2.0 * r.d_weight, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r2.d_hidden, 2.0 * r.d_hidden, rtol=1e-13, atol=1e-15)


def test_rejects_out_of_range_targets():
    x, w, b, y, _ = _case()
    with pytest.raises(ValueError):
        oracle.selective_logprob(x, w, b, np.array([0, 1, 2, 9]))
