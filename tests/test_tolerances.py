"""The parity allowances are tight: they accept the correctly rounded oracle
gradient, reject an error of 3 ulp almost everywhere, and widen to the float32
evaluation bound only at the rare tokens whose derivative terms cancel."""
import numpy as np
import torch

import oracle
import synthetic
from parity import (FP32_EVAL_ULPS, check_grad, f32, grad_errors, policy_grad_magnitude,
                    rkl_grad_magnitude, ulp)


def _bnpo_case():
    w = synthetic.WORKLOADS["bnpo_bf16_64x4096"]
    x = synthetic.inputs(w)
    r = oracle.bnpo(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], f32(w.beta),
                    f32(w.epsilon), f32(w.epsilon_high))
    scale = 1.0 / max(r.n_valid, 1)
    mag = policy_grad_magnitude(x["policy"], x["old"], x["ref"], x["advantages"], f32(w.beta), scale)
    valid = oracle.to_mask_u8(x["mask"]) != 0
    return x, r, mag, valid


def test_rounded_oracle_gradient_passes():
    x, r, mag, _ = _bnpo_case()
    rounded = torch.from_numpy(r.grad).to(torch.bfloat16)
    check_grad(rounded, r.grad, torch.bfloat16, "rounded oracle", mag=mag)


def test_three_ulp_error_is_rejected_almost_everywhere():
    x, r, mag, valid = _bnpo_case()
    off = r.grad + 3.0 * ulp(r.grad, torch.bfloat16) * np.sign(r.grad)
    err, allow = grad_errors(off, r.grad, torch.bfloat16, mag=mag)
    rejected = (err > allow)[valid & (r.grad != 0)]
    assert rejected.mean() > 0.999


def test_widened_allowance_is_rare_and_tracks_cancellation():
    x, r, mag, valid = _bnpo_case()
    two_ulp = 2.0 * ulp(r.grad, torch.bfloat16)
    widened = (FP32_EVAL_ULPS * 2.0 ** -24 * mag > two_ulp) & valid
    assert widened.mean() < 1e-3
    # where it is widened, the result is many times smaller than its terms
    if widened.any():
        assert np.all(mag[widened] > 1000.0 * np.abs(r.grad[widened]))


def test_dropped_kl_term_is_rejected_as_often_as_with_plain_ulps():
    # beta*(1 - exp(ref - lp)) is ~0.4 % of |A| here, so dropping it moves many
    # gradients by less than 2 bf16 ulp; the widened allowance must not hide it
    # at any token where 2 ulp alone would catch it (bar the cancelling ones).
    x, r, mag, valid = _bnpo_case()
    w = synthetic.WORKLOADS["bnpo_bf16_64x4096"]
    r0 = oracle.bnpo(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], 0.0,
                     f32(w.epsilon), f32(w.epsilon_high))
    wrong = r0.grad * (max(r0.n_valid, 1) / max(r.n_valid, 1))
    err, allow = grad_errors(wrong, r.grad, torch.bfloat16, mag=mag)
    err2, allow2 = grad_errors(wrong, r.grad, torch.bfloat16)
    widened = (err > allow)[valid].mean()
    plain = (err2 > allow2)[valid].mean()
    assert plain > 0.2
    assert widened >= plain - 1e-3


def test_rkl_allowance():
    w = synthetic.WORKLOADS["rkl_bf16_256x8192"].with_(bs=16, seq_len=1024, len_lo=64, len_hi=1024)
    x = synthetic.inputs(w)
    r = oracle.rkl(x["student"], x["teacher"], x["mask"])
    mag = rkl_grad_magnitude(x["student"], x["teacher"], 1.0 / r.n_valid)
    check_grad(torch.from_numpy(r.grad).to(torch.bfloat16), r.grad, torch.bfloat16, "rkl", mag=mag)
    off = r.grad * (1.0 + 2.0 ** -5)
    err, allow = grad_errors(off, r.grad, torch.bfloat16, mag=mag)
    valid = (oracle.to_mask_u8(x["mask"]) != 0) & (r.grad != 0)
    assert (err > allow)[valid].mean() > 0.99
