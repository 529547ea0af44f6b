"""Comparison of the HIP path with the oracle at the stated tolerances.

* fp32 planes: loss relative error <= 1e-5, gradient absolute error <= 1e-6.
* fp16 / bf16 planes: loss relative error <= 1e-3, gradient within 2 ulp of
  the output dtype (ulp taken at the oracle's value), or, where larger, within
  the float32 evaluation bound of the derivative (below).
* valid-token counts: bit-exact.

The kernels compute every per-token derivative in float32.  The derivative is
a sum of terms (-A*ratio and beta*(1 - exp(ref - lp)) for the policy losses,
1 - exp(x) for reverse KL) whose float32 evaluation carries an absolute error
of a few 2^-24 of the terms' magnitudes; where the terms nearly cancel, that
exceeds 2 ulp of the (much smaller) result.  The allowance is then
FP32_EVAL_ULPS * 2^-24 * (sum of the terms' magnitudes) * scale, which is
larger than 2 ulp of a bf16 result only where the terms cancel by more than a
factor of about 2^13.

Tokens whose ratio lies within 1e-5 (relative) of 1 + epsilon_high sit on the
clip kink: fp32 and double may take different branches there, and either
branch's gradient is accepted (the loss is continuous, so it is unaffected).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

MANT = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}
MIN_NORMAL_EXP = {torch.float32: -126, torch.float16: -14, torch.bfloat16: -126}


def ulp(x: np.ndarray, dtype) -> np.ndarray:
    """Spacing of `dtype` at |x| (subnormal spacing below the normal range)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)                       # ax = m * 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, MIN_NORMAL_EXP[dtype])
    return np.ldexp(1.0, e - MANT[dtype])


def f32(v: float) -> float:
    """The float32 value the GPU receives for a scalar parameter."""
    return float(np.float32(v))


def kink_tokens(policy, old, mask, epsilon_high) -> np.ndarray:
    lp, od = oracle.to_f64(policy), oracle.to_f64(old)
    hi = 1.0 + f32(epsilon_high)
    ratio = np.exp(lp - od)
    return (np.abs(ratio - hi) <= 1e-5 * hi) & (oracle.to_mask_u8(mask) != 0)


def kink_alternative(grad_ref, policy, old, advantages, mask, epsilon_high, scale):
    """Oracle gradient with the other clip branch taken at every token (used only at kinks)."""
    lp, od = oracle.to_f64(policy), oracle.to_f64(old)
    a = oracle.to_f64(advantages)[:, None]
    hi = 1.0 + f32(epsilon_high)
    ratio = np.exp(lp - od)
    unclipped = ratio <= hi
    g_pol = -a * ratio * scale
    return np.where(unclipped, grad_ref - g_pol, grad_ref + g_pol)


# v_exp_f32 (about 1 ulp), the rounding of its scaled argument and of the
# products and sums that form the derivative, with margin.
FP32_EVAL_ULPS = 8


def policy_grad_magnitude(policy, old, ref, advantages, beta, scale):
    """|A|*ratio + |beta|*(exp(ref - lp) + 1), times the gradient scale (per token)."""
    lp, od = oracle.to_f64(policy), oracle.to_f64(old)
    a = np.abs(oracle.to_f64(advantages))[:, None]
    mag = a * np.exp(lp - od)
    if beta != 0.0:
        mag = mag + abs(beta) * (np.exp(oracle.to_f64(ref) - lp) + 1.0)
    return mag * scale


def rkl_grad_magnitude(student, teacher, scale):
    """1 + exp(teacher - student), times the gradient scale (per token)."""
    return (1.0 + np.exp(oracle.to_f64(teacher) - oracle.to_f64(student))) * scale


def sign_aware_kinks(grad_ref, x, epsilon, epsilon_high, scale):
    """Kink tokens of the sign-aware form (ratio within 1e-5 of the bound that
    clips for the token's sign of A) and the oracle gradient with the other
    branch taken there."""
    lp, od = oracle.to_f64(x["policy"]), oracle.to_f64(x["old"])
    a = oracle.to_f64(x["advantages"])[:, None]
    ratio = np.exp(lp - od)
    bound = np.where(a < 0, 1.0 - f32(epsilon), 1.0 + f32(epsilon_high))
    kinks = (np.abs(ratio - bound) <= 1e-5 * bound) & (oracle.to_mask_u8(x["mask"]) != 0)
    unclipped = np.where(a < 0, ratio >= bound, ratio <= bound)
    g_pol = -a * ratio * scale
    alt = np.where(unclipped, grad_ref - g_pol, grad_ref + g_pol)
    return kinks, alt


def check_loss(got: float, want: float, dtype, what=""):
    tol = 1e-5 if dtype == torch.float32 else 1e-3
    if math.isnan(want):
        assert math.isnan(got), f"{what}: loss {got}, oracle NaN"
        return 0.0
    if want == 0.0:
        assert got == 0.0, f"{what}: loss {got}, oracle 0"
        return 0.0
    rel = abs(got - want) / abs(want)
    assert rel <= tol, f"{what}: loss {got!r} vs oracle {want!r}: rel err {rel:.3e} > {tol}"
    return rel


def grad_errors(got: np.ndarray, want: np.ndarray, dtype, alt: np.ndarray | None = None,
                kinks: np.ndarray | None = None, mag: np.ndarray | None = None):
    """Per-element error and allowance; at kink tokens the closer branch is used.
    `mag` (the per-token magnitude of the derivative's terms, scaled) widens the
    fp16/bf16 allowance to the float32 evaluation bound where that is larger."""
    err = np.abs(got - want)
    if alt is not None and kinks is not None and kinks.any():
        err = np.where(kinks, np.minimum(err, np.abs(got - alt)), err)
    if dtype == torch.float32:
        allow = np.full_like(want, 1e-6)
    else:
        allow = 2.0 * ulp(want, dtype)
        if mag is not None:
            allow = np.maximum(allow, FP32_EVAL_ULPS * 2.0 ** -24 * mag)
    return err, allow


def check_grad(got_t: torch.Tensor, want: np.ndarray, dtype, what="", alt=None, kinks=None, mag=None):
    got = got_t.detach().cpu().to(torch.float64).numpy()
    assert got.shape == want.shape
    err, allow = grad_errors(got, want, dtype, alt, kinks, mag)
    bad = err > allow
    if bad.any():
        i = np.unravel_index(np.argmax(err / allow), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} gradient elements out of tolerance; worst at "
            f"{i}: got {got[i]!r} oracle {want[i]!r} (allowed {allow[i]:.3e})")
    if mag is not None and dtype != torch.float32:
        # elements inside the float32 evaluation bound but beyond 2 ulp: cancelling terms
        n_cancel = int((err > 2.0 * ulp(want, dtype)).sum())
        if n_cancel:
            print(f"[parity] {what}: {n_cancel} of {err.size} gradient elements beyond 2 ulp, "
                  f"within the float32 bound of their cancelling terms", flush=True)
    # masked slots must be exactly +0
    return float(np.max(err / allow)) if err.size else 0.0


def check_masked_zero(grad_t: torch.Tensor, mask_t: torch.Tensor, what=""):
    g = grad_t.detach().cpu().to(torch.float32)
    m = mask_t.detach().cpu() != 0
    z = g[~m]
    assert torch.all(z == 0) and not torch.any(torch.signbit(z)), f"{what}: masked slots not +0"
