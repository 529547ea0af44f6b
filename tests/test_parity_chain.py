"""The log-prob -> GRPO chain end to end on the GPU against the same chain in
the oracle (page "Add SM100 CuTe DSL GRPO fast path", section "Summary": policy
and reference log-probs from hidden states and output projections, the GRPO
loss, and its backward into the policy's hidden states, projection and bias;
model card "Geometric-AI Kernels", section "GRPO Loss", for the loss).

GPU: selective_logprob_fwd (policy, reference) -> grpo_loss on the float32
log-prob planes -> selective_logprob_bwd with the loss gradient as upstream
gradient.  Oracle: the same three steps in double precision.  The behaviour
(old) log-probs are the oracle's policy log-probs plus the generator's noise,
rounded to float32, and serve both sides.

Tolerances carry the log-prob bounds of test_parity_logprob through the chain
to first order, doubled:

* loss: sum_i |d loss/d lp_i| tol_lp_i + sum_i |d loss/d ref_i| tol_ref_i,
  plus 1e-5 relative (the float32 loss of the planes);
* loss gradient per token: |d g/d lp| tol_lp + |d g/d ref| tol_ref plus the
  float32 evaluation bound of its terms; a token within reach of the clip kink
  (ratio within 2 (tol_lp + 2^-20) of 1 + eps_high) may take either branch;
* hidden, weight and bias gradients: the log-prob backward bounds with that
  gradient error added to the upstream gradient.
"""
import numpy as np
import pytest
import torch

import oracle
import rl_post_loss_amd as rl
import synthetic
from test_parity_logprob import EPS32, _bounds, _check, _f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
EPS, EPS_HIGH = 0.2, 0.28


def f32(v):
    return float(np.float32(v))


@pytest.mark.parametrize("bs,T,H,V,dtype,beta", [
    (4, 96, 128, 2000, "bf16", 0.04),
    (3, 40, 64, 513, "fp16", 0.04),
    (2, 300, 136, 1100, "bf16", 0.0),    # 600 tokens; beta = 0 (no reference term)
])
def test_chain(bs, T, H, V, dtype, beta):
    print(f"chain case bs={bs} T={T} H={H} V={V} {dtype} beta={beta}", flush=True)
    x = synthetic.chain_inputs(bs, T, H, V, dtype, seed=bs * T + V, len_lo=T // 4)
    hp, wp, bp = _f64(x["hidden"]), _f64(x["weight"]), _f64(x["bias"])
    hr, wr = _f64(x["ref_hidden"]), _f64(x["ref_weight"])
    y = x["targets"].numpy()
    n = bs * T

    # oracle chain
    o_pol = oracle.selective_logprob(hp, wp, bp, y)
    o_ref = oracle.selective_logprob(hr, wr, bp, y)
    old = (o_pol.logp.reshape(bs, T) + x["behaviour_noise"].numpy()).astype(np.float32)
    adv = x["advantages"].numpy()
    mask = x["mask"].numpy()
    lp_o, ref_o = o_pol.logp.reshape(bs, T), o_ref.logp.reshape(bs, T)
    o_loss = oracle.grpo(lp_o, old.astype(np.float64), ref_o if beta else None, adv.astype(np.float64), mask,
                         f32(beta), f32(EPS), f32(EPS_HIGH))
    o_bwd = oracle.selective_logprob(hp, wp, bp, y, o_loss.grad.reshape(n))

    # GPU chain
    d = {k: v.to(DEV) for k, v in x.items()}
    lp, lse = rl.selective_logprob_fwd(d["hidden"], d["weight"], d["bias"], d["targets"])
    ref, _ = rl.selective_logprob_fwd(d["ref_hidden"], d["ref_weight"], d["bias"], d["targets"])
    old_d = torch.from_numpy(old).to(DEV)
    loss, g = rl.grpo_loss(lp.reshape(bs, T), old_d, ref.reshape(bs, T) if beta else None,
                           d["advantages"], d["mask"], epsilon=EPS, epsilon_high=EPS_HIGH, beta=beta)
    dh, dw, db = rl.selective_logprob_bwd(d["hidden"], d["weight"], d["bias"], d["targets"], lse, g.reshape(n))
    torch.cuda.synchronize()

    # allowances
    t_lp = _bounds(hp, wp, bp, y, np.zeros(n), o_pol.lse, dtype)[0].reshape(bs, T)
    t_ref = _bounds(hr, wr, bp, y, np.zeros(n), o_ref.lse, dtype)[0].reshape(bs, T)
    m = (mask != 0).astype(np.float64)
    counts = np.maximum(m.sum(axis=1, keepdims=True), 1.0)
    scale = m / (counts * bs)
    a = adv.astype(np.float64)[:, None]
    ratio = np.exp(lp_o - old)
    hi = 1.0 + f32(EPS_HIGH)
    e = np.exp(ref_o - lp_o) if beta else np.zeros_like(lp_o)
    b = f32(beta)
    dg_dlp = np.abs(-a * ratio * (ratio <= hi) + b * e) * scale
    dg_dref = b * e * scale
    g_eval = 8 * EPS32 * (np.abs(a) * ratio + b * (1.0 + e)) * scale
    kink = np.abs(ratio - hi) <= 2.0 * ratio * (t_lp + 2.0 ** -20)
    g_tol = 2.0 * (dg_dlp * t_lp + dg_dref * t_ref + g_eval + kink * np.abs(a) * ratio * scale)
    loss_tol = 2.0 * (np.sum(np.abs(o_loss.grad) * t_lp) + np.sum(b * np.abs(e - 1.0) * scale * t_ref)) \
        + 1e-5 * abs(o_loss.loss)

    r = [_check("policy logp", lp.cpu().numpy().reshape(bs, T), lp_o, t_lp),
         _check("reference logp", ref.cpu().numpy().reshape(bs, T), ref_o, t_ref),
         _check("loss", np.array([float(loss)]), np.array([o_loss.loss]), np.array([loss_tol])),
         _check("loss gradient", g.cpu().numpy(), o_loss.grad, g_tol)]
    _, t_dh, t_dw, t_db = _bounds(hp, wp, bp, y, o_loss.grad.reshape(n), o_pol.lse, dtype,
                                  g_err=g_tol.reshape(n))
    r += [_check("grad_hidden", _f64(dh), o_bwd.d_hidden, t_dh),
          _check("grad_weight", _f64(dw), o_bwd.d_weight, t_dw),
          _check("grad_bias", _f64(db), o_bwd.d_bias, t_db)]
    print("  worst error / allowance:", ["%.3f" % v for v in r], flush=True)
    assert torch.all(g.reshape(bs, T)[torch.from_numpy(mask == 0).to(DEV)] == 0)
