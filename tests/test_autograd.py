"""Autograd-aware entry points: custom ops over the same kernels.

CPU: the ops are registered and their fake implementations give the output
shapes and dtypes (what tracing needs).  GPU: the autograd loss and the
gradient that loss.backward() leaves are bit-identical to the direct fused
call, scale with the incoming gradient, and trace under
torch.compile(fullgraph=True).
"""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode

import rl_post_loss_amd as rl
import synthetic

DEV = torch.device("cuda:0")


def test_ops_are_registered_with_fake_implementations():
    for name in ("bnpo_loss", "grpo_loss", "reverse_kl", "reverse_kl_logits"):
        assert hasattr(torch.ops.rlpl, name)
    with FakeTensorMode():
        lp = torch.empty(4, 64, dtype=torch.bfloat16)
        m = torch.empty(4, 64, dtype=torch.bool)
        loss, grad = torch.ops.rlpl.bnpo_loss(lp, lp, lp, torch.empty(4, dtype=torch.bfloat16), m, 0.2, 0.28, 0.04,
                                              False)
        assert loss.shape == () and loss.dtype == torch.float32
        assert grad.shape == lp.shape and grad.dtype == lp.dtype
        lg = torch.empty(2, 3, 100, dtype=torch.float16)
        loss, grad = torch.ops.rlpl.reverse_kl_logits(lg, lg, torch.empty(2, 3, dtype=torch.bool))
        assert loss.shape == () and grad.shape == lg.shape and grad.dtype == lg.dtype


def _policy_case():
    w = synthetic.WORKLOADS["bnpo_bf16_64x4096"]
    x = {k: v.to(DEV) for k, v in synthetic.inputs(w).items() if k != "lengths"}
    return w, x


@pytest.mark.gpu
@pytest.mark.parametrize("clip", ["literal", "sign_aware"])
@pytest.mark.parametrize("op", ["bnpo", "grpo"])
def test_policy_autograd_matches_direct(op, clip):
    w, x = _policy_case()
    kw = dict(epsilon=w.epsilon, epsilon_high=w.epsilon_high, beta=w.beta, clip=clip)
    direct = getattr(rl, f"{op}_loss")
    auto = getattr(rl, f"{op}_loss_autograd")
    loss0, grad0 = direct(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], **kw)
    lp = x["policy"].clone().requires_grad_()
    loss = auto(lp, x["old"], x["ref"], x["advantages"], x["mask"], **kw)
    loss.backward()
    torch.cuda.synchronize()
    assert torch.equal(loss.detach(), loss0)
    assert torch.equal(lp.grad, grad0)
    lp.grad = None
    (3.0 * auto(lp, x["old"], x["ref"], x["advantages"], x["mask"], **kw)).backward()
    assert torch.equal(lp.grad, (grad0.float() * 3.0).to(grad0.dtype))


@pytest.mark.gpu
def test_autograd_upstream_scale_against_the_oracle():
    """An upstream gradient that is not a power of two (gradient accumulation over 1/k):
    the gradient loss.backward() leaves is the oracle gradient times that scale, within
    2 ulp of the output dtype (the kernel rounds once, the scaling in float32 once)."""
    import numpy as np
    import oracle
    from parity import f32, kink_alternative, kink_tokens, policy_grad_magnitude, check_grad
    w = synthetic.WORKLOADS["bnpo_bf16_64x4096"]
    xc = synthetic.inputs(w)
    x = {k: v.to(DEV) for k, v in xc.items() if k != "lengths"}
    kw = dict(epsilon=w.epsilon, epsilon_high=w.epsilon_high, beta=w.beta)
    s = 1.0 / 3.0
    lp = x["policy"].clone().requires_grad_()
    (s * rl.bnpo_loss_autograd(lp, x["old"], x["ref"], x["advantages"], x["mask"], **kw)).backward()
    torch.cuda.synchronize()
    ref = oracle.bnpo(xc["policy"], xc["old"], xc["ref"], xc["advantages"], xc["mask"], f32(w.beta),
                      f32(w.epsilon), f32(w.epsilon_high))
    scale = s / max(ref.n_valid, 1)
    kinks = kink_tokens(xc["policy"], xc["old"], xc["mask"], w.epsilon_high)
    alt = kink_alternative(ref.grad * s, xc["policy"], xc["old"], xc["advantages"], xc["mask"], w.epsilon_high,
                           scale)
    mag = policy_grad_magnitude(xc["policy"], xc["old"], xc["ref"], xc["advantages"], f32(w.beta), scale)
    check_grad(lp.grad, ref.grad * s, torch.bfloat16, "autograd x 1/3", alt, kinks, mag)
    assert np.all(lp.grad.detach().float().cpu().numpy()[xc["mask"].numpy() == 0] == 0)


@pytest.mark.gpu
def test_reverse_kl_autograd_matches_direct():
    w = synthetic.WORKLOADS["rkl_bf16_256x8192"]
    x = {k: v.to(DEV) for k, v in synthetic.inputs(w).items() if k != "lengths"}
    loss0, grad0 = rl.reverse_kl(x["student"], x["teacher"], x["mask"])
    s = x["student"].clone().requires_grad_()
    loss = rl.reverse_kl_autograd(s, x["teacher"], x["mask"])
    loss.backward()
    assert torch.equal(loss.detach(), loss0) and torch.equal(s.grad, grad0)


@pytest.mark.gpu
def test_reverse_kl_logits_autograd_matches_direct():
    x = {k: v.to(DEV) for k, v in synthetic.vocab_inputs(48, 5000, "bf16", "bool", seed=2).items()}
    s3, t3, m3 = x["student"].view(4, 12, 5000), x["teacher"].view(4, 12, 5000), x["mask"].view(4, 12)
    loss0, grad0 = rl.reverse_kl_logits(s3, t3, m3)
    s = s3.clone().requires_grad_()
    loss = rl.reverse_kl_logits_autograd(s, t3, m3)
    loss.backward()
    assert torch.equal(loss.detach(), loss0) and torch.equal(s.grad, grad0)


@pytest.mark.gpu
def test_autograd_traces_under_compile_fullgraph():
    w, x = _policy_case()
    kw = dict(epsilon=w.epsilon, epsilon_high=w.epsilon_high, beta=w.beta)
    loss0, grad0 = rl.bnpo_loss(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], **kw)

    def step(lp):
        return rl.bnpo_loss_autograd(lp, x["old"], x["ref"], x["advantages"], x["mask"], **kw)

    # aot_eager: traced graph, autograd through the custom op, no generated kernels
    compiled = torch.compile(step, fullgraph=True, backend="aot_eager")
    lp = x["policy"].clone().requires_grad_()
    loss = compiled(lp)
    loss.backward()
    torch.cuda.synchronize()
    assert torch.equal(loss.detach(), loss0) and torch.equal(lp.grad, grad0)
