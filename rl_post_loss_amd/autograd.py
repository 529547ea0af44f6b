"""Autograd-aware entry points (model card "Geometric-AI Kernels", section
"Entry points": ``<name>_autograd``, the same kernel registered as a torch
custom op with an autograd formula, so that ``loss.backward()`` works and the
call traces under ``torch.compile(fullgraph=True)``).

Each op runs the fused forward+backward launch of the C ABI once, returns the
loss and keeps the gradient the launch wrote; backward multiplies that
gradient by the incoming scalar gradient of the loss (the chain rule for a
scalar loss), in float32, rounding once to the gradient's dtype.  There is no
other computation and no fallback: the ops call the same HIP kernels as the
direct entry points.

The direct entry points stay the lowest-overhead path; these add the custom-op
dispatch (and, under compile, a graph break-free call).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _policy, _rkl, _rkl_logits, selective_logprob_bwd, selective_logprob_fwd

__all__ = ["bnpo_loss_autograd", "grpo_loss_autograd", "reverse_kl_autograd",
           "reverse_kl_logits_autograd", "selective_logprob_autograd"]

_LIB = "rlpl"


def _scaled(g: torch.Tensor, grad_loss: torch.Tensor) -> torch.Tensor:
    """g * grad_loss with the product formed in float32 and rounded once to g's dtype
    (grad_loss itself is never rounded to a half-precision type)."""
    return (g.float() * grad_loss.float()).to(g.dtype)


def _policy_op(op: str):
    @torch.library.custom_op(f"{_LIB}::{op}_loss", mutates_args=())
    def fused(policy_logprobs: torch.Tensor, old_policy_logprobs: torch.Tensor,
              ref_logprobs: Optional[torch.Tensor], advantages: torch.Tensor,
              completions_mask: torch.Tensor, epsilon: float, epsilon_high: float,
              beta: float, sign_aware: bool) -> Tuple[torch.Tensor, torch.Tensor]:
        loss, grad = _policy(op, True, policy_logprobs, old_policy_logprobs, ref_logprobs, advantages,
                             completions_mask, epsilon, epsilon_high, beta, False, None,
                             "sign_aware" if sign_aware else "literal")
        return loss, grad

    @fused.register_fake
    def _(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask, epsilon,
          epsilon_high, beta, sign_aware):
        return (policy_logprobs.new_empty((), dtype=torch.float32), torch.empty_like(policy_logprobs))

    def setup_context(ctx, inputs, output):
        ctx.save_for_backward(output[1])

    def backward(ctx, grad_loss, _grad_of_grad):
        (g,) = ctx.saved_tensors
        return (_scaled(g, grad_loss), None, None, None, None, None, None, None, None)

    fused.register_autograd(backward, setup_context=setup_context)
    return fused


def _rkl_op(name: str, direct):
    @torch.library.custom_op(f"{_LIB}::{name}", mutates_args=())
    def fused(student: torch.Tensor, teacher: torch.Tensor,
              completions_mask: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        loss, grad = direct(True, student, teacher, completions_mask, False, None)
        return loss, grad

    @fused.register_fake
    def _(student, teacher, completions_mask):
        return student.new_empty((), dtype=torch.float32), torch.empty_like(student)

    def setup_context(ctx, inputs, output):
        ctx.save_for_backward(output[1])

    def backward(ctx, grad_loss, _grad_of_grad):
        (g,) = ctx.saved_tensors
        return _scaled(g, grad_loss), None, None

    fused.register_autograd(backward, setup_context=setup_context)
    return fused


_bnpo = _policy_op("bnpo")
_grpo = _policy_op("grpo")
_rkl_tok = _rkl_op("reverse_kl", _rkl)
_rkl_vocab = _rkl_op("reverse_kl_logits", _rkl_logits)


def bnpo_loss_autograd(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask, *,
                       epsilon=0.2, epsilon_high=None, beta=0.0, clip="literal"):
    """BNPO loss as a differentiable 0-d float32 tensor (gradient flows to policy_logprobs)."""
    eh = epsilon if epsilon_high is None else epsilon_high
    return _bnpo(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask,
                 float(epsilon), float(eh), float(beta), _sign_aware(clip))[0]


def grpo_loss_autograd(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask, *,
                       epsilon=0.2, epsilon_high=None, beta=0.0, clip="literal"):
    """GRPO loss as a differentiable 0-d float32 tensor."""
    eh = epsilon if epsilon_high is None else epsilon_high
    return _grpo(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask,
                 float(epsilon), float(eh), float(beta), _sign_aware(clip))[0]


def _sign_aware(clip: str) -> bool:
    if clip not in ("literal", "sign_aware"):
        raise ValueError("clip must be 'literal' or 'sign_aware'")
    return clip == "sign_aware"


def reverse_kl_autograd(student_logprobs, teacher_logprobs, completions_mask):
    """Per-token reverse KL as a differentiable 0-d float32 tensor (gradient flows to the student)."""
    return _rkl_tok(student_logprobs, teacher_logprobs, completions_mask)[0]


def reverse_kl_logits_autograd(student_logits, teacher_logits, completions_mask):
    """Full-vocab reverse KL as a differentiable 0-d float32 tensor (gradient flows to the student logits)."""
    return _rkl_vocab(student_logits, teacher_logits, completions_mask)[0]


@torch.library.custom_op(f"{_LIB}::selective_logprob", mutates_args=())
def _selective(hidden: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
               targets: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    return selective_logprob_fwd(hidden, weight, bias, targets)


@_selective.register_fake
def _(hidden, weight, bias, targets):
    n = hidden.shape[0]
    return (hidden.new_empty((n,), dtype=torch.float32), hidden.new_empty((n,), dtype=torch.float32))


@torch.library.custom_op(f"{_LIB}::selective_logprob_backward", mutates_args=())
def _selective_bwd(hidden: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                   targets: torch.Tensor, lse: torch.Tensor, grad_logp: torch.Tensor,
                   need_hidden: bool, need_weight: bool) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    dh, dw, db = selective_logprob_bwd(hidden, weight, bias, targets, lse, grad_logp,
                                       need_hidden=need_hidden, need_weight=need_weight)
    # custom ops return tensors only: empty placeholders stand for the gradients not asked for
    empty = hidden.new_empty((0,))
    return (dh if dh is not None else empty, dw if dw is not None else empty.float(),
            db if db is not None else empty.float())


@_selective_bwd.register_fake
def _(hidden, weight, bias, targets, lse, grad_logp, need_hidden, need_weight):
    n, H = hidden.shape
    V = weight.shape[0]
    dh = hidden.new_empty((n, H)) if need_hidden else hidden.new_empty((0,))
    dw = hidden.new_empty((V, H), dtype=torch.float32) if need_weight else hidden.new_empty((0,), dtype=torch.float32)
    db = hidden.new_empty((V,) if bias is not None else (0,), dtype=torch.float32)
    return dh, dw, db


def _selective_setup(ctx, inputs, output):
    hidden, weight, bias, targets = inputs
    ctx.has_bias = bias is not None
    ctx.save_for_backward(hidden, weight, bias, targets, output[1])


def _selective_backward(ctx, grad_logp, _grad_lse):
    hidden, weight, bias, targets, lse = ctx.saved_tensors
    need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
    need_b = ctx.has_bias and ctx.needs_input_grad[2]
    if not (need_h or need_w or need_b):
        return None, None, None, None
    dh, dw, db = _selective_bwd(hidden, weight, bias, targets, lse, grad_logp, need_h, need_w)
    return (dh if need_h else None, dw.to(weight.dtype) if need_w else None,
            db.to(bias.dtype) if need_b else None, None)


_selective.register_autograd(_selective_backward, setup_context=_selective_setup)


def selective_logprob_autograd(hidden, weight, bias, targets):
    """Per-token target log-probabilities (float32, (n,)) as a differentiable tensor: gradients flow to
    hidden, weight and bias (the weight and bias gradients are formed in float32, then cast to their dtype)."""
    return _selective(hidden, weight, bias, targets)[0]
