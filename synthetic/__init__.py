"""Seeded synthetic inputs for the fused PPO-family policy losses.

This module only draws random numbers and lays them out. It holds none of the
loss arithmetic, so both the CPU oracle and the HIP path can take their inputs
from it without sharing any part of the method.

Shapes and value distributions follow the workloads the loss kernels are run
on (model card "Geometric-AI Kernels", sections "BNPO Loss", "GRPO Loss" and
"Reverse KL": per-token log-prob planes of shape (bs, seq_len) in
fp32/fp16/bf16, per-row advantages of shape (bs,), a bool or int8 completion
mask of shape (bs, seq_len)):

* policy log-probs = -|N(0,1)|, rounded to the plane dtype;
* old-policy log-probs = policy + N(0, 0.05), rounded;
* reference log-probs  = policy + N(0, 0.1), rounded;
* advantages = N(0, 1) per row, rounded to the plane dtype;
* completion mask = a prefix of integer length U[lo, hi] (both ends
  inclusive) per row; optionally a fixed number of rows fully masked;
* reverse-KL: student = -|N(0,1)|, teacher = student + N(0, 0.3).
* full-vocab reverse-KL ("Reverse KL" example): student and teacher logits
  are independent N(0,1) draws of shape (rows, vocab), rounded to the dtype;
  the row mask is U(0,1) > 0.2 (about 80 % of rows valid).
* selective log-probs (page "Add SM100 CuTe DSL GRPO fast path", section
  "Summary": a group of up to 1024 tokens, hidden size H, vocabulary V): final
  hidden states N(0, 1) of shape (n, H); output projection N(0, (2/sqrt(H))^2)
  of shape (V, H), so that logits have a standard deviation near 2; bias
  N(0, 0.25); target ids uniform on [0, V); upstream gradient N(0, 1)/n.
* the log-prob -> GRPO chain (same page, "Summary": policy and reference
  log-probs, the GRPO loss and its backward): the policy's operands as above;
  the reference model's hidden states and projection are the policy's plus
  N(0, 0.1^2) and N(0, (0.1 * 2/sqrt(H))^2) perturbations, same bias;
  advantages N(0, 1) per row; prefix completion lengths U[lo, seq_len]; and
  N(0, 0.05^2) noise that the caller adds to the policy's log-probs to form
  the behaviour (old) log-probs.

All draws come from ``numpy.random.default_rng(seed)`` (PCG64) in float64, in
the fixed order listed in ``policy_inputs`` / ``rkl_inputs``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
MASK_DTYPES = {"bool": torch.bool, "int8": torch.int8}


@dataclass(frozen=True)
class Workload:
    """One loss invocation: which loss, its shape, dtypes, parameters and mask recipe."""
    name: str
    op: str                 # "bnpo", "bnpo_fwd", "grpo", "rkl"
    dtype: str              # plane dtype: fp32 / fp16 / bf16
    mask_dtype: str         # bool / int8
    bs: int
    seq_len: int
    len_lo: int             # prefix length drawn from U[len_lo, len_hi]
    len_hi: int
    beta: float = 0.0
    epsilon: float = 0.2
    epsilon_high: float = 0.28
    masked_rows: int = 0    # rows forced fully masked (drawn without replacement)
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def slots(self) -> int:
        return self.bs * self.seq_len


# The five workloads the path is specified on.  Where a parameter is not given
# for a workload, the value of the neighbouring workloads is used (eps=0.2,
# eps_high=0.28; int8 masks for the BNPO/GRPO planes, bool for reverse-KL; seed 0).
WORKLOADS = {
    "bnpo_fp32_4x64": Workload("bnpo_fp32_4x64", "bnpo", "fp32", "bool", 4, 64, 1, 64,
                               beta=0.04, epsilon=0.2, epsilon_high=0.28),
    "bnpo_bf16_16x1024": Workload("bnpo_bf16_16x1024", "bnpo", "bf16", "int8", 16, 1024, 1, 1024,
                                  beta=0.04, epsilon=0.2, epsilon_high=0.28),
    "bnpo_bf16_64x4096": Workload("bnpo_bf16_64x4096", "bnpo", "bf16", "int8", 64, 4096, 256, 4096,
                                  beta=0.04, epsilon=0.2, epsilon_high=0.28),
    "grpo_fp16_128x2048": Workload("grpo_fp16_128x2048", "grpo", "fp16", "int8", 128, 2048, 1, 2048,
                                   beta=0.04, epsilon=0.2, epsilon_high=0.2,
                                   masked_rows=round(0.05 * 128)),
    "rkl_bf16_256x8192": Workload("rkl_bf16_256x8192", "rkl", "bf16", "bool", 256, 8192, 1024, 8192),
}


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float64 array to the plane dtype (torch CPU conversion, round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(DTYPES[dtype])


def _prefix_mask(lengths: np.ndarray, seq_len: int, mask_dtype: str) -> torch.Tensor:
    m = np.arange(seq_len, dtype=np.int64)[None, :] < lengths[:, None]
    return torch.from_numpy(m).to(MASK_DTYPES[mask_dtype])


def _lengths(rng: np.random.Generator, w: Workload) -> np.ndarray:
    lengths = rng.integers(w.len_lo, w.len_hi + 1, size=w.bs)
    if w.masked_rows:
        rows = rng.choice(w.bs, size=w.masked_rows, replace=False)
        lengths[rows] = 0
    return lengths


def policy_inputs(w: Workload) -> dict:
    """Inputs of the BNPO/GRPO losses, as CPU tensors.

    Draw order: z1 (bs,T) -> policy; z2 (bs,T) -> old; z3 (bs,T) -> ref;
    z4 (bs,) -> advantages; prefix lengths; the fully-masked rows.
    """
    rng = np.random.default_rng(w.seed)
    shape = (w.bs, w.seq_len)
    policy = _round(-np.abs(rng.standard_normal(shape)), w.dtype)
    pol64 = policy.to(torch.float64).numpy()
    old = _round(pol64 + 0.05 * rng.standard_normal(shape), w.dtype)
    ref = _round(pol64 + 0.1 * rng.standard_normal(shape), w.dtype)
    adv = _round(rng.standard_normal(w.bs), w.dtype)
    lengths = _lengths(rng, w)
    mask = _prefix_mask(lengths, w.seq_len, w.mask_dtype)
    return {"policy": policy, "old": old, "ref": ref, "advantages": adv, "mask": mask,
            "lengths": lengths}


def rkl_inputs(w: Workload) -> dict:
    """Inputs of the per-token reverse-KL loss, as CPU tensors.

    Draw order: z1 (bs,T) -> student; z2 (bs,T) -> teacher; prefix lengths.
    """
    rng = np.random.default_rng(w.seed)
    shape = (w.bs, w.seq_len)
    student = _round(-np.abs(rng.standard_normal(shape)), w.dtype)
    teacher = _round(student.to(torch.float64).numpy() + 0.3 * rng.standard_normal(shape), w.dtype)
    lengths = _lengths(rng, w)
    mask = _prefix_mask(lengths, w.seq_len, w.mask_dtype)
    return {"student": student, "teacher": teacher, "mask": mask, "lengths": lengths}


def inputs(w: Workload) -> dict:
    return rkl_inputs(w) if w.op == "rkl" else policy_inputs(w)


def device_policy_inputs(w: Workload, device: str) -> dict:
    """Large-size inputs drawn directly on the device with torch's seeded generator.

    Same distributions as ``policy_inputs`` (not the same values); used where
    host-side float64 generation would be too slow (size sweeps).
    """
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    shape = (w.bs, w.seq_len)
    dt = DTYPES[w.dtype]
    policy = (-torch.randn(shape, generator=g, device=device, dtype=torch.float32).abs()).to(dt)
    pf = policy.float()
    old = (pf + 0.05 * torch.randn(shape, generator=g, device=device)).to(dt)
    ref = (pf + 0.1 * torch.randn(shape, generator=g, device=device)).to(dt)
    adv = torch.randn(w.bs, generator=g, device=device).to(dt)
    lengths = torch.randint(w.len_lo, w.len_hi + 1, (w.bs,), generator=g, device=device)
    mask = (torch.arange(w.seq_len, device=device)[None, :] < lengths[:, None]).to(MASK_DTYPES[w.mask_dtype])
    return {"policy": policy, "old": old, "ref": ref, "advantages": adv, "mask": mask}


def vocab_inputs(rows: int, vocab: int, dtype: str = "bf16", mask_dtype: str = "bool", seed: int = 0,
                 p_valid: float = 0.8) -> dict:
    """Inputs of the full-vocab reverse-KL loss, as CPU tensors.

    Draw order: z1 (rows, vocab) -> student; z2 (rows, vocab) -> teacher;
    u (rows,) -> mask = u > 1 - p_valid.
    """
    rng = np.random.default_rng(seed)
    student = _round(rng.standard_normal((rows, vocab)), dtype)
    teacher = _round(rng.standard_normal((rows, vocab)), dtype)
    u = rng.random(rows)
    mask = torch.from_numpy(u > 1.0 - p_valid).to(MASK_DTYPES[mask_dtype])
    return {"student": student, "teacher": teacher, "mask": mask}


def device_vocab_inputs(rows: int, vocab: int, dtype: str, mask_dtype: str, seed: int, device: str,
                        p_valid: float = 0.8) -> dict:
    """Large full-vocab inputs drawn on the device with torch's seeded generator
    (same distributions as ``vocab_inputs``, not the same values)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = DTYPES[dtype]
    student = torch.randn((rows, vocab), generator=g, device=device, dtype=torch.float32).to(dt)
    teacher = torch.randn((rows, vocab), generator=g, device=device, dtype=torch.float32).to(dt)
    mask = (torch.rand(rows, generator=g, device=device) > 1.0 - p_valid).to(MASK_DTYPES[mask_dtype])
    return {"student": student, "teacher": teacher, "mask": mask}


def logprob_inputs(n: int, hidden_size: int, vocab: int, dtype: str = "bf16", seed: int = 0,
                   bias: bool = True) -> dict:
    """Inputs of the selective log-probability producer, as CPU tensors.

    Draw order: hidden (n, H); weight (V, H); bias (V,) if wanted; targets (n,); grad_logp (n,).
    """
    rng = np.random.default_rng(seed)
    hidden = _round(rng.standard_normal((n, hidden_size)), dtype)
    weight = _round(rng.standard_normal((vocab, hidden_size)) * (2.0 / np.sqrt(hidden_size)), dtype)
    b = _round(0.5 * rng.standard_normal(vocab), dtype) if bias else None
    targets = torch.from_numpy(rng.integers(0, vocab, size=n).astype(np.int64))
    grad = torch.from_numpy(rng.standard_normal(n) / max(n, 1)).to(torch.float32)
    return {"hidden": hidden, "weight": weight, "bias": b, "targets": targets, "grad_logp": grad}


def device_logprob_inputs(n: int, hidden_size: int, vocab: int, dtype: str, seed: int, device: str,
                          bias: bool = True) -> dict:
    """Large selective log-prob inputs drawn on the device with torch's seeded generator
    (same distributions as ``logprob_inputs``, not the same values)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = DTYPES[dtype]
    hidden = torch.randn((n, hidden_size), generator=g, device=device).to(dt)
    weight = (torch.randn((vocab, hidden_size), generator=g, device=device) * (2.0 / hidden_size ** 0.5)).to(dt)
    b = (0.5 * torch.randn(vocab, generator=g, device=device)).to(dt) if bias else None
    targets = torch.randint(0, vocab, (n,), generator=g, device=device, dtype=torch.int64)
    grad = torch.randn(n, generator=g, device=device) / max(n, 1)
    return {"hidden": hidden, "weight": weight, "bias": b, "targets": targets, "grad_logp": grad}


def chain_inputs(bs: int, seq_len: int, hidden_size: int, vocab: int, dtype: str = "bf16", seed: int = 0,
                 len_lo: int = 1) -> dict:
    """Inputs of the log-prob -> GRPO chain over bs x seq_len tokens, as CPU tensors.

    Draw order: the policy's operands (``logprob_inputs`` order, n = bs * seq_len); reference
    hidden noise (n, H); reference weight noise (V, H); advantages (bs,); prefix lengths;
    behaviour noise (bs, seq_len).
    """
    n = bs * seq_len
    x = logprob_inputs(n, hidden_size, vocab, dtype, seed, bias=True)
    rng = np.random.default_rng([seed, 1])
    h64, w64 = x["hidden"].to(torch.float64).numpy(), x["weight"].to(torch.float64).numpy()
    ref_hidden = _round(h64 + 0.1 * rng.standard_normal((n, hidden_size)), dtype)
    ref_weight = _round(w64 + 0.1 * (2.0 / np.sqrt(hidden_size)) * rng.standard_normal((vocab, hidden_size)), dtype)
    adv = torch.from_numpy(rng.standard_normal(bs)).to(torch.float32)
    lengths = rng.integers(len_lo, seq_len + 1, size=bs)
    mask = _prefix_mask(lengths, seq_len, "int8")
    noise = torch.from_numpy(0.05 * rng.standard_normal((bs, seq_len)))
    return {"hidden": x["hidden"], "weight": x["weight"], "bias": x["bias"], "targets": x["targets"],
            "ref_hidden": ref_hidden, "ref_weight": ref_weight, "advantages": adv, "mask": mask,
            "behaviour_noise": noise}
