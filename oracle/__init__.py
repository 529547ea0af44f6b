"""CPU oracle for the fused PPO-family policy losses (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``rl_post_loss_amd``) never imports it, and the two share no
code: this wrapper only marshals arrays into ``rlpl_oracle.c``, a plain C99
double-precision implementation of the model card's formulas (see the header
of that file for the sections it follows and the readings it takes).

Inputs are widened exactly to float64 before the call, so the oracle sees the
same values the GPU reads from its bf16/fp16/fp32 planes.  Scalar parameters
(beta, epsilon, epsilon_high) are taken as given; callers that compare with
the GPU pass the float32 values the GPU receives.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rlpl_oracle.c")
_LIB = os.path.join(_HERE, "librlpl_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    d = ctypes.c_double
    lib.rlpl_oracle_bnpo.argtypes = [i64, i64, dp, dp, dp, dp, u8p, d, d, d, dp, dp, i64p]
    lib.rlpl_oracle_grpo.argtypes = [i64, i64, dp, dp, dp, dp, u8p, d, d, d, dp, dp, i64p]
    lib.rlpl_oracle_rkl.argtypes = [i64, i64, dp, dp, u8p, dp, dp, i64p]
    lib.rlpl_oracle_bnpo_ppo.argtypes = [i64, i64, dp, dp, dp, dp, u8p, d, d, d, dp, dp, i64p]
    lib.rlpl_oracle_grpo_ppo.argtypes = [i64, i64, dp, dp, dp, dp, u8p, d, d, d, dp, dp, i64p]
    lib.rlpl_oracle_rkl_logits.argtypes = [i64, i64, dp, dp, u8p, dp, dp, i64p, dp]
    lib.rlpl_oracle_selective_logprob.argtypes = [i64, i64, i64, dp, dp, dp, i64p, dp, dp, dp, dp, dp, dp]
    lib.rlpl_oracle_selective_logprob.restype = ctypes.c_int
    for f in (lib.rlpl_oracle_bnpo, lib.rlpl_oracle_grpo, lib.rlpl_oracle_rkl, lib.rlpl_oracle_rkl_logits,
              lib.rlpl_oracle_bnpo_ppo, lib.rlpl_oracle_grpo_ppo):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _use_library(path: Optional[str]) -> None:
    """Point the wrapper at another build of rlpl_oracle.c (the mutation test's planted copies).

    ``None`` returns to the default library.
    """
    global _lib, _LIB
    _lib = None
    _LIB = path or os.path.join(_HERE, "librlpl_oracle.so")


def to_f64(x) -> np.ndarray:
    """Exact widening of a torch tensor or array (fp32/fp16/bf16/fp64) to a contiguous float64 array."""
    if hasattr(x, "detach"):
        import torch
        return np.ascontiguousarray(x.detach().to("cpu").to(torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def to_mask_u8(m) -> np.ndarray:
    """Mask bytes as uint8 (nonzero means valid); bool and int8 keep their zero/nonzero pattern."""
    if hasattr(m, "detach"):
        import torch
        m = m.detach().to("cpu")
        m = m.to(torch.uint8) if m.dtype == torch.bool else m.contiguous().view(torch.uint8)
        return np.ascontiguousarray(m.numpy())
    m = np.asarray(m)
    return np.ascontiguousarray(m.astype(np.uint8) if m.dtype == np.bool_ else m.view(np.uint8))


def _p(a: Optional[np.ndarray], t):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(t))


@dataclass
class Result:
    loss: float
    grad: Optional[np.ndarray]      # float64, shape (bs, seq_len), or None
    n_valid: object                 # int (BNPO / reverse-KL) or int64 array (bs,) (GRPO)


def _policy_call(fn, policy, old, ref, advantages, mask, beta, epsilon, epsilon_high, grad, per_row):
    lp, od = to_f64(policy), to_f64(old)
    bs, T = lp.shape
    rf = to_f64(ref) if ref is not None else None
    a = to_f64(advantages).reshape(bs)
    m = to_mask_u8(mask).reshape(bs, T)
    loss = ctypes.c_double(0.0)
    g = np.empty((bs, T), dtype=np.float64) if grad else None
    n = np.zeros(bs if per_row else 1, dtype=np.int64)
    rc = fn(bs, T, _p(lp, ctypes.c_double), _p(od, ctypes.c_double), _p(rf, ctypes.c_double),
            _p(a, ctypes.c_double), _p(m, ctypes.c_uint8), float(beta), float(epsilon),
            float(epsilon_high), ctypes.byref(loss), _p(g, ctypes.c_double),
            _p(n, ctypes.c_int64))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return Result(loss.value, g, n if per_row else int(n[0]))


def bnpo(policy, old, ref, advantages, mask, beta, epsilon, epsilon_high, grad=True,
         sign_aware=False) -> Result:
    """BNPO loss (global token mean) and d loss / d policy; sign_aware takes the
    PPO form -min(A*ratio, A*clipped) for per_token."""
    lib = _load()
    return _policy_call(lib.rlpl_oracle_bnpo_ppo if sign_aware else lib.rlpl_oracle_bnpo, policy, old,
                        ref, advantages, mask, beta, epsilon, epsilon_high, grad, per_row=False)


def grpo(policy, old, ref, advantages, mask, beta, epsilon, epsilon_high, grad=True,
         sign_aware=False) -> Result:
    """GRPO loss (per-response token mean, then mean over rows) and d loss / d policy."""
    lib = _load()
    return _policy_call(lib.rlpl_oracle_grpo_ppo if sign_aware else lib.rlpl_oracle_grpo, policy, old,
                        ref, advantages, mask, beta, epsilon, epsilon_high, grad, per_row=True)


def rkl(student, teacher, mask, grad=True) -> Result:
    """Per-token reverse-KL (k3 estimator, unclamped global token mean) and d loss / d student."""
    s, t = to_f64(student), to_f64(teacher)
    bs, T = s.shape
    m = to_mask_u8(mask).reshape(bs, T)
    loss = ctypes.c_double(0.0)
    g = np.empty((bs, T), dtype=np.float64) if grad else None
    n = np.zeros(1, dtype=np.int64)
    rc = _load().rlpl_oracle_rkl(bs, T, _p(s, ctypes.c_double), _p(t, ctypes.c_double),
                                 _p(m, ctypes.c_uint8), ctypes.byref(loss),
                                 _p(g, ctypes.c_double), _p(n, ctypes.c_int64))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return Result(loss.value, g, int(n[0]))


@dataclass
class VocabResult:
    loss: float
    grad: Optional[np.ndarray]      # float64, shape of the logits, or None
    n_valid: int
    kl_rows: np.ndarray             # float64 (rows,): kl of each valid row, 0 for masked rows


def rkl_logits(student, teacher, mask, grad=True) -> VocabResult:
    """Full-vocab reverse KL between the softmaxes of two (*, V) logit slabs, the
    unclamped mean over valid rows, and d loss / d student logits."""
    s, t = to_f64(student), to_f64(teacher)
    shape = s.shape
    V = shape[-1]
    s2, t2 = s.reshape(-1, V), t.reshape(-1, V)
    rows = s2.shape[0]
    m = to_mask_u8(mask).reshape(rows)
    loss = ctypes.c_double(0.0)
    g = np.empty((rows, V), dtype=np.float64) if grad else None
    n = np.zeros(1, dtype=np.int64)
    kl = np.zeros(rows, dtype=np.float64)
    rc = _load().rlpl_oracle_rkl_logits(rows, V, _p(s2, ctypes.c_double), _p(t2, ctypes.c_double),
                                        _p(m, ctypes.c_uint8), ctypes.byref(loss),
                                        _p(g, ctypes.c_double), _p(n, ctypes.c_int64),
                                        _p(kl, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return VocabResult(loss.value, None if g is None else g.reshape(shape), int(n[0]), kl)


@dataclass
class LogprobResult:
    logp: np.ndarray                 # (n,)
    lse: np.ndarray                  # (n,)
    d_hidden: Optional[np.ndarray]   # (n, h)
    d_weight: Optional[np.ndarray]   # (vocab, h)
    d_bias: Optional[np.ndarray]     # (vocab,)


def selective_logprob(hidden, weight, bias, targets, grad_logp=None) -> LogprobResult:
    """Per-token log-probability of the target under softmax(hidden . weight^T + bias), and,
    for an upstream gradient grad_logp, the gradients of sum(grad_logp * logp)."""
    x, w = to_f64(hidden), to_f64(weight)
    n, h = x.shape
    V = w.shape[0]
    b = to_f64(bias) if bias is not None else None
    y = np.ascontiguousarray(np.asarray(targets.cpu() if hasattr(targets, "cpu") else targets, dtype=np.int64))
    logp, lse = np.empty(n), np.empty(n)
    g = to_f64(grad_logp) if grad_logp is not None else None
    dh = np.empty((n, h)) if g is not None else None
    dw = np.empty((V, h)) if g is not None else None
    db = np.empty(V) if (g is not None and b is not None) else None
    rc = _load().rlpl_oracle_selective_logprob(n, h, V, _p(x, ctypes.c_double), _p(w, ctypes.c_double),
                                               _p(b, ctypes.c_double), _p(y, ctypes.c_int64),
                                               _p(logp, ctypes.c_double), _p(lse, ctypes.c_double),
                                               _p(g, ctypes.c_double), _p(dh, ctypes.c_double),
                                               _p(dw, ctypes.c_double), _p(db, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return LogprobResult(logp, lse, dh, dw, db)
