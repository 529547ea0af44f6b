"""Parity of the selective log-probability kernels (matrix-core contraction
with in-place cross-entropy; page "Add SM100 CuTe DSL GRPO fast path",
section "Summary") with the CPU oracle, through the C ABI binding.

Tolerances are bounds derived from the kernels' arithmetic, evaluated per
element from the inputs (test-side float64, only to size the allowance), then
doubled:

* logits: products of fp16/bf16 operands are exact in float32; the sums over
  H carry at most (H + 4) * 2^-24 * S, S = |hidden| . |weight|^T + |bias|.
* lse: the p-weighted logit error, plus (tiles + 300) * 2^-24 for the float32
  tile sums, the exp2/log approximations and the final rounding, plus
  4 * 2^-24 * |lse|.  logp = z_target - lse adds both errors and 2^-23 * (|z_t| + |lse|).
* dz = g (onehot - p): the error of p (relative: logit error + lse error +
  4 * 2^-24 * (|z - lse| + 1)), the float32 evaluation, and the rounding of dz
  to the operand dtype (unit roundoff u = 2^-8 for bf16, 2^-11 for fp16, plus
  2^-25 absolute below fp16's normal range).  This rounding dominates: the
  two gradient products take dz as an fp16/bf16 operand.
* grad_hidden = sum_v dz_v weight_v: sum_v |err dz_v| |weight_v| +
  (V + 8) * 2^-24 * sum_v |dz_v| |weight_v| + the rounding of the result to
  the dtype (u |result| + 2^-25 for fp16).
* grad_weight = sum_i dz_i hidden_i and grad_bias = sum_i dz_i: likewise with
  (n + 8) * 2^-24 for the float32 sums; both are float32 outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import rl_post_loss_amd as rl
import synthetic

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
EPS32 = 2.0 ** -24
UNIT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
SUB = {"bf16": 0.0, "fp16": 2.0 ** -25}
MARGIN = 2.0


def _f64(t):
    return None if t is None else oracle.to_f64(t)


def _bounds(x, w, b, y, g, lse_o, dtype, rows=None, g_err=None):
    """Per-element allowances (logp, grad_hidden, grad_weight, grad_bias) for the given inputs (float64).
    g_err: a bound on the error of the upstream gradient g itself, per token (or None)."""
    n, H = x.shape
    V = w.shape[0]
    u, sub = UNIT[dtype], SUB[dtype]
    bb = np.zeros(V) if b is None else b
    z = x @ w.T + bb
    S = np.abs(x) @ np.abs(w).T + np.abs(bb)
    ez = (H + 4) * EPS32 * S
    p = np.exp(z - lse_o[:, None])
    tiles = -(-V // 128)
    else_ = (p * ez).sum(axis=1) + (tiles + 300) * EPS32 + 4 * EPS32 * np.abs(lse_o)
    idx = np.arange(n)
    zt = z[idx, y]
    logp_tol = ez[idx, y] + else_ + 2 * EPS32 * (np.abs(zt) + np.abs(lse_o))
    dp = p * (ez + else_[:, None] + 4 * EPS32 * (np.abs(z - lse_o[:, None]) + 1.0))
    onehot = np.zeros_like(p)
    onehot[idx, y] = 1.0
    dz = g[:, None] * (onehot - p)
    ag = np.abs(g)[:, None]
    edz = ag * dp + 2 * EPS32 * ag * (onehot + p) + u * (np.abs(dz) + ag * dp) + sub
    if g_err is not None:
        edz = edz + (1.0 + u) * g_err[:, None] * (onehot + p)
    dh = dz @ w
    dh_tol = edz @ np.abs(w) + (V + 8) * EPS32 * (np.abs(dz) @ np.abs(w)) + u * np.abs(dh) + sub
    wr = slice(None) if rows is None else rows
    dw_tol = edz[:, wr].T @ np.abs(x) + (n + 8) * EPS32 * (np.abs(dz[:, wr]).T @ np.abs(x))
    db_tol = edz.sum(axis=0) + (n + 8) * EPS32 * np.abs(dz).sum(axis=0)
    return MARGIN * logp_tol, MARGIN * dh_tol, MARGIN * dw_tol, MARGIN * db_tol


def _check(what, got, want, tol):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(np.isfinite(err), err / tol, np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; worst at {i}: "
                             f"got {got[i]!r} oracle {want[i]!r} (allowed {tol[i]:.3e})")
    pos = tol > 0
    return float((err[pos] / tol[pos]).max()) if pos.any() else 0.0


def _to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def run_case(n, H, V, dtype="bf16", bias=True, seed=0):
    print(f"selective logprob case n={n} H={H} V={V} {dtype} bias={bias} seed={seed}", flush=True)
    x = synthetic.logprob_inputs(n, H, V, dtype, seed, bias)
    d = _to_dev(x)
    logp, lse = rl.selective_logprob_fwd(d["hidden"], d["weight"], d["bias"], d["targets"])
    dh, dw, db = rl.selective_logprob_bwd(d["hidden"], d["weight"], d["bias"], d["targets"], lse, d["grad_logp"])
    torch.cuda.synchronize()
    xh, xw, xb = _f64(x["hidden"]), _f64(x["weight"]), _f64(x["bias"])
    y, g = x["targets"].numpy(), _f64(x["grad_logp"])
    ref = oracle.selective_logprob(xh, xw, xb, y, g)
    t_logp, t_dh, t_dw, t_db = _bounds(xh, xw, xb, y, g, ref.lse, dtype)
    r = [_check("logp", logp.cpu().numpy(), ref.logp, t_logp),
         _check("lse", lse.cpu().numpy(), ref.lse, t_logp),
         _check("grad_hidden", _f64(dh), ref.d_hidden, t_dh),
         _check("grad_weight", _f64(dw), ref.d_weight, t_dw)]
    if bias:
        r.append(_check("grad_bias", _f64(db), ref.d_bias, t_db))
    else:
        assert db is None
    print("  worst error / allowance:", ["%.3f" % v for v in r], flush=True)
    return d, (logp, lse, dh, dw, db)


CASES = [
    (1, 8, 1), (3, 8, 5), (64, 256, 1000), (129, 136, 257), (200, 512, 2051), (37, 64, 8200),
    (1030, 64, 300),   # two row groups: the weight and bias gradients accumulate across them
]


@pytest.mark.parametrize("n,H,V", CASES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_parity(n, H, V, dtype):
    run_case(n, H, V, dtype, bias=True, seed=n + V)


@pytest.mark.parametrize("n,H,V", [(64, 256, 1000), (130, 128, 129)])
def test_parity_without_bias(n, H, V):
    run_case(n, H, V, "bf16", bias=False, seed=3)


def test_single_class_gives_zero_logp():
    d, (logp, lse, dh, dw, db) = run_case(5, 16, 1, "bf16", seed=7)
    assert torch.all(logp == 0)
    assert torch.all(dh == 0) and torch.all(dw == 0) and torch.all(db == 0)


def test_repeat_calls_are_bitwise_identical():
    d, (logp, lse, dh, dw, db) = run_case(300, 128, 3000, "bf16", seed=11)
    logp2, lse2 = rl.selective_logprob_fwd(d["hidden"], d["weight"], d["bias"], d["targets"])
    dh2, dw2, db2 = rl.selective_logprob_bwd(d["hidden"], d["weight"], d["bias"], d["targets"], lse2,
                                             d["grad_logp"])
    for a, b in ((logp, logp2), (lse, lse2), (dh, dh2), (dw, dw2), (db, db2)):
        assert torch.equal(a, b)


def test_accumulate_adds_to_the_gradients():
    x = _to_dev(synthetic.logprob_inputs(100, 64, 700, "bf16", 5))
    logp, lse = rl.selective_logprob_fwd(x["hidden"], x["weight"], x["bias"], x["targets"])
    _, dw, db = rl.selective_logprob_bwd(x["hidden"], x["weight"], x["bias"], x["targets"], lse, x["grad_logp"],
                                         need_hidden=False)
    acc_w, acc_b = dw.clone(), db.clone()
    rl.selective_logprob_bwd(x["hidden"], x["weight"], x["bias"], x["targets"], lse, x["grad_logp"],
                             need_hidden=False, grad_weight=acc_w, grad_bias=acc_b)
    assert torch.equal(acc_w, 2 * dw) and torch.equal(acc_b, 2 * db)


def test_out_of_range_target_gives_nan():
    x = _to_dev(synthetic.logprob_inputs(6, 32, 50, "bf16", 2))
    x["targets"][2] = 50
    x["targets"][4] = -1
    logp, lse = rl.selective_logprob_fwd(x["hidden"], x["weight"], x["bias"], x["targets"])
    ok = torch.tensor([True, True, False, True, False, True], device=DEV)
    assert torch.isnan(logp[~ok]).all() and torch.isfinite(logp[ok]).all() and torch.isfinite(lse).all()


def test_rejects_bad_shapes():
    x = _to_dev(synthetic.logprob_inputs(4, 12, 20, "bf16", 1))   # H = 12 is not a multiple of 8
    with pytest.raises(rl.RlplError, match="SHAPE"):
        rl.selective_logprob_fwd(x["hidden"], x["weight"], x["bias"], x["targets"])
    with pytest.raises(TypeError):
        rl.selective_logprob_fwd(x["hidden"].float(), x["weight"].float(), None, x["targets"])


def test_autograd_matches_direct_backward():
    x = _to_dev(synthetic.logprob_inputs(70, 64, 600, "bf16", 9))
    h = x["hidden"].clone().requires_grad_(True)
    w = x["weight"].clone().requires_grad_(True)
    b = x["bias"].clone().requires_grad_(True)
    logp = rl.selective_logprob_autograd(h, w, b, x["targets"])
    (logp * x["grad_logp"]).sum().backward()
    lp2, lse = rl.selective_logprob_fwd(x["hidden"], x["weight"], x["bias"], x["targets"])
    dh, dw, db = rl.selective_logprob_bwd(x["hidden"], x["weight"], x["bias"], x["targets"], lse, x["grad_logp"])
    assert torch.equal(logp.detach(), lp2)
    assert torch.equal(h.grad, dh) and torch.equal(w.grad, dw.to(w.dtype)) and torch.equal(b.grad, db.to(b.dtype))


def test_full_size_sampled_rows():
    """The 1024-token group at H = 4096, V = 128256 (bf16), the size the producer is
    timed at: logp/lse on sampled rows, and the backward with the upstream gradient
    non-zero only on those rows, so that the oracle on those rows gives every
    gradient exactly (the other rows contribute exact zeros)."""
    n, H, V = 1024, 4096, 128256
    print(f"selective logprob full size n={n} H={H} V={V}", flush=True)
    d = synthetic.device_logprob_inputs(n, H, V, "bf16", 21, str(DEV))
    rows = np.array([0, 333, 777, 1023])
    g = torch.zeros(n, device=DEV)
    g[torch.from_numpy(rows).to(DEV)] = torch.tensor([0.75, -1.25, 0.5, 2.0], device=DEV)
    logp, lse = rl.selective_logprob_fwd(d["hidden"], d["weight"], d["bias"], d["targets"])
    dh, dw, db = rl.selective_logprob_bwd(d["hidden"], d["weight"], d["bias"], d["targets"], lse, g)
    torch.cuda.synchronize()
    xh = _f64(d["hidden"][torch.from_numpy(rows).to(DEV)])
    xw, xb = _f64(d["weight"]), _f64(d["bias"])
    y = d["targets"].cpu().numpy()[rows]
    gg = g.cpu().double().numpy()[rows]
    ref = oracle.selective_logprob(xh, xw, xb, y, gg)
    vocab_rows = np.unique(np.concatenate([y, np.random.default_rng(0).integers(0, V, 200)]))
    t_logp, t_dh, t_dw, t_db = _bounds(xh, xw, xb, y, gg, ref.lse, "bf16", rows=vocab_rows)
    _check("logp", logp.cpu().numpy()[rows], ref.logp, t_logp)
    _check("lse", lse.cpu().numpy()[rows], ref.lse, t_logp)
    _check("grad_hidden", _f64(dh)[rows], ref.d_hidden, t_dh)
    others = np.setdiff1d(np.arange(n), rows)
    assert torch.all(dh[torch.from_numpy(others).to(DEV)] == 0)
    _check("grad_weight", _f64(dw[torch.from_numpy(vocab_rows).to(DEV)]), ref.d_weight[vocab_rows], t_dw)
    _check("grad_bias", _f64(db), ref.d_bias, t_db)
    assert torch.isfinite(logp).all() and torch.isfinite(lse).all()
