"""The entry points captured in HIP graphs.

A call enqueues its kernels on the caller's stream with no host
synchronisation, allocation or memset inside the library (the workspace comes
from the caller and every call leaves it as it found it), so a captured call
can be replayed.  Each test captures the calls once, then replays the graph
several times with new input contents copied in between, with eager work and
synchronisations between the replays, and checks every replay bit for bit
against the same calls made eagerly on the same inputs.
"""
import pytest
import torch

import rl_post_loss_amd as rl
import synthetic

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _capture(fn):
    """A graph of fn's launches (warmed up on a side stream first) and its outputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _replay_and_check(g, out, static, sets, eager):
    for i, x in enumerate(sets):
        for k, t in static.items():
            t.copy_(x[k].to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(out, want)):
            if a is None:
                continue
            assert torch.equal(a, b), f"replay {i}, output {j} differs from the eager call"


def test_policy_losses_replay():
    w = synthetic.WORKLOADS["bnpo_bf16_16x1024"]
    sets = [synthetic.policy_inputs(w.with_(seed=s)) for s in range(4)]
    keys = ("policy", "old", "ref", "advantages", "mask")
    static = {k: sets[0][k].to(DEV) for k in keys}
    ws = torch.zeros(rl.library().rlpl_workspace_bytes(w.bs, w.seq_len, 0), dtype=torch.uint8, device=DEV)
    kw = dict(epsilon=w.epsilon, epsilon_high=w.epsilon_high, beta=w.beta)

    def calls(workspace):
        loss, grad = rl.bnpo_loss(static["policy"], static["old"], static["ref"], static["advantages"],
                                  static["mask"], workspace=workspace, **kw)
        gloss, ggrad = rl.grpo_loss(static["policy"], static["old"], static["ref"], static["advantages"],
                                    static["mask"], workspace=workspace, **kw)
        floss = rl.bnpo_loss_fwd(static["policy"], static["old"], static["ref"], static["advantages"],
                                 static["mask"], workspace=workspace, **kw)
        return loss, grad, gloss, ggrad, floss

    g, out = _capture(lambda: calls(ws))
    _replay_and_check(g, out, static, sets[1:], lambda: calls(None))


def test_logit_rows_replay():
    sets = [synthetic.vocab_inputs(6, 5000, "bf16", "bool", seed=s) for s in range(4)]
    static = {k: sets[0][k].to(DEV) for k in ("student", "teacher", "mask")}
    ws = torch.zeros(rl.library().rlpl_workspace_bytes(6, 5000, rl.OP["rkl_logits"]), dtype=torch.uint8,
                     device=DEV)

    def calls(workspace):
        loss, grad = rl.reverse_kl_logits(static["student"], static["teacher"], static["mask"], workspace=workspace)
        floss = rl.reverse_kl_logits_fwd(static["student"], static["teacher"], static["mask"], workspace=workspace)
        return loss, grad, floss

    g, out = _capture(lambda: calls(ws))
    _replay_and_check(g, out, static, sets[1:], lambda: calls(None))


def test_selective_logprobs_replay():
    n, H, V = 300, 64, 1000
    sets = [synthetic.logprob_inputs(n, H, V, "bf16", seed=s) for s in range(4)]
    keys = ("hidden", "weight", "bias", "targets", "grad_logp")
    static = {k: sets[0][k].to(DEV) for k in keys}
    lib = rl.library()
    ws_f = torch.empty(lib.selective_logprob_workspace_bytes(n, H, V, 0) + 256, dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(lib.selective_logprob_workspace_bytes(n, H, V, 1) + 256, dtype=torch.uint8, device=DEV)

    def calls(wf, wb):
        logp, lse = rl.selective_logprob_fwd(static["hidden"], static["weight"], static["bias"], static["targets"],
                                             workspace=wf)
        dh, dw, db = rl.selective_logprob_bwd(static["hidden"], static["weight"], static["bias"], static["targets"],
                                              lse, static["grad_logp"], workspace=wb)
        return logp, lse, dh, dw, db

    g, out = _capture(lambda: calls(ws_f, ws_b))
    _replay_and_check(g, out, static, sets[1:], lambda: calls(None, None))
