"""The cross-workgroup protocol of the per-token losses, on the GPU, through the C ABI.

Every wait of the protocol has a fallback that computes the awaited value
itself: the coordinator computes a worker's count or partial loss when it has
not been published within the steal limit, a worker forms the global count
itself when the release has not come within the release limit.  The limits
are forced from the host (rlpl_workspace_set_limits, one tick = 10 ns) so
that the fallbacks run, and every result must be bit-identical to the
ordinary path, for every kernel shape and op.  Exchange kernels launched
together on two streams (whose grids cannot all be resident at once) must
finish with the same bits.  A full-vocab reverse-KL call whose waits give up
writes a NaN loss and sets the sticky flag, which check_workspace reports;
the waits for a split row's piece sums fall back like the per-token ones.
"""
import pytest
import torch

import rl_post_loss_amd as rl
import synthetic

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# (bs, seq_len) per kernel shape for bf16 planes: one tile per worker with the
# narrow lane, one tile per worker with the wide lane, several tiles per worker.
SHAPES = {"small": (64, 4096), "large": (256, 4096), "stream": (2048, 4096)}
OPS = ["bnpo", "bnpo_fwd", "grpo", "grpo_fwd", "rkl", "rkl_fwd"]


def inputs(op, bs, T, seed=0):
    w = synthetic.WORKLOADS["bnpo_bf16_64x4096"].with_(bs=bs, seq_len=T, len_lo=1, len_hi=T, seed=seed)
    return synthetic.device_policy_inputs(w, "cuda:0"), w


def fresh_workspace():
    return torch.zeros(rl.library().rlpl_workspace_bytes(1, 1, 0), dtype=torch.uint8, device=DEV)


def call(op, x, w, ws):
    kw = dict(return_n_valid=True, workspace=ws)
    if op.startswith("rkl"):
        f = rl.reverse_kl if op == "rkl" else rl.reverse_kl_fwd
        out = f(x["policy"], x["ref"], x["mask"], **kw)
    else:
        f = {"bnpo": rl.bnpo_loss, "bnpo_fwd": rl.bnpo_loss_fwd, "grpo": rl.grpo_loss,
             "grpo_fwd": rl.grpo_loss_fwd}[op]
        out = f(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"], epsilon=w.epsilon,
                epsilon_high=w.epsilon_high, beta=w.beta, **kw)
    if op.endswith("_fwd"):
        loss, n = out
        grad = None
    else:
        loss, grad, n = out
    torch.cuda.synchronize()
    return loss.clone(), None if grad is None else grad.clone(), n.clone()


def same_bits(a, b):
    la, ga, na = a
    lb, gb, nb = b
    assert la.view(torch.int32).item() == lb.view(torch.int32).item(), (la.item(), lb.item())
    assert torch.equal(na, nb)
    if ga is not None:
        assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("op", OPS)
def test_fallbacks_are_bit_identical(op, shape):
    bs, T = SHAPES[shape]
    x, w = inputs(op, bs, T)
    grid, vec, tiles = rl.launch_shape(bs, T, torch.bfloat16, op)
    if shape == "stream":
        assert grid < tiles                                  # workgroups stride over the tiles
    else:
        assert grid == tiles + 1 and vec == (4 if shape == "small" else 16)
    ref = call(op, x, w, fresh_workspace())
    for steal, release in ((1, 0), (0, 1), (1, 1)):
        ws = fresh_workspace()
        rl.set_wait_limits(ws, steal_ticks=steal, release_ticks=release)
        same_bits(call(op, x, w, ws), ref)
        # The same workspace, back at the default limits, with other inputs: values that
        # late workgroups of the forced call left in it must not leak into this call.
        rl.set_wait_limits(ws)
        x2, _ = inputs(op, bs, T, seed=1)
        same_bits(call(op, x2, w, ws), call(op, x2, w, fresh_workspace()))
        assert rl.workspace_flags(ws) == 0


# GRPO rows that cross worker boundaries gather the other workers' pieces of the
# row: one-tile (long rows; rows not dividing a tile) and striding kernels.
GRPO_ROW_SHAPES = [(16, 131072), (64, 3000), (64, 100000), (2000, 3000), (3, 1_500_000)]


@pytest.mark.parametrize("shape", GRPO_ROW_SHAPES)
@pytest.mark.parametrize("op", ["grpo", "grpo_fwd"])
def test_grpo_row_piece_fallback_is_bit_identical(op, shape):
    bs, T = shape
    x, w = inputs(op, bs, T)
    ref = call(op, x, w, fresh_workspace())
    ws = fresh_workspace()
    rl.set_wait_limits(ws, steal_ticks=1)
    for _ in range(2):
        same_bits(call(op, x, w, ws), ref)
    rl.set_wait_limits(ws)
    x2, _ = inputs(op, bs, T, seed=1)
    same_bits(call(op, x2, w, ws), call(op, x2, w, fresh_workspace()))
    assert rl.workspace_flags(ws) == 0


@pytest.mark.parametrize("op", ["bnpo", "rkl"])
def test_exchange_kernels_on_two_streams(op):
    """Two capacity-sized exchange grids in flight together cannot all be resident; each
    finishes with the bits it has alone."""
    bs, T = SHAPES["stream"]
    xs = [inputs(op, bs, T, seed=s) for s in (0, 1)]
    refs = [call(op, x, w, fresh_workspace()) for x, w in xs]
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    wss = [fresh_workspace(), fresh_workspace()]
    torch.cuda.synchronize()
    outs = [[], []]
    for _ in range(20):
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                x, w = xs[i]
                if op == "rkl":
                    outs[i].append(rl.reverse_kl(x["policy"], x["ref"], x["mask"], return_n_valid=True,
                                                 workspace=wss[i]))
                else:
                    outs[i].append(rl.bnpo_loss(x["policy"], x["old"], x["ref"], x["advantages"], x["mask"],
                                                epsilon=w.epsilon, epsilon_high=w.epsilon_high, beta=w.beta,
                                                return_n_valid=True, workspace=wss[i]))
    torch.cuda.synchronize()
    for i in (0, 1):
        for loss, grad, n in outs[i]:
            same_bits((loss, grad, n), refs[i])
        assert rl.workspace_flags(wss[i]) == 0


# Full-vocab shapes whose rows are split into pieces: kept in registers between the
# two passes (fused; in one round, and in several rounds per workgroup), read a second
# time (fused, pieces above 1024 blocks), forward only.
VOCAB_SHAPES = [(8, 248320), (200, 248320), (2, 4_500_000), (5, 33000)]


def vocab_call(fused, x, ws):
    f = rl.reverse_kl_logits if fused else rl.reverse_kl_logits_fwd
    out = f(x["student"], x["teacher"], x["mask"], return_n_valid=True, workspace=ws)
    torch.cuda.synchronize()
    if fused:
        loss, grad, n = out
        return loss.clone(), grad.clone(), n.clone()
    loss, n = out
    return loss.clone(), None, n.clone()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("shape", VOCAB_SHAPES)
def test_vocab_piece_fallback_is_bit_identical(shape, fused):
    """A split row's workgroups wait for the other pieces' sums; with a steal limit of one
    tick nearly every wait falls back to summing the piece itself.  Loss, count and
    gradient are bit-identical to a call with the default limits, and the same workspace
    then serves a call with other inputs exactly."""
    rows, V = shape
    x = synthetic.device_vocab_inputs(rows, V, "bf16", "bool", 0, "cuda:0")
    ref = vocab_call(fused, x, fresh_workspace())
    ws = fresh_workspace()
    rl.set_wait_limits(ws, steal_ticks=1)
    for _ in range(3):
        same_bits(vocab_call(fused, x, ws), ref)
    rl.set_wait_limits(ws)
    x2 = synthetic.device_vocab_inputs(rows, V, "bf16", "bool", 1, "cuda:0")
    same_bits(vocab_call(fused, x2, ws), vocab_call(fused, x2, fresh_workspace()))
    assert rl.workspace_flags(ws) == 0


def test_vocab_give_up_is_loud():
    """Logit rows split across workgroups exchange their sums; with a give-up limit of one
    tick, a wait that does not succeed at once gives up: the loss is NaN, the flag is set,
    and check_workspace raises and zero-fills the workspace.  A call whose waits all
    succeeded at once is exact.  One of several calls must have given up."""
    x = synthetic.device_vocab_inputs(8, 248320, "bf16", "bool", 0, "cuda:0")
    ref = rl.reverse_kl_logits(x["student"], x["teacher"], x["mask"], workspace=fresh_workspace())[0]
    torch.cuda.synchronize()
    gave_up = 0
    for _ in range(5):
        ws = fresh_workspace()
        rl.set_wait_limits(ws, giveup_ticks=1)
        loss, _ = rl.reverse_kl_logits(x["student"], x["teacher"], x["mask"], workspace=ws)
        flags = rl.workspace_flags(ws)
        if flags:
            gave_up += 1
            assert flags == 1 and torch.isnan(loss).item()
            with pytest.raises(RuntimeError, match="gave up"):
                rl.check_workspace(ws)
            assert int(ws.count_nonzero()) == 0
        else:
            assert loss.view(torch.int32).item() == ref.view(torch.int32).item()
    assert gave_up > 0
