"""bnpo_loss_noalloc (the entry point that allocates nothing: its workspace is the
library's own static scratch) against bnpo_loss with a caller-owned workspace,
through the C ABI: loss, gradient and valid count bit-identical, on two calls in
a row, the second on a smaller problem (so the scratch still holds the first
call's entries), and a third call on the first problem again."""
import ctypes

import pytest
import torch

import rl_post_loss_amd as rl
import synthetic

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def run(fn_name, x, w, ws=None):
    lib = rl.library()
    lp = x["policy"]
    bs, T = lp.shape
    loss = torch.empty((), dtype=torch.float32, device=DEV)
    grad = torch.empty_like(lp)
    n = torch.empty(1, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    args = [lp.data_ptr(), x["old"].data_ptr(), x["ref"].data_ptr(), x["advantages"].data_ptr(),
            x["mask"].data_ptr(), bs, T, rl.DTYPE[lp.dtype], rl.MASK_DTYPE[x["mask"].dtype], w.beta, w.epsilon,
            w.epsilon_high, loss.data_ptr(), grad.data_ptr(), n.data_ptr()]
    if ws is not None:
        args += [ws.data_ptr(), ws.numel()]
    status = getattr(lib, fn_name)(*args, stream)
    assert status == 0, lib.rlpl_status_string(status).decode()
    torch.cuda.synchronize()
    return loss, grad, n


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_no_alloc_entry_point_matches_bnpo_loss(dtype):
    ws = torch.zeros(rl.library().rlpl_workspace_bytes(1, 1, 0), dtype=torch.uint8, device=DEV)
    shapes = [(64, 4096), (16, 1000), (64, 4096)]      # a smaller second call, then the first again
    for i, (bs, T) in enumerate(shapes):
        w = synthetic.WORKLOADS["bnpo_bf16_64x4096"].with_(dtype=dtype, bs=bs, seq_len=T, len_lo=1, len_hi=T,
                                                           seed=i)
        x = {k: v.to(DEV) for k, v in synthetic.inputs(w).items() if k != "lengths"}
        ref = run("bnpo_loss", x, w, ws)
        got = run("bnpo_loss_noalloc", x, w)
        assert got[0].view(torch.int32).item() == ref[0].view(torch.int32).item()
        assert torch.equal(got[1].view(torch.int16 if dtype == "bf16" else torch.int32),
                           ref[1].view(torch.int16 if dtype == "bf16" else torch.int32))
        assert got[2].item() == ref[2].item() == int(torch.count_nonzero(x["mask"]))


def test_no_alloc_entry_point_rejects_bad_arguments_before_any_launch():
    lib = rl.library()
    loss = torch.empty((), dtype=torch.float32, device=DEV)
    status = lib.bnpo_loss_noalloc(None, None, None, None, None, 4, 64, 0, 0, 0.0, 0.2, 0.2, loss.data_ptr(),
                                   None, None, None)
    assert rl.STATUS[status] == "RLPL_ERR_NULL"
    x = torch.zeros(16, dtype=torch.float32, device=DEV)
    status = lib.bnpo_loss_noalloc(x.data_ptr(), x.data_ptr(), None, x.data_ptr(), x.data_ptr(), 1 << 16,
                                   1 << 16, 0, 0, 0.0, 0.2, 0.2, loss.data_ptr(), x.data_ptr(), None, None)
    assert rl.STATUS[status] == "RLPL_ERR_SHAPE"
