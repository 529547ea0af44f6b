"""Fused forward+backward PPO-family policy losses on MI355X (gfx950).

Thin Python binding over the C ABI of ``librl_post_loss.so`` (declared in
``include/rl_post_loss.h``).  It only marshals arguments: it checks and
flattens tensors, allocates the outputs and the per-stream workspace with
torch, and passes raw device pointers plus the current HIP stream.  Every step
of the loss runs in the library's HIP kernels; there is no fallback.  If the
library is missing it is built from ``csrc/`` with hipcc; if that fails, or no
gfx950 GPU is current, the calls raise.

Entry points (model card "Geometric-AI Kernels": sections "BNPO Loss",
"GRPO Loss", "Reverse KL"; the same names as the C ABI):

* ``bnpo_loss(lp, old, ref, advantages, mask, epsilon=, epsilon_high=, beta=)`` -> (loss, grad)
* ``bnpo_loss_fwd(...)`` -> loss
* ``grpo_loss(...)`` -> (loss, grad);  ``grpo_loss_fwd(...)`` -> loss
* ``reverse_kl(student_lp, teacher_lp, mask)`` -> (loss, grad);  ``reverse_kl_fwd(...)`` -> loss
  (per-token log-probs, the card's per-token KL estimator)
* ``reverse_kl_logits(student_logits, teacher_logits, mask)`` -> (loss, grad);
  ``reverse_kl_logits_fwd(...)`` -> loss  (full (*, V) logit rows, the card's softmax form)
* ``selective_logprob_fwd(hidden, weight, bias, targets)`` -> (logp, lse) and
  ``selective_logprob_bwd(hidden, weight, bias, targets, lse, grad_logp)`` ->
  (grad_hidden, grad_weight, grad_bias): the policy log-probs from the last
  hidden states and the output projection, on the matrix cores (page "Add SM100
  CuTe DSL GRPO fast path", section "Summary")

Autograd-aware forms (``rl_post_loss_amd.autograd``): ``bnpo_loss_autograd``,
``grpo_loss_autograd``, ``reverse_kl_autograd`` and ``reverse_kl_logits_autograd``
return the loss as a differentiable tensor (torch custom ops over the same
kernels; ``loss.backward()`` and ``torch.compile(fullgraph=True)`` work).

The policy losses take ``clip="literal"`` (the card's per_token
-A*min(ratio, clipped)) or ``clip="sign_aware"`` (the standard PPO
-min(A*ratio, A*clipped); C entry point ``rlpl_policy_loss``).

``loss`` is a 0-d float32 tensor on the device; ``grad`` has the dtype and
shape of the policy/student log-probs.  Pass ``return_n_valid=True`` to also
get the valid-token count(s) as an int32 tensor (one entry, or bs for GRPO).
``workspace=`` takes a caller-owned zero-initialised uint8 tensor of
``rlpl_workspace_bytes`` bytes; by default one workspace per (device, stream)
is created on first use and reused.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import threading

import torch  # loaded first so the library binds to torch's HIP runtime

from . import build as _build

__all__ = ["bnpo_loss", "bnpo_loss_fwd", "grpo_loss", "grpo_loss_fwd", "reverse_kl",
           "reverse_kl_fwd", "library", "library_path", "RlplError", "STATUS", "workspace_for",
           "set_wait_limits", "workspace_flags", "check_workspace",
           "launch_shape", "reverse_kl_logits", "reverse_kl_logits_fwd", "bnpo_loss_autograd",
           "grpo_loss_autograd", "reverse_kl_autograd", "reverse_kl_logits_autograd",
           "selective_logprob_fwd", "selective_logprob_bwd", "selective_logprob_autograd"]

STATUS = {0: "RLPL_OK", 1: "RLPL_ERR_NULL", 2: "RLPL_ERR_SHAPE", 3: "RLPL_ERR_ALIGN",
          4: "RLPL_ERR_DTYPE", 5: "RLPL_ERR_PARAM", 6: "RLPL_ERR_WORKSPACE", 7: "RLPL_ERR_DEVICE",
          8: "RLPL_ERR_LAUNCH"}
DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
MASK_DTYPE = {torch.bool: 0, torch.int8: 1, torch.uint8: 1}
OP = {"bnpo": 0, "bnpo_fwd": 1, "grpo": 2, "grpo_fwd": 3, "rkl": 4, "rkl_fwd": 5, "rkl_logits": 6,
      "rkl_logits_fwd": 7}


class RlplError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = library().rlpl_status_string(status).decode()
        super().__init__(f"{fn}: {msg}")


_lib = None
_lock = threading.Lock()
_workspaces: dict = {}


def _release_device_state():
    """Interpreter exit: wait for the device, drop the cached workspaces and hand torch's
    cached device memory back to the HIP runtime.  Python's exit handlers run before the
    C-level ones (the HIP runtime's own teardown, and the finalisation of a profiler tool
    attached to it), so no device buffer of ours is still to be freed once those start."""
    if not torch.cuda.is_initialized():
        return
    try:
        torch.cuda.synchronize()
    except RuntimeError:
        pass
    _workspaces.clear()
    torch.cuda.empty_cache()


atexit.register(_release_device_state)


def library_path() -> str:
    return _build.LIB


def _declare(lib):
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sz = ctypes.c_size_t
    policy = [vp, vp, vp, vp, vp, i64, i64, i32, i32, f32, f32, f32, vp, vp, vp, vp, sz, vp]
    policy_fwd = [vp, vp, vp, vp, vp, i64, i64, i32, i32, f32, f32, f32, vp, vp, vp, sz, vp]
    rkl = [vp, vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, sz, vp]
    rkl_fwd = [vp, vp, vp, i64, i64, i32, i32, vp, vp, vp, sz, vp]
    for name, args in (("bnpo_loss", policy), ("grpo_loss", policy), ("bnpo_loss_fwd", policy_fwd),
                       ("grpo_loss_fwd", policy_fwd), ("reverse_kl", rkl), ("reverse_kl_fwd", rkl_fwd)):
        f = getattr(lib, name)
        f.argtypes, f.restype = args, ctypes.c_int
    for name, args in (("reverse_kl_logits", rkl), ("reverse_kl_logits_fwd", rkl_fwd)):
        f = getattr(lib, name)
        f.argtypes, f.restype = args, ctypes.c_int
    lib.bnpo_loss_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, f32, f32, f32, vp, vp, vp, vp]
    lib.bnpo_loss_noalloc.restype = ctypes.c_int
    lp_common = [vp, vp, vp, vp]
    lib.selective_logprob_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.selective_logprob_workspace_bytes.restype = sz
    lib.selective_logprob_fwd.argtypes = lp_common + [i64, i64, i64, i32, vp, vp, vp, sz, vp]
    lib.selective_logprob_fwd.restype = ctypes.c_int
    lib.selective_logprob_bwd.argtypes = lp_common + [vp, vp, i64, i64, i64, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.selective_logprob_bwd.restype = ctypes.c_int
    lib.rlpl_policy_loss.argtypes = [i32, ctypes.c_uint32] + policy
    lib.rlpl_policy_loss.restype = ctypes.c_int
    lib.rlpl_workspace_bytes.argtypes, lib.rlpl_workspace_bytes.restype = [i64, i64, i32], sz
    lib.rlpl_workspace_flags.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
    lib.rlpl_workspace_flags.restype = ctypes.c_int
    u32 = ctypes.c_uint32
    lib.rlpl_workspace_set_limits.argtypes = [vp, u32, u32, u32, vp]
    lib.rlpl_workspace_set_limits.restype = ctypes.c_int
    lib.rlpl_launch_shape.argtypes = [i64, i64, i32, i32] + [ctypes.POINTER(ctypes.c_int)] * 3
    lib.rlpl_launch_shape.restype = ctypes.c_int
    lib.rlpl_status_string.argtypes, lib.rlpl_status_string.restype = [i32], ctypes.c_char_p
    lib.rlpl_version.argtypes, lib.rlpl_version.restype = [], ctypes.c_int
    return lib


def library():
    """The loaded C library (built from csrc/ first if it is not there)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_build.LIB):
                    _build.build()
                _lib = _declare(ctypes.CDLL(_build.LIB))
    return _lib


def workspace_for(device: torch.device, stream_ptr: int, op: str = "bnpo") -> torch.Tensor:
    """The zero-initialised workspace used for calls on (device, stream); reused across calls."""
    key = (device.index, stream_ptr)
    ws = _workspaces.get(key)
    if ws is None:
        nbytes = library().rlpl_workspace_bytes(1, 1, OP[op])
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def set_wait_limits(workspace: torch.Tensor, steal_ticks: int = 0, release_ticks: int = 0,
                    giveup_ticks: int = 0) -> None:
    """Limits (100 MHz ticks; 0 = default) of the cross-workgroup waits of calls using
    `workspace`, enqueued on the current stream (C ABI rlpl_workspace_set_limits)."""
    stream = torch.cuda.current_stream(workspace.device).cuda_stream
    _check("rlpl_workspace_set_limits", library().rlpl_workspace_set_limits(
        workspace.data_ptr(), int(steal_ticks), int(release_ticks), int(giveup_ticks), stream))


def workspace_flags(workspace: torch.Tensor) -> int:
    """Sticky error bits left in `workspace` (synchronises the current stream)."""
    flags = ctypes.c_uint32(0)
    stream = torch.cuda.current_stream(workspace.device).cuda_stream
    _check("rlpl_workspace_flags", library().rlpl_workspace_flags(workspace.data_ptr(), ctypes.byref(flags), stream))
    return flags.value


def check_workspace(workspace: torch.Tensor) -> None:
    """Raises if a call on `workspace` gave up a wait (its results are then invalid);
    the workspace is zero-filled again first, so it can be re-used."""
    flags = workspace_flags(workspace)
    if flags:
        workspace.zero_()
        raise RuntimeError(f"rl_post_loss: a cross-workgroup wait gave up (workspace flags {flags:#x}); "
                           "the results of the calls since the last check are not valid")


def launch_shape(bs: int, seq_len: int, dtype: torch.dtype, op: str = "bnpo"):
    """(workgroups, slots per lane, tiles) a call would launch with on the current device."""
    grid, vec, tiles = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check("rlpl_launch_shape", library().rlpl_launch_shape(bs, seq_len, DTYPE[dtype], OP[op], ctypes.byref(grid),
                                                            ctypes.byref(vec), ctypes.byref(tiles)))
    return grid.value, vec.value, tiles.value


def _aligned(t: torch.Tensor) -> torch.Tensor:
    t = t.contiguous()
    return t if t.data_ptr() % 16 == 0 else t.clone()


def _plane(t: torch.Tensor, name: str, shape, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dim() != 2 or (shape is not None and tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name} must have shape (bs, seq_len){'' if shape is None else ' = ' + str(tuple(shape))}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return _aligned(t)


def _mask(m: torch.Tensor, shape) -> torch.Tensor:
    if m.dtype not in MASK_DTYPE:
        raise TypeError("completions_mask must be bool, int8 or uint8")
    return _plane(m, "completions_mask", shape)


def _check(fn: str, status: int):
    if status != 0:
        raise RlplError(fn, status)


def _workspace(dev, stream, op, workspace):
    if workspace is None:
        return workspace_for(dev, stream, op)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    return workspace


CLIP = {"literal": 0, "sign_aware": 1}   # rlpl_policy_loss flags (RLPL_CLIP_SIGN_AWARE)


def _policy(op: str, fused: bool, policy_logprobs, old_policy_logprobs, ref_logprobs, advantages,
            completions_mask, epsilon, epsilon_high, beta, return_n_valid, workspace, clip="literal"):
    lp = policy_logprobs.detach()
    if lp.dtype not in DTYPE:
        raise TypeError("log-probs must be float32, float16 or bfloat16")
    lp = _plane(lp, "policy_logprobs", None)
    bs, T = lp.shape
    old = _plane(old_policy_logprobs.detach(), "old_policy_logprobs", lp.shape, lp.dtype)
    beta = float(beta)
    ref = None
    if ref_logprobs is not None:
        ref = _plane(ref_logprobs.detach(), "ref_logprobs", lp.shape, lp.dtype)
    adv = advantages.detach().contiguous()
    if adv.dtype != lp.dtype or tuple(adv.shape) != (bs,) or not adv.is_cuda:
        raise ValueError(f"advantages must be a ({bs},) CUDA tensor of dtype {lp.dtype}")
    mask = _mask(completions_mask.detach(), lp.shape)
    eps_high = epsilon if epsilon_high is None else epsilon_high
    dev = lp.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws = _workspace(dev, stream, op, workspace)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    grad = torch.empty_like(lp) if fused else None
    n = torch.empty(bs if op.startswith("grpo") else 1, dtype=torch.int32, device=dev) \
        if return_n_valid else None
    if clip not in CLIP:
        raise ValueError(f"clip must be one of {sorted(CLIP)}")
    lib = library()
    name = f"{op}_loss" + ("" if fused else "_fwd")
    args = [lp.data_ptr(), old.data_ptr(), None if ref is None else ref.data_ptr(), adv.data_ptr(),
            mask.data_ptr(), bs, T, DTYPE[lp.dtype], MASK_DTYPE[mask.dtype], beta, float(epsilon),
            float(eps_high), loss.data_ptr()]
    if clip == "literal":
        if fused:
            args.append(grad.data_ptr())
        args += [None if n is None else n.data_ptr(), ws.data_ptr(), ws.numel(), stream]
        _check(name, getattr(lib, name)(*args))
    else:
        args.append(grad.data_ptr() if fused else None)
        args += [None if n is None else n.data_ptr(), ws.data_ptr(), ws.numel(), stream]
        _check("rlpl_policy_loss", lib.rlpl_policy_loss(OP[op if fused else op + "_fwd"], CLIP[clip], *args))
    out = (loss, grad) if fused else (loss,)
    if return_n_valid:
        out = out + (n,)
    return out if len(out) > 1 else out[0]


def bnpo_loss(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask, *,
              epsilon=0.2, epsilon_high=None, beta=0.0, return_n_valid=False, workspace=None,
              clip="literal"):
    """BNPO fused forward+backward: (loss, d loss / d policy_logprobs) from one launch."""
    return _policy("bnpo", True, policy_logprobs, old_policy_logprobs, ref_logprobs, advantages,
                   completions_mask, epsilon, epsilon_high, beta, return_n_valid, workspace, clip)


def bnpo_loss_fwd(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask,
                  *, epsilon=0.2, epsilon_high=None, beta=0.0, return_n_valid=False, workspace=None,
                  clip="literal"):
    """BNPO forward only: the scalar loss, no gradient buffer."""
    return _policy("bnpo", False, policy_logprobs, old_policy_logprobs, ref_logprobs, advantages,
                   completions_mask, epsilon, epsilon_high, beta, return_n_valid, workspace, clip)


def grpo_loss(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask, *,
              epsilon=0.2, epsilon_high=None, beta=0.0, return_n_valid=False, workspace=None,
              clip="literal"):
    """GRPO (per-response normalised) fused forward+backward: (loss, grad)."""
    return _policy("grpo", True, policy_logprobs, old_policy_logprobs, ref_logprobs, advantages,
                   completions_mask, epsilon, epsilon_high, beta, return_n_valid, workspace, clip)


def grpo_loss_fwd(policy_logprobs, old_policy_logprobs, ref_logprobs, advantages, completions_mask,
                  *, epsilon=0.2, epsilon_high=None, beta=0.0, return_n_valid=False, workspace=None,
                  clip="literal"):
    """GRPO forward only: the scalar loss."""
    return _policy("grpo", False, policy_logprobs, old_policy_logprobs, ref_logprobs, advantages,
                   completions_mask, epsilon, epsilon_high, beta, return_n_valid, workspace, clip)


def _rkl(fused: bool, student_logprobs, teacher_logprobs, completions_mask, return_n_valid, workspace):
    s = student_logprobs.detach()
    if s.dtype not in DTYPE:
        raise TypeError("log-probs must be float32, float16 or bfloat16")
    s = _plane(s, "student_logprobs", None)
    bs, T = s.shape
    t = _plane(teacher_logprobs.detach(), "teacher_logprobs", s.shape, s.dtype)
    mask = _mask(completions_mask.detach(), s.shape)
    dev = s.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws = _workspace(dev, stream, "rkl", workspace)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    grad = torch.empty_like(s) if fused else None
    n = torch.empty(1, dtype=torch.int32, device=dev) if return_n_valid else None
    lib = library()
    args = [s.data_ptr(), t.data_ptr(), mask.data_ptr(), bs, T, DTYPE[s.dtype], MASK_DTYPE[mask.dtype],
            loss.data_ptr()]
    if fused:
        args.append(grad.data_ptr())
    args += [None if n is None else n.data_ptr(), ws.data_ptr(), ws.numel(), stream]
    name = "reverse_kl" if fused else "reverse_kl_fwd"
    _check(name, getattr(lib, name)(*args))
    out = (loss, grad) if fused else (loss,)
    if return_n_valid:
        out = out + (n,)
    return out if len(out) > 1 else out[0]


def reverse_kl(student_logprobs, teacher_logprobs, completions_mask, *, return_n_valid=False,
               workspace=None):
    """Per-token reverse KL(student || teacher), fused forward+backward: (loss, d loss / d student)."""
    return _rkl(True, student_logprobs, teacher_logprobs, completions_mask, return_n_valid, workspace)


def reverse_kl_fwd(student_logprobs, teacher_logprobs, completions_mask, *, return_n_valid=False,
                   workspace=None):
    """Per-token reverse KL, forward only: the scalar loss."""
    return _rkl(False, student_logprobs, teacher_logprobs, completions_mask, return_n_valid, workspace)


def _rkl_logits(fused: bool, student_logits, teacher_logits, completions_mask, return_n_valid, workspace,
                check=False):
    s = student_logits.detach()
    if not isinstance(s, torch.Tensor) or not s.is_cuda or s.dtype not in DTYPE or s.dim() < 1:
        raise TypeError("student_logits must be a float32, float16 or bfloat16 CUDA (HIP) tensor")
    t = teacher_logits.detach()
    if not isinstance(t, torch.Tensor) or t.shape != s.shape or t.dtype != s.dtype or t.device != s.device:
        raise ValueError("teacher_logits must match student_logits in shape, dtype and device")
    m = completions_mask.detach()
    if m.dtype not in MASK_DTYPE or tuple(m.shape) != tuple(s.shape[:-1]) or m.device != s.device:
        raise ValueError(f"completions_mask must be a bool/int8 tensor of shape {tuple(s.shape[:-1])}")
    V = s.shape[-1]
    rows = s.numel() // V if V else 0
    s2, t2 = _aligned(s.reshape(rows, V)), _aligned(t.reshape(rows, V))
    m2 = _aligned(m.reshape(rows))
    dev = s.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws = _workspace(dev, stream, "rkl_logits", workspace)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    grad = torch.empty_like(s2) if fused else None
    n = torch.empty(1, dtype=torch.int32, device=dev) if return_n_valid else None
    args = [s2.data_ptr(), t2.data_ptr(), m2.data_ptr(), rows, V, DTYPE[s.dtype], MASK_DTYPE[m2.dtype],
            loss.data_ptr()]
    if fused:
        args.append(grad.data_ptr())
    args += [None if n is None else n.data_ptr(), ws.data_ptr(), ws.numel(), stream]
    name = "reverse_kl_logits" if fused else "reverse_kl_logits_fwd"
    _check(name, getattr(library(), name)(*args))
    if check:
        check_workspace(ws)
    out = (loss, grad.reshape(s.shape)) if fused else (loss,)
    if return_n_valid:
        out = out + (n,)
    return out if len(out) > 1 else out[0]


def reverse_kl_logits(student_logits, teacher_logits, completions_mask, *, return_n_valid=False,
                      workspace=None, check=False):
    """Reverse KL(student || teacher) over full (*, V) logit rows, fused forward+backward:
    (loss, d loss / d student_logits) from one launch.  check=True synchronises and raises
    if the call gave up a cross-workgroup wait (see check_workspace)."""
    return _rkl_logits(True, student_logits, teacher_logits, completions_mask, return_n_valid, workspace,
                       check)


def reverse_kl_logits_fwd(student_logits, teacher_logits, completions_mask, *, return_n_valid=False,
                          workspace=None, check=False):
    """Reverse KL over full logit rows, forward only: the scalar loss (one read of each valid row).
    check=True as for reverse_kl_logits."""
    return _rkl_logits(False, student_logits, teacher_logits, completions_mask, return_n_valid, workspace,
                       check)



def _lp_operands(hidden, weight, bias, targets):
    x, w = hidden.detach(), weight.detach()
    for name, t in (("hidden", x), ("weight", w)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 2:
            raise TypeError(f"{name} must be a 2-d CUDA (HIP) tensor")
    if x.dtype not in (torch.float16, torch.bfloat16) or w.dtype != x.dtype:
        raise TypeError("hidden and weight must share a float16 or bfloat16 dtype")
    if x.shape[1] != w.shape[1] or w.device != x.device:
        raise ValueError("hidden (n, H) and weight (V, H) must agree in H and device")
    n, V = x.shape[0], w.shape[0]
    b = None
    if bias is not None:
        b = bias.detach().contiguous()
        if b.dtype != x.dtype or tuple(b.shape) != (V,) or b.device != x.device:
            raise ValueError(f"bias must be a ({V},) tensor of the operands' dtype and device")
    y = targets.detach().contiguous()
    if y.dtype != torch.int64 or tuple(y.shape) != (n,) or y.device != x.device:
        raise ValueError(f"targets must be an int64 ({n},) tensor on the operands' device")
    return _aligned(x), _aligned(w), b, y


def _lp_workspace(n, H, V, backward, workspace, dev):
    nbytes = library().selective_logprob_workspace_bytes(n, H, V, int(backward))
    if nbytes == 0:
        _check("selective_logprob_workspace_bytes", 2)
    if workspace is None:
        return torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the operands' device")
    return workspace


def _ws_ptr(ws: torch.Tensor):
    p = ws.data_ptr()
    off = (-p) % 256
    return p + off, ws.numel() - off


def selective_logprob_fwd(hidden, weight, bias, targets, *, workspace=None):
    """Per-token log-probability of ``targets`` under softmax(hidden . weight^T + bias):
    (logp, lse), float32 (n,) each.  hidden (n, H) and weight (V, H) float16/bfloat16."""
    x, w, b, y = _lp_operands(hidden, weight, bias, targets)
    n, H = x.shape
    V = w.shape[0]
    dev = x.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws = _lp_workspace(n, H, V, False, workspace, dev)
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    wp, wn = _ws_ptr(ws)
    _check("selective_logprob_fwd", library().selective_logprob_fwd(
        x.data_ptr(), w.data_ptr(), None if b is None else b.data_ptr(), y.data_ptr(), n, H, V,
        DTYPE[x.dtype], logp.data_ptr(), lse.data_ptr(), wp, wn, stream))
    return logp, lse


def selective_logprob_bwd(hidden, weight, bias, targets, lse, grad_logp, *, need_hidden=True,
                          need_weight=True, grad_weight=None, grad_bias=None, workspace=None):
    """Gradients of sum(grad_logp * logp): (grad_hidden in the operands' dtype or None,
    grad_weight float32 (V, H) or None, grad_bias float32 (V,) or None).  Passing
    ``grad_weight`` / ``grad_bias`` (float32) accumulates into them."""
    x, w, b, y = _lp_operands(hidden, weight, bias, targets)
    n, H = x.shape
    V = w.shape[0]
    dev = x.device
    ls = lse.detach().to(torch.float32).contiguous()
    g = grad_logp.detach().to(torch.float32).contiguous()
    if tuple(ls.shape) != (n,) or tuple(g.shape) != (n,):
        raise ValueError(f"lse and grad_logp must have shape ({n},)")
    accumulate = grad_weight is not None or grad_bias is not None
    for name, t, shape in (("grad_weight", grad_weight, (V, H)), ("grad_bias", grad_bias, (V,))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous()
                              or t.device != dev):
            raise ValueError(f"{name} must be a contiguous float32 {shape} tensor on the operands' device")
    if accumulate and ((need_weight and grad_weight is None) or (b is not None and grad_bias is None)):
        raise ValueError("to accumulate, pass both grad_weight (when wanted) and grad_bias (with a bias)")
    dh = torch.empty_like(x) if need_hidden else None
    dw = grad_weight if grad_weight is not None else (
        torch.empty((V, H), dtype=torch.float32, device=dev) if need_weight else None)
    db = grad_bias if grad_bias is not None else (
        torch.empty(V, dtype=torch.float32, device=dev) if b is not None else None)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws = _lp_workspace(n, H, V, True, workspace, dev)
    wp, wn = _ws_ptr(ws)
    _check("selective_logprob_bwd", library().selective_logprob_bwd(
        x.data_ptr(), w.data_ptr(), None if b is None else b.data_ptr(), y.data_ptr(), ls.data_ptr(),
        g.data_ptr(), n, H, V, DTYPE[x.dtype], None if dh is None else dh.data_ptr(),
        None if dw is None else dw.data_ptr(), None if db is None else db.data_ptr(), int(accumulate),
        wp, wn, stream))
    return dh, dw, db


from .autograd import (bnpo_loss_autograd, grpo_loss_autograd, reverse_kl_autograd,  # noqa: E402
                       reverse_kl_logits_autograd, selective_logprob_autograd)
