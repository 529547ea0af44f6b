"""The C ABI on the host: exported symbols, constants and argument validation.

Validation is pure host code that runs before any HIP call, so every status
below is checked without a GPU.  Pointers here are fake integers: the calls
must reject them before touching the device (the one call that passes
validation is only made when no GPU is present).
"""
import ctypes
import os
import re

import pytest
import torch

import rl_post_loss_amd as rl

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "rl_post_loss.h")

A = 0x7F0000001000          # a fake 16-byte-aligned "device" address
WS = 0x7F0000100000         # fake 256-byte-aligned workspace


def header_text():
    src = open(HEADER).read()
    return re.sub(r"/\*.*?\*/", "", src, flags=re.S)


def declared_functions():
    return re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", header_text(), flags=re.M)


def header_enum(name):
    body = re.search(r"enum\s+%s\s*\{(.*?)\}" % name, header_text(), flags=re.S).group(1)
    return {k: int(v) for k, v in re.findall(r"(\w+)\s*=\s*(\d+)", body)}


@pytest.fixture(scope="module")
def lib():
    return rl.library()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) >= {"bnpo_loss", "bnpo_loss_fwd", "grpo_loss", "grpo_loss_fwd", "reverse_kl",
                          "reverse_kl_fwd", "rlpl_workspace_bytes", "rlpl_workspace_flags",
                          "rlpl_status_string", "rlpl_version", "rlpl_launch_shape",
                          "reverse_kl_logits", "reverse_kl_logits_fwd", "rlpl_policy_loss"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.rlpl_version() == 1


def test_header_constants_match_binding():
    st = header_enum("rlpl_status")
    assert {v: k for k, v in st.items()} == rl.STATUS
    dt = header_enum("rlpl_dtype")
    assert dt == {"RLPL_F32": rl.DTYPE[torch.float32], "RLPL_F16": rl.DTYPE[torch.float16],
                  "RLPL_BF16": rl.DTYPE[torch.bfloat16]}
    md = header_enum("rlpl_mask_dtype")
    assert md == {"RLPL_MASK_BOOL": rl.MASK_DTYPE[torch.bool], "RLPL_MASK_INT8": rl.MASK_DTYPE[torch.int8]}
    ops = header_enum("rlpl_op")
    assert ops == {"RLPL_OP_" + k.upper(): v for k, v in rl.OP.items()}


def test_status_strings(lib):
    seen = set()
    for code, name in rl.STATUS.items():
        s = lib.rlpl_status_string(code).decode()
        assert s.startswith(name)
        seen.add(s)
    assert len(seen) == len(rl.STATUS)
    assert "unknown" in lib.rlpl_status_string(99).decode()


def test_workspace_bytes(lib):
    for op in range(8):
        n = lib.rlpl_workspace_bytes(64, 4096, op)
        assert n >= 256 + 4 * 1024 and n % 256 == 0
    assert lib.rlpl_workspace_bytes(64, 4096, 8) == 0
    assert lib.rlpl_workspace_bytes(64, 4096, -1) == 0


def _bnpo_args(**over):
    a = dict(lp=A, old=A + 0x100000, ref=A + 0x200000, adv=A + 0x300000, mask=A + 0x400000,
             bs=4, T=64, dtype=2, mask_dtype=1, beta=0.04, eps=0.2, eps_high=0.28,
             loss=A + 0x500000, grad=A + 0x600000, n=A + 0x700000, ws=WS, ws_bytes=8 << 20,
             stream=None)
    a.update(over)
    return a


def call_bnpo(lib, fused=True, **over):
    a = _bnpo_args(**over)
    args = [a["lp"], a["old"], a["ref"], a["adv"], a["mask"], a["bs"], a["T"], a["dtype"],
            a["mask_dtype"], a["beta"], a["eps"], a["eps_high"], a["loss"]]
    if fused:
        args.append(a["grad"])
    args += [a["n"], a["ws"], a["ws_bytes"], a["stream"]]
    return (lib.bnpo_loss if fused else lib.bnpo_loss_fwd)(*args)


def call_rkl(lib, fused=True, **over):
    a = _bnpo_args(**over)
    args = [a["lp"], a["ref"], a["mask"], a["bs"], a["T"], a["dtype"], a["mask_dtype"], a["loss"]]
    if fused:
        args.append(a["grad"])
    args += [a["n"], a["ws"], a["ws_bytes"], a["stream"]]
    return (lib.reverse_kl if fused else lib.reverse_kl_fwd)(*args)


CASES = [
    ("RLPL_ERR_NULL", dict(lp=None)),
    ("RLPL_ERR_NULL", dict(old=None)),
    ("RLPL_ERR_NULL", dict(adv=None)),
    ("RLPL_ERR_NULL", dict(mask=None)),
    ("RLPL_ERR_NULL", dict(loss=None)),
    ("RLPL_ERR_NULL", dict(ref=None)),                 # beta != 0 needs ref
    ("RLPL_ERR_SHAPE", dict(bs=0)),
    ("RLPL_ERR_SHAPE", dict(T=0)),
    ("RLPL_ERR_SHAPE", dict(bs=-3)),
    ("RLPL_ERR_SHAPE", dict(bs=1 << 16, T=1 << 15)),   # exactly 2^31 slots
    ("RLPL_ERR_SHAPE", dict(bs=1 << 40, T=1 << 40)),   # overflow guard
    ("RLPL_ERR_DTYPE", dict(dtype=3)),
    ("RLPL_ERR_DTYPE", dict(dtype=-1)),
    ("RLPL_ERR_DTYPE", dict(mask_dtype=2)),
    ("RLPL_ERR_ALIGN", dict(lp=A + 2)),
    ("RLPL_ERR_ALIGN", dict(old=A + 8)),
    ("RLPL_ERR_ALIGN", dict(ref=A + 4)),
    ("RLPL_ERR_ALIGN", dict(mask=A + 0x400000 + 1)),
    ("RLPL_ERR_ALIGN", dict(adv=A + 0x300000 + 1)),
    ("RLPL_ERR_ALIGN", dict(loss=A + 0x500000 + 2)),
    ("RLPL_ERR_ALIGN", dict(n=A + 0x700000 + 1)),
    ("RLPL_ERR_ALIGN", dict(ws=WS + 64)),
    ("RLPL_ERR_PARAM", dict(beta=float("nan"))),
    ("RLPL_ERR_PARAM", dict(beta=float("inf"))),
    ("RLPL_ERR_PARAM", dict(eps=float("nan"))),
    ("RLPL_ERR_PARAM", dict(eps_high=float("-inf"))),
    ("RLPL_ERR_PARAM", dict(eps=-0.5, eps_high=-0.6)),  # 1-eps > 1+eps_high
    ("RLPL_ERR_WORKSPACE", dict(ws=None)),
    ("RLPL_ERR_WORKSPACE", dict(ws_bytes=1024)),
]


@pytest.mark.parametrize("want,over", CASES, ids=[f"{w}-{list(o)[0]}" for w, o in CASES])
def test_bnpo_validation(lib, want, over):
    assert rl.STATUS[call_bnpo(lib, **over)] == want
    if "grad" not in over:
        assert rl.STATUS[call_bnpo(lib, fused=False, **over)] == want


def test_fused_needs_grad_and_grad_alignment(lib):
    assert rl.STATUS[call_bnpo(lib, grad=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_bnpo(lib, grad=A + 0x600000 + 2)] == "RLPL_ERR_ALIGN"
    for fn in (lib.grpo_loss,):
        a = _bnpo_args(grad=None)
        assert rl.STATUS[fn(a["lp"], a["old"], a["ref"], a["adv"], a["mask"], 4, 64, 2, 1, 0.04,
                            0.2, 0.28, a["loss"], None, None, WS, 8 << 20, None)] == "RLPL_ERR_NULL"


def test_rkl_validation(lib):
    assert rl.STATUS[call_rkl(lib, lp=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_rkl(lib, ref=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_rkl(lib, grad=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_rkl(lib, lp=A + 2)] == "RLPL_ERR_ALIGN"
    assert rl.STATUS[call_rkl(lib, T=0)] == "RLPL_ERR_SHAPE"
    assert rl.STATUS[call_rkl(lib, dtype=7)] == "RLPL_ERR_DTYPE"
    assert rl.STATUS[call_rkl(lib, ws_bytes=0)] == "RLPL_ERR_WORKSPACE"


def test_workspace_flags_validation(lib):
    flags = ctypes.c_uint32(0)
    assert rl.STATUS[lib.rlpl_workspace_flags(None, ctypes.byref(flags), None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[lib.rlpl_workspace_flags(WS + 4, ctypes.byref(flags), None)] == "RLPL_ERR_ALIGN"


def test_workspace_set_limits_validation(lib):
    assert rl.STATUS[lib.rlpl_workspace_set_limits(None, 1, 1, 1, None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[lib.rlpl_workspace_set_limits(WS + 16, 1, 1, 1, None)] == "RLPL_ERR_ALIGN"


def test_beta_zero_allows_missing_ref_without_a_device(lib):
    # Passes validation (beta == 0 compiles the KL term out, ref may be NULL) and then
    # stops at the device check: only meaningful, and only safe, on a host with no GPU.
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: a call that passes validation would launch")
    assert rl.STATUS[call_bnpo(lib, beta=0.0, ref=None)] == "RLPL_ERR_DEVICE"
    assert rl.STATUS[call_rkl(lib)] == "RLPL_ERR_DEVICE"


def test_binding_rejects_cpu_tensors():
    x = torch.zeros(2, 16)
    with pytest.raises(TypeError):
        rl.bnpo_loss(x, x, x, torch.zeros(2), torch.ones(2, 16, dtype=torch.bool), beta=0.04)


def test_launch_shape_validation(lib):
    g, v, t = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    out = (ctypes.byref(g), ctypes.byref(v), ctypes.byref(t))
    assert rl.STATUS[lib.rlpl_launch_shape(0, 64, 2, 0, *out)] == "RLPL_ERR_SHAPE"
    assert rl.STATUS[lib.rlpl_launch_shape(4, 64, 9, 0, *out)] == "RLPL_ERR_DTYPE"
    assert rl.STATUS[lib.rlpl_launch_shape(4, 64, 2, 17, *out)] == "RLPL_ERR_PARAM"
    assert rl.STATUS[lib.rlpl_launch_shape(4, 64, 2, 0, None, ctypes.byref(v), ctypes.byref(t))] == "RLPL_ERR_NULL"
    if not torch.cuda.is_available():
        assert rl.STATUS[lib.rlpl_launch_shape(4, 64, 2, 0, *out)] == "RLPL_ERR_DEVICE"


def call_vocab(lib, fused=True, **over):
    a = dict(s=A, t=A + 0x100000, mask=A + 0x200000, rows=8, V=1000, dtype=2, mask_dtype=0,
             loss=A + 0x300000, grad=A + 0x400000, n=A + 0x500000, ws=WS, ws_bytes=8 << 20, stream=None)
    a.update(over)
    args = [a["s"], a["t"], a["mask"], a["rows"], a["V"], a["dtype"], a["mask_dtype"], a["loss"]]
    if fused:
        args.append(a["grad"])
    args += [a["n"], a["ws"], a["ws_bytes"], a["stream"]]
    return (lib.reverse_kl_logits if fused else lib.reverse_kl_logits_fwd)(*args)


VOCAB_CASES = [
    ("RLPL_ERR_NULL", dict(s=None)),
    ("RLPL_ERR_NULL", dict(t=None)),
    ("RLPL_ERR_NULL", dict(mask=None)),
    ("RLPL_ERR_NULL", dict(loss=None)),
    ("RLPL_ERR_SHAPE", dict(rows=0)),
    ("RLPL_ERR_SHAPE", dict(V=0)),
    ("RLPL_ERR_SHAPE", dict(rows=1 << 31)),
    ("RLPL_ERR_SHAPE", dict(rows=1 << 20, V=(1 << 42) + 1)),   # rows * vocab > 2^62
    ("RLPL_ERR_DTYPE", dict(dtype=5)),
    ("RLPL_ERR_DTYPE", dict(mask_dtype=3)),
    ("RLPL_ERR_ALIGN", dict(s=A + 2)),
    ("RLPL_ERR_ALIGN", dict(t=A + 0x100000 + 8)),
    ("RLPL_ERR_ALIGN", dict(mask=A + 0x200000 + 1)),
    ("RLPL_ERR_ALIGN", dict(loss=A + 0x300000 + 2)),
    ("RLPL_ERR_ALIGN", dict(n=A + 0x500000 + 1)),
    ("RLPL_ERR_WORKSPACE", dict(ws=None)),
    ("RLPL_ERR_WORKSPACE", dict(ws_bytes=4096)),
    ("RLPL_ERR_ALIGN", dict(ws=WS + 64)),
]


@pytest.mark.parametrize("want,over", VOCAB_CASES, ids=[f"{w}-{list(o)[0]}" for w, o in VOCAB_CASES])
def test_reverse_kl_logits_validation(lib, want, over):
    assert rl.STATUS[call_vocab(lib, **over)] == want
    assert rl.STATUS[call_vocab(lib, fused=False, **over)] == want


def test_reverse_kl_logits_grad_pointer(lib):
    assert rl.STATUS[call_vocab(lib, grad=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_vocab(lib, grad=A + 0x400000 + 4)] == "RLPL_ERR_ALIGN"
    if not torch.cuda.is_available():
        # valid arguments stop at the device check on a host with no GPU
        assert rl.STATUS[call_vocab(lib)] == "RLPL_ERR_DEVICE"
        assert rl.STATUS[call_vocab(lib, rows=3, V=50257, dtype=0)] == "RLPL_ERR_DEVICE"


def test_launch_shape_vocab_validation(lib):
    g, v, t = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    out = (ctypes.byref(g), ctypes.byref(v), ctypes.byref(t))
    # vocab ops take (rows, vocab): 2^31 slots and more are fine there
    assert rl.STATUS[lib.rlpl_launch_shape(1 << 20, 1 << 20, 2, 6, *out)] in ("RLPL_OK", "RLPL_ERR_DEVICE")
    assert rl.STATUS[lib.rlpl_launch_shape(0, 1000, 2, 7, *out)] == "RLPL_ERR_SHAPE"


def call_ex(lib, op=0, flags=1, **over):
    a = _bnpo_args(**over)
    return lib.rlpl_policy_loss(op, flags, a["lp"], a["old"], a["ref"], a["adv"], a["mask"], a["bs"], a["T"],
                                a["dtype"], a["mask_dtype"], a["beta"], a["eps"], a["eps_high"], a["loss"],
                                a["grad"], a["n"], a["ws"], a["ws_bytes"], a["stream"])


def test_policy_loss_ex_validation(lib):
    assert rl.STATUS[call_ex(lib, flags=2)] == "RLPL_ERR_PARAM"          # unknown flag bit
    assert rl.STATUS[call_ex(lib, op=4)] == "RLPL_ERR_PARAM"             # reverse-KL is not a policy op
    assert rl.STATUS[call_ex(lib, op=0, grad=None)] == "RLPL_ERR_NULL"   # fused needs grad_out
    assert rl.STATUS[call_ex(lib, op=1, grad=None, lp=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_ex(lib, op=3, bs=0)] == "RLPL_ERR_SHAPE"
    assert rl.STATUS[call_ex(lib, op=2, eps=0.5, eps_high=-0.6)] == "RLPL_ERR_PARAM"
    if not torch.cuda.is_available():
        assert rl.STATUS[call_ex(lib, op=1, grad=None)] == "RLPL_ERR_DEVICE"   # _FWD ignores grad_out


def call_lp(lib, backward=False, **over):
    a = dict(h=A, w=A + 0x100000, b=A + 0x200000, y=A + 0x300000, lse=A + 0x400000, g=A + 0x500000,
             n=64, H=256, V=1000, dtype=2, logp=A + 0x600000, dh=A + 0x700000, dw=A + 0x800000,
             db=A + 0x900000, acc=0, ws=WS, ws_bytes=64 << 20, stream=None)
    a.update(over)
    if not backward:
        return lib.selective_logprob_fwd(a["h"], a["w"], a["b"], a["y"], a["n"], a["H"], a["V"], a["dtype"],
                                         a["logp"], a["lse"], a["ws"], a["ws_bytes"], a["stream"])
    return lib.selective_logprob_bwd(a["h"], a["w"], a["b"], a["y"], a["lse"], a["g"], a["n"], a["H"], a["V"],
                                     a["dtype"], a["dh"], a["dw"], a["db"], a["acc"], a["ws"], a["ws_bytes"],
                                     a["stream"])


LP_CASES = [
    ("RLPL_ERR_NULL", dict(h=None)),
    ("RLPL_ERR_NULL", dict(w=None)),
    ("RLPL_ERR_NULL", dict(y=None)),
    ("RLPL_ERR_SHAPE", dict(n=0)),
    ("RLPL_ERR_SHAPE", dict(H=12)),              # not a multiple of 8
    ("RLPL_ERR_SHAPE", dict(H=0)),
    ("RLPL_ERR_SHAPE", dict(H=65544)),
    ("RLPL_ERR_SHAPE", dict(V=0)),
    ("RLPL_ERR_SHAPE", dict(V=1 << 26)),
    ("RLPL_ERR_DTYPE", dict(dtype=0)),           # fp32 operands are not taken
    ("RLPL_ERR_DTYPE", dict(dtype=7)),
    ("RLPL_ERR_ALIGN", dict(h=A + 8)),
    ("RLPL_ERR_ALIGN", dict(w=A + 0x100000 + 2)),
    ("RLPL_ERR_ALIGN", dict(b=A + 0x200000 + 1)),
    ("RLPL_ERR_ALIGN", dict(y=A + 0x300000 + 4)),
    ("RLPL_ERR_WORKSPACE", dict(ws=None)),
    ("RLPL_ERR_WORKSPACE", dict(ws_bytes=256)),
    ("RLPL_ERR_ALIGN", dict(ws=WS + 64)),
]


@pytest.mark.parametrize("want,over", LP_CASES, ids=[f"{w}-{list(o)[0]}" for w, o in LP_CASES])
def test_selective_logprob_validation(lib, want, over):
    assert rl.STATUS[call_lp(lib, **over)] == want
    assert rl.STATUS[call_lp(lib, backward=True, **over)] == want


def test_selective_logprob_outputs_and_workspace(lib):
    assert rl.STATUS[call_lp(lib, logp=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_lp(lib, logp=A + 0x600000 + 2)] == "RLPL_ERR_ALIGN"
    assert rl.STATUS[call_lp(lib, backward=True, lse=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_lp(lib, backward=True, g=None)] == "RLPL_ERR_NULL"
    assert rl.STATUS[call_lp(lib, backward=True, dw=A + 0x800000 + 2)] == "RLPL_ERR_ALIGN"
    fwd = lib.selective_logprob_workspace_bytes(1024, 4096, 128256, 0)
    bwd = lib.selective_logprob_workspace_bytes(1024, 4096, 128256, 1)
    # forward: per-tile (max, sum) pairs and target logits of one 1024-token group
    assert fwd >= 1024 * 501 * 8 + 1024 * 4 and fwd < 9 << 20
    # backward: the group's logits gradient (bf16, rows padded to 8), four fp32 planes of
    # (1024, 4096) and the column sums of four 256-row tiles
    assert bwd >= 1024 * 128256 * 2 + 4 * 1024 * 4096 * 4 + 4 * 128256 * 4 and bwd < 320 << 20
    assert lib.selective_logprob_workspace_bytes(5000, 4096, 128256, 1) == bwd   # sized by the group, not n
    assert lib.selective_logprob_workspace_bytes(0, 4096, 128256, 1) == 0
    assert lib.selective_logprob_workspace_bytes(8, 100, 1000, 0) == 0
    if not torch.cuda.is_available():
        assert rl.STATUS[call_lp(lib)] == "RLPL_ERR_DEVICE"
        assert rl.STATUS[call_lp(lib, backward=True, dh=None, dw=None, db=None, b=None)] == "RLPL_ERR_DEVICE"
