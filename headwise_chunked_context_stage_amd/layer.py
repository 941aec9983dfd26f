"""Caller-side helpers: allocate the tensors the C ABI writes (torch is used for
device memory and streams only) and run the layer through the binding."""
from __future__ import annotations

import torch

from . import upipe
from .synth import torch_dtype


def alloc_outputs(plan: "upipe.Plan", device, backward: bool = True, ws_extra: int = 0):
    """O, LSE, the workspace (peak_bytes, 256-byte aligned by torch's allocator)
    and, for the backward, dX and the three weight gradients (fp32)."""
    S, D, H, G, d = plan.S, plan.D, plan.H, plan.G, plan.d
    td = torch_dtype(plan.dtype)
    out = {
        "O": torch.empty((S, H * d), dtype=td, device=device),
        "LSE": torch.empty((H, S), dtype=torch.float32, device=device),
        "ws": torch.empty((max(1, plan.peak_bytes + ws_extra),), dtype=torch.uint8, device=device),
    }
    if backward:
        out["dX"] = torch.empty((S, D), dtype=torch.float32, device=device)
        out["dWq"] = torch.empty((H * d, D), dtype=torch.float32, device=device)
        out["dWk"] = torch.empty((G * d, D), dtype=torch.float32, device=device)
        out["dWv"] = torch.empty((G * d, D), dtype=torch.float32, device=device)
    return out


def forward(plan, inp, out, stream=None):
    plan.fwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], out["O"], out["LSE"], out["ws"],
             stream=stream)


def backward(plan, inp, out, stream=None):
    plan.bwd(inp["dO"], inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], out["O"], out["LSE"], out["dX"],
             out["dWq"], out["dWk"], out["dWv"], out["ws"], stream=stream)


def run(plan, inp, backward_pass: bool = True, stream=None):
    """Forward (and backward) on the current stream; returns the output dict."""
    dev = inp["X"].device
    out = alloc_outputs(plan, dev, backward=backward_pass)
    forward(plan, inp, out, stream)
    if backward_pass:
        backward(plan, inp, out, stream)
    return out


def run_out(plan, inp, backward_pass: bool = True, stream=None):
    """The layer with its output projection (plan created with out_proj=True;
    inputs also hold Wo [D][H*d] and dY [S][D]): forward into O, LSE and
    Y (fp32 [S][D]), and the backward into dX, dWq, dWk, dWv, dWo (fp32)."""
    dev = inp["X"].device
    out = alloc_outputs(plan, dev, backward=backward_pass)
    out["Y"] = torch.empty((plan.S, plan.D), dtype=torch.float32, device=dev)
    plan.fwd_out(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], out["O"], out["LSE"],
                 out["Y"], out["ws"], stream=stream)
    if backward_pass:
        out["dWo"] = torch.empty((plan.D, plan.H * plan.d), dtype=torch.float32, device=dev)
        plan.bwd_out(inp["dY"], inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], out["O"],
                     out["LSE"], out["dX"], out["dWq"], out["dWk"], out["dWv"], out["dWo"],
                     out["ws"], stream=stream)
    return out


def run_ex(plan, inp, backward_pass: bool = True, stream=None):
    """Any plan through upipe_fwd_ex / upipe_bwd_ex: the QK-norm weights
    (q_norm, k_norm) and the output projection (Wo, dY) are taken from `inp`
    when the plan uses them; returns O, LSE (and Y) and, for the backward,
    dX, dWq, dWk, dWv (and dq_norm, dk_norm, dWo)."""
    dev = inp["X"].device
    out = alloc_outputs(plan, dev, backward=backward_pass)
    io = {k: inp[k] for k in ("X", "Wq", "Wk", "Wv")}
    io.update(O=out["O"], LSE=out["LSE"])
    if plan.qk_norm:
        io.update(q_norm=inp["q_norm"], k_norm=inp["k_norm"])
    if plan.out_proj:
        out["Y"] = torch.empty((plan.S, plan.D), dtype=torch.float32, device=dev)
        io.update(Wo=inp["Wo"], Y=out["Y"])
    plan.fwd_ex(io, out["ws"], stream=stream)
    if backward_pass:
        bio = {k: io[k] for k in ("X", "Wq", "Wk", "Wv", "O", "LSE")}
        bio.update({k: out[k] for k in ("dX", "dWq", "dWk", "dWv")})
        if plan.qk_norm:
            out["dq_norm"] = torch.empty((plan.d,), dtype=torch.float32, device=dev)
            out["dk_norm"] = torch.empty((plan.d,), dtype=torch.float32, device=dev)
            bio.update(q_norm=inp["q_norm"], k_norm=inp["k_norm"], dq_norm=out["dq_norm"],
                       dk_norm=out["dk_norm"])
        if plan.out_proj:
            out["dWo"] = torch.empty((plan.D, plan.H * plan.d), dtype=torch.float32, device=dev)
            bio.update(Wo=inp["Wo"], dY=inp["dY"], dWo=out["dWo"])
        else:
            bio["dO"] = inp["dO"]
        plan.bwd_ex(bio, out["ws"], stream=stream)
    return out
