"""Error floor of the bf16 path, for diagnostics in the GPU parity tests.

Emulates, with fp32 torch on the CPU, the rounding points the bf16 kernels
use: Q, K, V and O stored in bf16; P and dS rounded to bf16 at the matrix-core
inputs; dQ, dK, dV rounded to bf16 before the weight and input gradient
products; everything else fp32.  Comparing this emulation with the fp64 oracle
gives the error any implementation with these rounding points makes; the GPU
must not exceed it by more than a small factor (it would if a kernel added a
rounding step or lost precision).  This is test code only: it shares nothing
with the HIP library and is not an oracle.
"""
from __future__ import annotations

import math

import torch


def bf16_path_emulation(inp, H: int, G: int, d: int, causal: bool = True) -> dict:
    bf = lambda t: t.to(torch.bfloat16).float()
    X, Wq, Wk, Wv, dO = [inp[k].detach().cpu().float() for k in ("X", "Wq", "Wk", "Wv", "dO")]
    S = X.shape[0]
    r = H // G
    tau = 1.0 / math.sqrt(d)
    Q = bf(X @ Wq.T).reshape(S, H, d).transpose(0, 1)
    K = bf(X @ Wk.T).reshape(S, G, d).transpose(0, 1).repeat_interleave(r, 0)
    V = bf(X @ Wv.T).reshape(S, G, d).transpose(0, 1).repeat_interleave(r, 0)
    s = (Q @ K.transpose(1, 2).contiguous()) * tau
    if causal:
        mask = torch.ones(S, S, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    m = s.amax(-1, keepdim=True)
    pt = torch.exp(s - m)
    l = pt.sum(-1, keepdim=True)
    O = bf((bf(pt) @ V) / l)
    lse = (m + torch.log(l)).squeeze(-1)
    go = dO.reshape(S, H, d).transpose(0, 1)
    Dd = (go * O).sum(-1, keepdim=True)
    P = torch.exp(s - lse[..., None])
    dP = go @ V.transpose(1, 2).contiguous()
    dS = P * (dP - Dd)
    dQ = bf(tau * (bf(dS) @ K))
    dKh = bf(dS).transpose(1, 2).contiguous() @ Q
    dVh = bf(P).transpose(1, 2).contiguous() @ go
    dK = bf(tau * dKh.reshape(G, r, S, d).sum(1))
    dV = bf(dVh.reshape(G, r, S, d).sum(1))
    dQf = dQ.transpose(0, 1).reshape(S, H * d)
    dKf = dK.transpose(0, 1).reshape(S, G * d)
    dVf = dV.transpose(0, 1).reshape(S, G * d)
    return {
        "O": O.transpose(0, 1).reshape(S, H * d),
        "LSE": lse,
        "dX": dQf @ Wq + dKf @ Wk + dVf @ Wv,
        "dWq": dQf.T @ X,
        "dWk": dKf.T @ X,
        "dWv": dVf.T @ X,
    }
