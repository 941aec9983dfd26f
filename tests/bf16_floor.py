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


def _rotation(S: int, d: int, theta: float):
    """cos and sin [S][d/2] of the rotary angles i * theta^(-2c/d), from fp64."""
    half = d // 2
    w = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * w[None, :]
    return torch.cos(ang).float(), torch.sin(ang).float()


def _rotate(x, cs, sn, sign):
    """Rotate-half rotation of the last dim of x [heads][S][d]; sign -1 is the
    transpose (for gradients)."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    sn = sn * sign
    return torch.cat([a * cs - b * sn, b * cs + a * sn], dim=-1)


def _rms_fwd(x, gamma, eps):
    """QK-norm in fp32: returns gamma * xhat, xhat and 1/rms [..., 1]."""
    r = torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + eps)
    xh = x * r
    return xh * gamma, xh, r


def _rms_bwd(g, xh, r, gamma):
    """gradient of the unnormalised rows for g = gradient of gamma * xhat."""
    t = (gamma * g * xh).sum(-1, keepdim=True) / xh.shape[-1]
    return r * (gamma * g - xh * t)


def bf16_path_emulation(inp, H: int, G: int, d: int, causal: bool = True,
                        rope_theta: float = 0.0, out_proj: bool = False,
                        round_grads: bool = True, qk_norm_eps=None) -> dict:
    """With rope_theta > 0, queries and keys are rotated in fp32 before their
    rounding, and dQ, dK take the transposed rotation before theirs.  With
    out_proj, Y = O Wo^T and dWo = dY^T O in fp32 from the stored O, and the
    attention backward runs with dO = dY Wo rounded to bf16 once.
    round_grads=False keeps dQ, dK, dV in fp32 for the gradient products (a
    variant the kernels do not implement; it isolates that rounding point).
    qk_norm_eps (with inp["q_norm"], inp["k_norm"]) adds QK-norm in fp32
    before the rotation and rounding; its backward runs on the fp32
    gradients, and dq_norm / dk_norm are returned as well."""
    bf = lambda t: t.to(torch.bfloat16).float()
    bfg = bf if round_grads else (lambda t: t)
    X, Wq, Wk, Wv = [inp[k].detach().cpu().float() for k in ("X", "Wq", "Wk", "Wv")]
    if out_proj:
        Wo, dY = inp["Wo"].detach().cpu().float(), inp["dY"].detach().cpu().float()
        dO = bf(dY @ Wo)
    else:
        dO = inp["dO"].detach().cpu().float()
    S = X.shape[0]
    r = H // G
    tau = 1.0 / math.sqrt(d)
    if rope_theta > 0:
        cs, sn = _rotation(S, d, rope_theta)
        rot = lambda t, sign: _rotate(t, cs, sn, sign)
    else:
        rot = lambda t, sign: t
    qn = qk_norm_eps is not None
    qp = (X @ Wq.T).reshape(S, H, d).transpose(0, 1)
    kp = (X @ Wk.T).reshape(S, G, d).transpose(0, 1)
    if qn:
        gq, gk = inp["q_norm"].detach().cpu().float(), inp["k_norm"].detach().cpu().float()
        qp, xq, rq = _rms_fwd(qp, gq, qk_norm_eps)
        kp, xk, rk = _rms_fwd(kp, gk, qk_norm_eps)
    Q = bf(rot(qp, 1))
    K = bf(rot(kp, 1)).repeat_interleave(r, 0)
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
    dQ = rot(tau * (bf(dS) @ K), -1)
    dKh = bf(dS).transpose(1, 2).contiguous() @ Q
    dVh = bf(P).transpose(1, 2).contiguous() @ go
    dK = rot(tau * dKh.reshape(G, r, S, d).sum(1), -1)
    extra = {}
    if qn:
        extra["dq_norm"] = (dQ * xq).sum((0, 1))
        extra["dk_norm"] = (dK * xk).sum((0, 1))
        dQ = _rms_bwd(dQ, xq, rq, gq)
        dK = _rms_bwd(dK, xk, rk, gk)
    dQ = bfg(dQ)
    dK = bfg(dK)
    dV = bfg(dVh.reshape(G, r, S, d).sum(1))
    dQf = dQ.transpose(0, 1).reshape(S, H * d)
    dKf = dK.transpose(0, 1).reshape(S, G * d)
    dVf = dV.transpose(0, 1).reshape(S, G * d)
    if out_proj:
        Of = O.transpose(0, 1).reshape(S, H * d)
        extra.update({"Y": Of @ Wo.T, "dWo": dY.T @ Of})
    return {
        **extra,
        "O": O.transpose(0, 1).reshape(S, H * d),
        "LSE": lse,
        "dX": dQf @ Wq + dKf @ Wk + dVf @ Wv,
        "dWq": dQf.T @ X,
        "dWk": dKf.T @ X,
        "dWv": dVf.T @ X,
    }
