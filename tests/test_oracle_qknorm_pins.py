"""Pins for the oracle's QK-norm (per-head RMS normalisation of queries and
keys with weights gamma_q, gamma_k shared by the heads, before the rotary
embedding), each against something other than the oracle itself:

* torch's own fp64 rms_norm + scaled_dot_product_attention + autograd (library
  routines the oracle never calls), every output including the two weight
  gradients, causal and full, with and without the rotary embedding;
* central finite differences of L = sum(O * dO) in gamma_q, gamma_k, X, Wq;
* invariances that hold for the exact layer: scaling gamma_q by a and gamma_k
  by 1/a leaves every score unchanged, so <dgamma_q, gamma_q> =
  <dgamma_k, gamma_k>; with eps = 0 the layer does not depend on the scale of
  Wq or of Wk, so <dWq, Wq> = <dWk, Wk> = 0;
* closed form: gamma_q = 0 makes every score 0 (uniform attention: prefix
  means of V, LSE = ln(i + 1)), and then dgamma_k = 0 and dWk = 0.

QK-norm is not on the pages; it belongs to the Qwen3 family whose attention
shape the pages train (paper.rainbus.top summary of "Untied Ulysses",
section 实验结果), and a drop-in attention module for it has to include it.
"""
import math

import numpy as np
import pytest
import torch

from test_oracle_pins import close, draw

EPS = 1e-6


def draw_norm(d, seed):
    rng = np.random.default_rng(seed)
    return 1.0 + 0.3 * rng.standard_normal(d), 1.0 + 0.3 * rng.standard_normal(d)


def torch_layer_qkn(X, Wq, Wk, Wv, dO, gq, gk, H, G, d, causal, theta=0.0, eps=EPS):
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k != "dO"))
         for k, v in dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv, dO=dO, gq=gq, gk=gk).items()}
    S = X.shape[0]
    F = torch.nn.functional

    def rope(x):
        if theta == 0.0:
            return x
        half = d // 2
        freq = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
        ang = torch.arange(S, dtype=torch.float64)[:, None] * freq[None, :]
        z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
        return torch.cat([z.real, z.imag], dim=-1)

    q = (t["X"] @ t["Wq"].T).reshape(S, H, d).transpose(0, 1)
    k = (t["X"] @ t["Wk"].T).reshape(S, G, d).transpose(0, 1)
    q = rope(F.rms_norm(q, (d,), weight=t["gq"], eps=eps))
    k = rope(F.rms_norm(k, (d,), weight=t["gk"], eps=eps))
    v = (t["X"] @ t["Wv"].T).reshape(S, G, d).transpose(0, 1)
    k = k.repeat_interleave(H // G, dim=0)
    v = v.repeat_interleave(H // G, dim=0)
    o = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=causal)[0]
    O = o.transpose(0, 1).reshape(S, H * d)
    (O * t["dO"]).sum().backward()
    scores = (q @ k.transpose(1, 2)) / math.sqrt(d)
    if causal:
        scores = scores.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
    return dict(O=O.detach().numpy(), LSE=torch.logsumexp(scores, -1).detach().numpy(),
                dX=t["X"].grad.numpy(), dWq=t["Wq"].grad.numpy(), dWk=t["Wk"].grad.numpy(),
                dWv=t["Wv"].grad.numpy(), dq_norm=t["gq"].grad.numpy(),
                dk_norm=t["gk"].grad.numpy())


@pytest.mark.parametrize("shape", [(37, 24, 4, 2, 8), (29, 16, 3, 3, 8), (50, 24, 8, 1, 8)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("theta", [0.0, 10000.0])
def test_qknorm_against_torch_library(oracle_mod, shape, causal, theta):
    S, D, H, G, d = shape
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=S + 7)
    gq, gk = draw_norm(d, seed=S)
    got = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal, rope_theta=theta,
                              q_norm=gq, k_norm=gk, qk_eps=EPS)
    ref = torch_layer_qkn(X, Wq, Wk, Wv, dO, gq, gk, H, G, d, causal, theta)
    for name in ("O", "LSE", "dX", "dWq", "dWk", "dWv", "dq_norm", "dk_norm"):
        close(got[name], ref[name])
    O, LSE = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d, causal=causal, rope_theta=theta,
                                q_norm=gq, k_norm=gk, qk_eps=EPS)
    np.testing.assert_array_equal(O, got["O"])
    np.testing.assert_array_equal(LSE, got["LSE"])
    plain = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d, causal=causal, rope_theta=theta)[0]
    assert np.abs(plain - O).max() > 1e-3  # the normalisation is applied
    rows = [0, 3, S // 2, S - 1]
    Or, Lr = oracle_mod.forward_rows(X, Wq, Wk, Wv, H, G, d, rows, causal=causal, rope_theta=theta,
                                     q_norm=gq, k_norm=gk, qk_eps=EPS)
    close(Or, O[rows])
    close(Lr, LSE[:, rows])


def test_qknorm_finite_differences(oracle_mod):
    S, D, H, G, d = 21, 12, 4, 2, 8
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=3)
    gq, gk = draw_norm(d, seed=4)
    kw = dict(causal=True, rope_theta=100.0, qk_eps=1e-3)
    g = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, q_norm=gq, k_norm=gk, **kw)

    def loss(X_, Wq_, gq_, gk_):
        O, _ = oracle_mod.forward(X_, Wq_, Wk, Wv, H, G, d, q_norm=gq_, k_norm=gk_,
                                  causal=kw["causal"], rope_theta=kw["rope_theta"],
                                  qk_eps=kw["qk_eps"])
        return float((O * dO).sum())

    rng = np.random.default_rng(5)
    args = {"X": X, "Wq": Wq, "gq": gq, "gk": gk}
    grads = {"X": g["dX"], "Wq": g["dWq"], "gq": g["dq_norm"], "gk": g["dk_norm"]}
    for name in ("gq", "gk", "X", "Wq"):
        for _ in range(8):
            idx = tuple(rng.integers(0, n) for n in args[name].shape)
            a = {k: v.copy() for k, v in args.items()}
            h = 1e-6 * max(1.0, abs(a[name][idx]))
            a[name][idx] += h
            up = loss(a["X"], a["Wq"], a["gq"], a["gk"])
            a[name][idx] -= 2 * h
            dn = loss(a["X"], a["Wq"], a["gq"], a["gk"])
            fd = (up - dn) / (2 * h)
            assert abs(fd - grads[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd,
                                                                          grads[name][idx])


@pytest.mark.parametrize("causal", [True, False])
def test_qknorm_invariances(oracle_mod, causal):
    S, D, H, G, d = 40, 24, 4, 2, 8
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=11)
    gq, gk = draw_norm(d, seed=12)
    g = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal, q_norm=gq, k_norm=gk,
                            qk_eps=EPS, rope_theta=500.0)
    a, b = float(g["dq_norm"] @ gq), float(g["dk_norm"] @ gk)
    assert abs(a - b) <= 1e-10 * max(1.0, abs(a)), (a, b)
    g0 = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal, q_norm=gq, k_norm=gk,
                             qk_eps=0.0)
    for dw, w in ((g0["dWq"], Wq), (g0["dWk"], Wk)):
        ip = float((dw * w).sum())
        assert abs(ip) <= 1e-10 * np.linalg.norm(dw) * np.linalg.norm(w), ip
    # with eps > 0 the scale of Wq matters a little
    ip = float((g["dWq"] * Wq).sum())
    assert ip != 0.0


def test_qknorm_zero_query_weight_gives_uniform_attention(oracle_mod):
    S, D, H, G, d = 33, 16, 4, 2, 8
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=21)
    gq, gk = draw_norm(d, seed=22)
    gq[:] = 0.0
    g = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=True, q_norm=gq, k_norm=gk,
                            qk_eps=EPS)
    V = X @ Wv.T
    prefix = np.cumsum(V, axis=0) / np.arange(1, S + 1)[:, None]
    for h in range(H):
        kv = h // (H // G)
        close(g["O"][:, h * d:(h + 1) * d], prefix[:, kv * d:(kv + 1) * d], 1e-12)
        close(g["LSE"][h], np.log(np.arange(1, S + 1)), 1e-12)
    assert np.all(g["dk_norm"] == 0.0) and np.all(g["dWk"] == 0.0)
    assert np.abs(g["dq_norm"]).max() > 0.0
