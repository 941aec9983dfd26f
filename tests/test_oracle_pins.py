"""Pins for the fp64 oracle, each against something other than the oracle itself.

* torch CPU fp64 scaled_dot_product_attention + autograd (a library routine the
  oracle never calls) for every output, causal and full, GQA/MHA/single head;
* brute force: the whole masked S x S score matrix softmaxed at once (scipy);
* central finite differences of L = sum(O * dO) for the backward;
* closed forms: S = 1, row 0, uniform attention when Wq = 0 (prefix means,
  LSE = ln(i+1), dWk = 0 exactly, dWv from prefix sums);
* causal invariance (future rows do not change earlier outputs, bitwise);
* softmax rows sum to one; scaling identities that hold at any size;
* independence of the thread count (bitwise).

The definition being pinned: paper.rainbus.top summary of "Untied Ulysses",
section 前置知识 (Ulysses: full attention per head over all positions; GQA:
H/G consecutive query heads share a KV head) and section 方法步骤详情 (each
stage projects its heads' Q, K, V from X, then attends over the full sequence).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

SHAPES = [
    # S, D, H, G, d
    (37, 24, 4, 2, 8),     # GQA, ragged S
    (64, 32, 6, 3, 16),    # GQA r=2
    (29, 16, 3, 3, 8),     # MHA (G = H)
    (33, 20, 1, 1, 12),    # single head
    (50, 24, 8, 1, 8),     # MQA (G = 1)
]


def draw(S, D, H, G, d, seed=0, wq_zero=False):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((S, D))
    Wq = rng.standard_normal((H * d, D)) / math.sqrt(D)
    Wk = rng.standard_normal((G * d, D)) / math.sqrt(D)
    Wv = rng.standard_normal((G * d, D)) / math.sqrt(D)
    dO = rng.standard_normal((S, H * d))
    if wq_zero:
        Wq[:] = 0.0
    return X, Wq, Wk, Wv, dO


def torch_layer(X, Wq, Wk, Wv, dO, H, G, d, causal):
    """The same layer built from torch library calls, fp64, autograd backward."""
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k != "dO"))
         for k, v in dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv, dO=dO).items()}
    S = X.shape[0]
    q = (t["X"] @ t["Wq"].T).reshape(S, H, d).transpose(0, 1)
    k = (t["X"] @ t["Wk"].T).reshape(S, G, d).transpose(0, 1)
    v = (t["X"] @ t["Wv"].T).reshape(S, G, d).transpose(0, 1)
    k = k.repeat_interleave(H // G, dim=0)
    v = v.repeat_interleave(H // G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None],
                                                         is_causal=causal)[0]
    O = o.transpose(0, 1).reshape(S, H * d)
    (O * t["dO"]).sum().backward()
    scores = (q @ k.transpose(1, 2)) / math.sqrt(d)
    if causal:
        mask = torch.ones(S, S, dtype=torch.bool).tril()
        scores = scores.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    return dict(O=O.detach().numpy(), LSE=lse.detach().numpy(), dX=t["X"].grad.numpy(),
                dWq=t["Wq"].grad.numpy(), dWk=t["Wk"].grad.numpy(), dWv=t["Wv"].grad.numpy())


def close(a, b, tol=1e-10):
    scale = max(1.0, float(np.max(np.abs(b))))
    err = float(np.max(np.abs(a - b))) / scale
    assert err <= tol, "max rel err %.3e > %.1e" % (err, tol)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_library(oracle_mod, shape, causal):
    S, D, H, G, d = shape
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=S)
    got = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal)
    ref = torch_layer(X, Wq, Wk, Wv, dO, H, G, d, causal)
    for name in ("O", "LSE", "dX", "dWq", "dWk", "dWv"):
        close(got[name], ref[name])
    # forward entry point agrees with the forward half of the backward one
    O, LSE = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d, causal=causal)
    np.testing.assert_array_equal(O, got["O"])
    np.testing.assert_array_equal(LSE, got["LSE"])


@pytest.mark.parametrize("shape", SHAPES[:3])
def test_brute_force_score_matrix(oracle_mod, shape):
    S, D, H, G, d = shape
    X, Wq, Wk, Wv, _ = draw(S, D, H, G, d, seed=1)
    O, LSE = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d)
    r = H // G
    mask = np.tril(np.ones((S, S), bool))
    for h in range(H):
        g = h // r
        q = X @ Wq[h * d:(h + 1) * d].T
        k = X @ Wk[g * d:(g + 1) * d].T
        v = X @ Wv[g * d:(g + 1) * d].T
        sc = np.where(mask, (q @ k.T) / math.sqrt(d), -np.inf)
        P = scipy.special.softmax(sc, axis=1)
        close(O[:, h * d:(h + 1) * d], P @ v, 1e-12)
        close(LSE[h], scipy.special.logsumexp(sc, axis=1), 1e-12)
        # rows of the softmax sum to one, with the oracle's own LSE
        Pl = np.where(mask, np.exp(sc - LSE[h][:, None]), 0.0)
        assert np.max(np.abs(Pl.sum(axis=1) - 1.0)) <= 1e-12


@pytest.mark.parametrize("shape", [(23, 12, 4, 2, 6), (19, 10, 2, 1, 5)])
@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences(oracle_mod, shape, causal):
    S, D, H, G, d = shape
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=7)
    g = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal)
    params = dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv)
    rng = np.random.default_rng(3)

    def loss(p):
        O, _ = oracle_mod.forward(p["X"], p["Wq"], p["Wk"], p["Wv"], H, G, d, causal=causal,
                                  nthreads=1)
        return float(np.sum(O * dO))

    for name, grad in (("X", "dX"), ("Wq", "dWq"), ("Wk", "dWk"), ("Wv", "dWv")):
        for _ in range(20):
            idx = tuple(int(rng.integers(0, n)) for n in params[name].shape)
            base = params[name][idx]
            eps = 1e-6 * max(1.0, abs(base))
            plus = {k: v.copy() for k, v in params.items()}
            minus = {k: v.copy() for k, v in params.items()}
            plus[name][idx] = base + eps
            minus[name][idx] = base - eps
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = g[grad][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


def test_single_token(oracle_mod):
    S, D, H, G, d = 1, 16, 4, 2, 8
    X, Wq, Wk, Wv, _ = draw(S, D, H, G, d, seed=11)
    O, LSE = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d)
    for h in range(H):
        g = h // 2
        q = X[0] @ Wq[h * d:(h + 1) * d].T
        k = X[0] @ Wk[g * d:(g + 1) * d].T
        v = X[0] @ Wv[g * d:(g + 1) * d].T
        close(O[0, h * d:(h + 1) * d], v, 1e-14)
        close(LSE[h, 0], q @ k / math.sqrt(d), 1e-14)


def test_row_zero_is_first_value(oracle_mod):
    S, D, H, G, d = 40, 16, 4, 1, 8
    X, Wq, Wk, Wv, _ = draw(S, D, H, G, d, seed=12)
    O, _ = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d)
    v0 = X[0] @ Wv[0:d].T
    for h in range(H):
        close(O[0, h * d:(h + 1) * d], v0, 1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_uniform_attention_when_wq_zero(oracle_mod, causal):
    """Wq = 0 makes every score 0: P_ij = 1/n_i, O is a (prefix) mean of V,
    LSE = ln n_i, Q = 0 so dK = 0 and dWk = 0 exactly, and
    dV_j = sum_h sum_{i sees j} dO_i / n_i."""
    S, D, H, G, d = 31, 12, 4, 2, 6
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=13, wq_zero=True)
    out = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal)
    n = np.arange(1, S + 1, dtype=np.float64) if causal else np.full(S, float(S))
    r = H // G
    for h in range(H):
        g = h // r
        v = X @ Wv[g * d:(g + 1) * d].T
        mean = np.cumsum(v, axis=0) / n[:, None] if causal else np.broadcast_to(v.mean(0), v.shape)
        close(out["O"][:, h * d:(h + 1) * d], mean, 1e-13)
        close(out["LSE"][h], np.log(n), 1e-14)
    assert np.all(out["dWk"] == 0.0)
    for g in range(G):
        w = np.zeros((S, d))
        for h in range(g * r, (g + 1) * r):
            w += dO[:, h * d:(h + 1) * d] / n[:, None]
        # dV_j = sum_{i >= j} w_i (causal) or sum_i w_i (full): a reverse prefix sum
        dV = np.cumsum(w[::-1], axis=0)[::-1] if causal else np.broadcast_to(w.sum(0), w.shape)
        close(out["dWv"][g * d:(g + 1) * d], dV.T @ X, 1e-12)


def test_causal_invariance(oracle_mod):
    S, D, H, G, d = 48, 16, 4, 2, 8
    X, Wq, Wk, Wv, _ = draw(S, D, H, G, d, seed=14)
    O1, L1 = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d)
    t = 20
    X2 = X.copy()
    X2[t + 1:] = np.random.default_rng(99).standard_normal(X2[t + 1:].shape)
    O2, L2 = oracle_mod.forward(X2, Wq, Wk, Wv, H, G, d)
    np.testing.assert_array_equal(O1[:t + 1], O2[:t + 1])
    np.testing.assert_array_equal(L1[:, :t + 1], L2[:, :t + 1])
    assert not np.array_equal(O1[t + 1:], O2[t + 1:])


@pytest.mark.parametrize("causal", [True, False])
def test_scaling_identities(oracle_mod, causal):
    """<dWv,Wv> = <dO,O> (O is linear in Wv); <dWq,Wq> = <dWk,Wk> (scores are
    unchanged by Wq*a, Wk/a); <dX,X> = sum of <dW,W> (X*a equals all W*a)."""
    S, D, H, G, d = 45, 20, 6, 2, 8
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=15)
    o = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal)
    ip = lambda a, b: float(np.sum(a * b))
    assert abs(ip(o["dWv"], Wv) - ip(dO, o["O"])) <= 1e-10 * abs(ip(dO, o["O"])) + 1e-10
    assert abs(ip(o["dWq"], Wq) - ip(o["dWk"], Wk)) <= 1e-10 * abs(ip(o["dWq"], Wq)) + 1e-10
    tot = ip(o["dWq"], Wq) + ip(o["dWk"], Wk) + ip(o["dWv"], Wv)
    assert abs(ip(o["dX"], X) - tot) <= 1e-10 * abs(tot) + 1e-10


def test_thread_count_independent(oracle_mod):
    S, D, H, G, d = 41, 16, 4, 2, 8
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=16)
    a = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, nthreads=1)
    b = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, nthreads=5)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_sampled_rows_match_full(oracle_mod):
    S, D, H, G, d = 70, 16, 4, 2, 8
    X, Wq, Wk, Wv, _ = draw(S, D, H, G, d, seed=17)
    O, LSE = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d)
    rows = [0, 1, 33, 69, 5]
    Or, Lr = oracle_mod.forward_rows(X, Wq, Wk, Wv, H, G, d, rows)
    np.testing.assert_array_equal(Or, O[rows])
    np.testing.assert_array_equal(Lr, LSE[:, rows])


def test_input_encodings_decode_exactly(oracle_mod):
    """bf16 bit patterns and fp32 storage decode to the values they hold."""
    S, D, H, G, d = 20, 16, 2, 1, 8
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=18)
    tb = [torch.tensor(a, dtype=torch.float32).to(torch.bfloat16) for a in (X, Wq, Wk, Wv, dO)]
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in tb]
    vals = [t.to(torch.float64).numpy() for t in tb]
    a = oracle_mod.backward(*bits, H, G, d)
    b = oracle_mod.backward(*vals, H, G, d)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    f32 = [np.asarray(v, np.float32) for v in (X, Wq, Wk, Wv)]
    c = oracle_mod.forward(*f32, H, G, d)
    e = oracle_mod.forward(*[v.astype(np.float64) for v in f32], H, G, d)
    np.testing.assert_array_equal(c[0], e[0])


def test_rejects_bad_shapes(oracle_mod):
    X, Wq, Wk, Wv, _ = draw(8, 8, 3, 2, 4)  # G does not divide H
    with pytest.raises(ValueError):
        oracle_mod.forward(X, Wq, Wk, Wv, 3, 2, 4)


def test_sampled_rows_head_subset(oracle_mod):
    S, D, H, G, d = 40, 16, 6, 3, 8
    X, Wq, Wk, Wv, _ = draw(S, D, H, G, d, seed=19)
    O, LSE = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d)
    rows = [39, 0, 7]
    Or, Lr = oracle_mod.forward_rows(X, Wq, Wk, Wv, H, G, d, rows, heads=(1, 4))
    np.testing.assert_array_equal(Or[:, d:4 * d], O[rows][:, d:4 * d])
    np.testing.assert_array_equal(Lr[1:4], LSE[1:4][:, rows])
    assert np.all(np.isnan(Or[:, :d])) and np.all(np.isnan(Lr[4:]))


# ------------------------------------------------------------ rotary embedding
# Rotate-half rotary position embedding (an option of the layer, from the model
# families that run it, not from the pages): the pair (c, c + d/2) of a query
# or key row at position i turns by i * theta^(-2c/d).

def torch_layer_rope(X, Wq, Wk, Wv, dO, H, G, d, causal, theta):
    """torch fp64 reference with the rotation written as a complex product
    (z_c = x_c + i x_{c+d/2} times exp(i * angle)), autograd backward."""
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k != "dO"))
         for k, v in dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv, dO=dO).items()}
    S = X.shape[0]
    half = d // 2
    freq = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * freq[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)  # [S][half] complex

    def rope(x):  # x [heads][S][d]
        z = torch.complex(x[..., :half], x[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    q = rope((t["X"] @ t["Wq"].T).reshape(S, H, d).transpose(0, 1))
    k = rope((t["X"] @ t["Wk"].T).reshape(S, G, d).transpose(0, 1))
    v = (t["X"] @ t["Wv"].T).reshape(S, G, d).transpose(0, 1)
    k = k.repeat_interleave(H // G, dim=0)
    v = v.repeat_interleave(H // G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None],
                                                         is_causal=causal)[0]
    O = o.transpose(0, 1).reshape(S, H * d)
    (O * t["dO"]).sum().backward()
    scores = (q @ k.transpose(1, 2)) / math.sqrt(d)
    if causal:
        mask = torch.ones(S, S, dtype=torch.bool).tril()
        scores = scores.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    return dict(O=O.detach().numpy(), LSE=lse.detach().numpy(), dX=t["X"].grad.numpy(),
                dWq=t["Wq"].grad.numpy(), dWk=t["Wk"].grad.numpy(), dWv=t["Wv"].grad.numpy())


@pytest.mark.parametrize("shape", [(37, 24, 4, 2, 8), (29, 16, 3, 3, 8), (50, 24, 8, 1, 8)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("theta", [10000.0, 3.0])
def test_rope_against_torch_complex_rotation(oracle_mod, shape, causal, theta):
    S, D, H, G, d = shape
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=S + 1)
    got = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal, rope_theta=theta)
    ref = torch_layer_rope(X, Wq, Wk, Wv, dO, H, G, d, causal, theta)
    for name in ("O", "LSE", "dX", "dWq", "dWk", "dWv"):
        close(got[name], ref[name])
    O, LSE = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d, causal=causal, rope_theta=theta)
    np.testing.assert_array_equal(O, got["O"])
    np.testing.assert_array_equal(LSE, got["LSE"])
    rows = [0, 5, S - 1]
    Or, Lr = oracle_mod.forward_rows(X, Wq, Wk, Wv, H, G, d, rows, causal=causal, rope_theta=theta)
    close(Or, O[rows])
    close(Lr, LSE[:, rows])


def test_rope_two_tokens_by_hand(oracle_mod):
    """S = 2, d = 2 (one frequency, w_0 = 1), Q = K = V = X = identity rows.
    Position 0 is not rotated; position 1 turns (0, 1) by one radian to
    (-sin 1, cos 1).  Row 1: scores tau*(-sin 1) against key 0 and tau*1
    against itself."""
    X = np.eye(2)
    W = np.eye(2)
    O, LSE = oracle_mod.forward(X, W, W, W, 1, 1, 2, rope_theta=500000.0)
    tau = 1.0 / math.sqrt(2.0)
    s0, s1 = -tau * math.sin(1.0), tau
    l1 = math.log(math.exp(s0) + math.exp(s1))
    assert abs(LSE[0, 0] - tau) <= 1e-15
    assert abs(LSE[0, 1] - l1) <= 1e-15
    np.testing.assert_allclose(O[0], [1.0, 0.0], atol=1e-15)
    np.testing.assert_allclose(O[1], [math.exp(s0 - l1), math.exp(s1 - l1)], atol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
def test_rope_finite_differences(oracle_mod, causal):
    S, D, H, G, d = 21, 12, 4, 2, 6
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=9)
    theta = 7.0
    g = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, causal=causal, rope_theta=theta)
    params = dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv)
    rng = np.random.default_rng(4)

    def loss(p):
        O, _ = oracle_mod.forward(p["X"], p["Wq"], p["Wk"], p["Wv"], H, G, d, causal=causal,
                                  nthreads=1, rope_theta=theta)
        return float(np.sum(O * dO))

    for name, grad in (("X", "dX"), ("Wq", "dWq"), ("Wk", "dWk"), ("Wv", "dWv")):
        for _ in range(20):
            idx = tuple(int(rng.integers(0, n)) for n in params[name].shape)
            base = params[name][idx]
            eps = 1e-6 * max(1.0, abs(base))
            plus = {k: v.copy() for k, v in params.items()}
            minus = {k: v.copy() for k, v in params.items()}
            plus[name][idx] = base + eps
            minus[name][idx] = base - eps
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = g[grad][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


def test_rope_leaves_position_zero_and_values_alone(oracle_mod):
    """Position 0 turns by angle 0: with causal masking, row 0 of O and LSE is
    the same with or without the rotation.  With Wq = 0 every score is 0 and
    the rotation of a zero query changes nothing: O is the prefix mean of V."""
    S, D, H, G, d = 17, 12, 4, 2, 6
    X, Wq, Wk, Wv, _ = draw(S, D, H, G, d, seed=2)
    O0, L0 = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d)
    O1, L1 = oracle_mod.forward(X, Wq, Wk, Wv, H, G, d, rope_theta=10000.0)
    np.testing.assert_array_equal(O0[0], O1[0])
    np.testing.assert_array_equal(L0[:, 0], L1[:, 0])
    assert np.max(np.abs(O0[1:] - O1[1:])) > 1e-3  # it does act on later rows
    Wq0 = np.zeros_like(Wq)
    O2, L2 = oracle_mod.forward(X, Wq0, Wk, Wv, H, G, d, rope_theta=10000.0)
    r = H // G
    for h in range(H):
        g = h // r
        v = X @ Wv[g * d:(g + 1) * d].T
        pref = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
        close(O2[:, h * d:(h + 1) * d], pref, 1e-13)
        close(L2[h], np.log(np.arange(1, S + 1)), 1e-13)


def test_rope_rejects_odd_head_dim(oracle_mod):
    X, Wq, Wk, Wv, _ = draw(8, 6, 2, 1, 3)
    with pytest.raises(ValueError):
        oracle_mod.forward(X, Wq, Wk, Wv, 2, 1, 3, rope_theta=10000.0)
    with pytest.raises(ValueError):
        oracle_mod.forward(X, Wq, Wk, Wv, 2, 1, 3, rope_theta=-1.0)


# ------------------------------------------------------------ output projection
# Y = O Wo^T after the attention (the linear map that follows attention in the
# Llama and Qwen blocks; not on the pages' step list).  Loss L = sum(Y * dY).

def torch_layer_out(X, Wq, Wk, Wv, Wo, dY, H, G, d, causal, theta=0.0):
    """torch fp64 library layer with the output projection as a Linear map,
    autograd backward (rotary embedding as a complex product when theta > 0)."""
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k != "dY"))
         for k, v in dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, dY=dY).items()}
    S = X.shape[0]
    half = d // 2

    def rope(x):
        if theta <= 0:
            return x
        freq = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
        ang = torch.arange(S, dtype=torch.float64)[:, None] * freq[None, :]
        z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
        return torch.cat([z.real, z.imag], dim=-1)

    q = rope((t["X"] @ t["Wq"].T).reshape(S, H, d).transpose(0, 1))
    k = rope((t["X"] @ t["Wk"].T).reshape(S, G, d).transpose(0, 1)).repeat_interleave(H // G, 0)
    v = (t["X"] @ t["Wv"].T).reshape(S, G, d).transpose(0, 1).repeat_interleave(H // G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None],
                                                         is_causal=causal)[0]
    O = o.transpose(0, 1).reshape(S, H * d)
    Y = torch.nn.functional.linear(O, t["Wo"])
    (Y * t["dY"]).sum().backward()
    return dict(O=O.detach().numpy(), Y=Y.detach().numpy(), dX=t["X"].grad.numpy(),
                dWq=t["Wq"].grad.numpy(), dWk=t["Wk"].grad.numpy(), dWv=t["Wv"].grad.numpy(),
                dWo=t["Wo"].grad.numpy())


def draw_out(S, D, H, G, d, seed):
    X, Wq, Wk, Wv, _ = draw(S, D, H, G, d, seed=seed)
    rng = np.random.default_rng(seed + 100)
    Wo = rng.standard_normal((D, H * d)) / math.sqrt(H * d)
    dY = rng.standard_normal((S, D))
    return X, Wq, Wk, Wv, Wo, dY


@pytest.mark.parametrize("shape", SHAPES[:3])
@pytest.mark.parametrize("causal,theta", [(True, 0.0), (False, 0.0), (True, 10000.0)])
def test_out_proj_against_torch_library(oracle_mod, shape, causal, theta):
    S, D, H, G, d = shape
    X, Wq, Wk, Wv, Wo, dY = draw_out(S, D, H, G, d, seed=S + 1)
    got = oracle_mod.backward_out(X, Wq, Wk, Wv, Wo, dY, H, G, d, causal=causal, rope_theta=theta)
    ref = torch_layer_out(X, Wq, Wk, Wv, Wo, dY, H, G, d, causal, theta)
    for name in ("O", "Y", "dX", "dWq", "dWk", "dWv", "dWo"):
        close(got[name], ref[name])


def test_out_proj_finite_differences(oracle_mod):
    S, D, H, G, d = 17, 10, 2, 1, 6
    X, Wq, Wk, Wv, Wo, dY = draw_out(S, D, H, G, d, seed=21)
    g = oracle_mod.backward_out(X, Wq, Wk, Wv, Wo, dY, H, G, d)
    rng = np.random.default_rng(5)

    def loss(p):
        O, _ = oracle_mod.forward(p["X"], Wq, Wk, Wv, H, G, d, nthreads=1)
        Y, _, _ = oracle_mod.out_proj(O, p["Wo"], nthreads=1)
        return float(np.sum(Y * dY))

    params = dict(X=X, Wo=Wo)
    for name, grad in (("Wo", "dWo"), ("X", "dX")):
        for _ in range(20):
            idx = tuple(int(rng.integers(0, n)) for n in params[name].shape)
            base = params[name][idx]
            eps = 1e-6 * max(1.0, abs(base))
            plus = {k: v.copy() for k, v in params.items()}
            minus = {k: v.copy() for k, v in params.items()}
            plus[name][idx] = base + eps
            minus[name][idx] = base - eps
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = g[grad][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


def test_out_proj_identity_weight_and_scaling(oracle_mod):
    """Wo = I (d_model = H*d): Y = O, and the layer's gradients equal those of
    the plain layer with dO = dY; dWo = dY^T O.  For any Wo, <dWo, Wo> =
    <dY, Y> (Y is linear in Wo)."""
    S, D, H, G, d = 26, 16, 4, 2, 4
    X, Wq, Wk, Wv, _, dY = draw_out(S, D, H, G, d, seed=23)
    eye = np.eye(D)
    got = oracle_mod.backward_out(X, Wq, Wk, Wv, eye, dY, H, G, d)
    plain = oracle_mod.backward(X, Wq, Wk, Wv, dY, H, G, d)
    np.testing.assert_array_equal(got["Y"], got["O"])
    for name in ("O", "LSE", "dX", "dWq", "dWk", "dWv"):
        np.testing.assert_array_equal(got[name], plain[name])
    close(got["dWo"], dY.T @ got["O"], 1e-14)
    _, _, _, _, Wo, _ = draw_out(S, D, H, G, d, seed=24)
    r = oracle_mod.backward_out(X, Wq, Wk, Wv, Wo, dY, H, G, d)
    lhs, rhs = float(np.sum(r["dWo"] * Wo)), float(np.sum(dY * r["Y"]))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))


# ------------------------------------------------------------ dX at the last rows
@pytest.mark.parametrize("shape", [(37, 24, 4, 2, 8), (50, 24, 8, 1, 8), (29, 16, 3, 3, 8)])
@pytest.mark.parametrize("theta", [0.0, 10000.0])
def test_dx_tail_matches_full_backward(oracle_mod, shape, theta):
    """The tail routine (only query rows >= t0 attend) reproduces the full
    backward's dX rows t0 .. S-1, and torch's, for several t0 including 0."""
    S, D, H, G, d = shape
    X, Wq, Wk, Wv, dO = draw(S, D, H, G, d, seed=31)
    full = oracle_mod.backward(X, Wq, Wk, Wv, dO, H, G, d, rope_theta=theta)
    ref = (torch_layer_rope(X, Wq, Wk, Wv, dO, H, G, d, True, theta) if theta > 0
           else torch_layer(X, Wq, Wk, Wv, dO, H, G, d, True))
    for t0 in (0, 1, S // 2, S - 3, S - 1):
        tail = oracle_mod.dx_tail(X, Wq, Wk, Wv, dO, H, G, d, t0, rope_theta=theta)
        assert tail.shape == (S - t0, D)
        close(tail, full["dX"][t0:], 1e-12)
        close(tail, ref["dX"][t0:])


def test_dx_tail_rejects_bad_rows(oracle_mod):
    X, Wq, Wk, Wv, dO = draw(8, 8, 2, 1, 4, seed=1)
    for t0 in (-1, 8):
        with pytest.raises(ValueError):
            oracle_mod.dx_tail(X, Wq, Wk, Wv, dO, 2, 1, 4, t0)
