"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
the same seeded inputs, bit-exactness across every legal U, determinism, and
the edge cases (ragged S, S = 1, the empty sequence, non-causal, GQA/MHA).

Tolerances (outputs vs the oracle, unit-variance inputs): max-abs <= 2e-2 and
mean-abs <= 2e-3 on every output in fp32, and on O and LSE in bf16.  In bf16
the gradients carry the error of storing Q, K, V and O in bf16 (which the
pages' per-stage byte count presupposes), of P and dS at the matrix-core
inputs and of dQ/dK/dV before the gradient GEMMs.  That floor, measured by
emulating exactly those rounding points (tests/bf16_floor.py), exceeds the
absolute bounds for dX at some shapes (short sequences, GQA) and several times
over for the weight gradients, whatever the implementation.  So bf16
gradients are gated on max and mean error within 1.25x of the emulated floor
(at most shapes tighter than the absolute bounds) and on relative Frobenius
error <= 1e-2; whether the absolute bounds are also met is printed.  The
floor check also catches any extra rounding step a kernel would add.

Headwise chunking partitions independent per-head work (paper.rainbus.top
summary of "Untied Ulysses", section 方法步骤详情), so every U must give the
same bits.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from headwise_chunked_context_stage_amd import upipe
from headwise_chunked_context_stage_amd.layer import alloc_outputs, backward, forward, run, run_out
from headwise_chunked_context_stage_amd.synth import CONFIGS, LayerShape, make_inputs, to_numpy_exact

from bf16_floor import bf16_path_emulation

pytestmark = pytest.mark.gpu

OUTS = ("O", "LSE", "dX", "dWq", "dWk", "dWv")


def legal_us(H, G):
    r = H // G
    return [U for U in range(1, H + 1) if H % U == 0 and (r % U == 0 or U % r == 0)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    upipe.lib()  # loud failure if the HIP library is missing
    oracle.build(force=False)


def say(*a):
    print(*a, flush=True)


def host(t):
    return t.detach().double().cpu().numpy()


def run_layer(shape, dtype, U, inp, causal=True, backward=True, pipeline=False, rope_theta=0.0):
    plan = upipe.Plan(shape.S, shape.D, shape.H, shape.G, shape.d, U, causal=causal, dtype=dtype,
                      pipeline=pipeline, rope_theta=rope_theta)
    out = run(plan, inp, backward_pass=backward)
    torch.cuda.synchronize()
    out.pop("ws")
    return out


def oracle_full(shape, inp, causal=True, rope_theta=0.0):
    np_in = [to_numpy_exact(inp[k]) for k in ("X", "Wq", "Wk", "Wv", "dO")]
    return oracle.backward(*np_in, shape.H, shape.G, shape.d, causal=causal, rope_theta=rope_theta)


def compare(name, got, ref, max_abs, mean_abs):
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    say("  %-4s max %.3e mean %.3e" % (name, mx, mn))
    assert mx <= max_abs and mn <= mean_abs, (name, mx, mn)


def rel_frob(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def check_against_oracle(out, ref, dtype, inp=None, shape=None, causal=True, rope_theta=0.0):
    if dtype == "f32":
        for k in OUTS:
            compare(k, host(out[k]), ref[k], 2e-2, 2e-3)
        return
    for k in ("O", "LSE"):
        compare(k, host(out[k]), ref[k], 2e-2, 2e-3)
    emu = bf16_path_emulation(inp, shape.H, shape.G, shape.d, causal=causal, rope_theta=rope_theta)
    for k in ("O", "LSE", "dX", "dWq", "dWk", "dWv"):
        got = host(out[k])
        floor = np.abs(emu[k].double().numpy() - ref[k])
        floor_fr = rel_frob(emu[k].double().numpy(), ref[k])
        err = np.abs(got - ref[k])
        fr = rel_frob(got, ref[k])
        say("  %-4s max %.3e mean %.3e relfrob %.3e | floor max %.3e mean %.3e"
            % (k, err.max(), err.mean(), fr, floor.max(), floor.mean()))
        assert err.max() <= 1.25 * floor.max() + 1e-3, (k, "max above the bf16 floor")
        assert err.mean() <= 1.25 * floor.mean() + 1e-5, (k, "mean above the bf16 floor")
        if k == "dX":
            # the literal mean bound, wherever the bf16 floor itself allows it;
            # at S = 1 the floor's own mean is 2.06e-3 (dV of a group is the
            # sum of its heads' dO, rounded to bf16), a recorded deviation
            if 1.25 * floor.mean() <= 2e-3:
                assert err.mean() <= 2e-3, (k, "mean above 2e-3", err.mean())
            else:
                say("       literal mean bound: the floor (%.3e) is above it at this shape"
                    % floor.mean())
        if k.startswith("dW"):
            # a recorded deviation: the bf16 floor of the weight gradients is
            # above the literal bounds for any implementation (bf16 storage of
            # Q, K, V, O alone puts their mean error near 1e-2)
            say("       literal bounds (2e-2 / 2e-3): %s" %
                ("met" if err.max() <= 2e-2 and err.mean() <= 2e-3 else
                 "not met -- known deviation, floor max %.3e mean %.3e" % (floor.max(), floor.mean())))
            if np.linalg.norm(ref[k]) == 0.0:  # e.g. dWq at S = 1: dQ of row 0 is exactly 0
                assert err.max() <= 1e-3, (k, err.max())
            else:
                # 1e-2 for Gaussian weights (their floor is 3-4e-3); inputs whose
                # own floor is higher (e.g. identity weights) get 1.25x that floor
                assert fr <= max(1e-2, 1.25 * floor_fr), (k, fr, floor_fr)


def assert_same_bits(a, b, what):
    for k in a:
        assert torch.equal(a[k], b[k]), "%s: %s differs" % (what, k)


# ---------------------------------------------------------------- fp32 (tiny)
def test_tiny_f32_all_U_match_oracle_and_each_other():
    cfg = CONFIGS["tiny_f32"]
    shape = cfg["shape"]
    inp = make_inputs(shape, "f32", seed=0, device="cpu")
    ref = oracle_full(shape, inp)
    inp = {k: v.cuda() for k, v in inp.items()}
    first = None
    for U in legal_us(shape.H, shape.G):
        say("tiny_f32 U=%d" % U)
        out = run_layer(shape, "f32", U, inp)
        check_against_oracle(out, ref, "f32")
        if first is None:
            first = out
        else:
            assert_same_bits(first, out, "U=%d" % U)
    again = run_layer(shape, "f32", 2, inp)
    assert_same_bits(first, again, "rerun")


# ---------------------------------------------------------------- bf16 parity
BF16_CASES = [
    # S, D, H, G  (d = 128)
    (512, 1024, 4, 1),
    (1000, 1024, 4, 1),   # ragged: not a multiple of any tile
    (2048, 1024, 4, 1),
    (768, 512, 8, 2),     # two groups of four
    (384, 256, 4, 4),     # MHA
    (4096, 4096, 4, 1),   # one KV group of the Llama3-8B shape at full d_model
]


@pytest.mark.parametrize("S,D,H,G", BF16_CASES)
def test_bf16_matches_oracle_and_is_U_invariant(S, D, H, G):
    shape = LayerShape(S=S, D=D, H=H, G=G, d=128)
    cpu_inp = make_inputs(shape, "bf16", seed=1, device="cpu")
    ref = oracle_full(shape, cpu_inp)
    inp = {k: v.cuda() for k, v in cpu_inp.items()}
    first = None
    for U in legal_us(H, G):
        say("bf16 S=%d D=%d H=%d G=%d U=%d" % (S, D, H, G, U))
        out = run_layer(shape, "bf16", U, inp)
        if first is None:
            check_against_oracle(out, ref, "bf16", cpu_inp, shape)
            first = out
        else:
            assert_same_bits(first, out, "U=%d" % U)
    again = run_layer(shape, "bf16", legal_us(H, G)[-1], inp)
    assert_same_bits(first, again, "rerun")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_core_on_given_qkv(dtype):
    """The attention kernels on given Q, K, V: with X = [A | B] and selector
    weights (Wq head 0 = [I 0], head 1 = [0 I], Wk = [I 0], Wv = [0 I]) the
    projections copy the blocks exactly (Q0 = K = A, Q1 = V = B), so O, LSE
    and the gradients test the forward, D, dK/dV and dQ kernels on those
    operands against the oracle."""
    d = 128 if dtype == "bf16" else 64
    S, H, G = 1000, 2, 1
    shape = LayerShape(S=S, D=2 * d, H=H, G=G, d=d)
    inp = make_inputs(shape, dtype, seed=23, device="cpu")
    eye, zero = torch.eye(d), torch.zeros(d, d)
    td = inp["X"].dtype
    inp["Wq"] = torch.cat([torch.cat([eye, zero], 1), torch.cat([zero, eye], 1)], 0).to(td)
    inp["Wk"] = torch.cat([eye, zero], 1).to(td)
    inp["Wv"] = torch.cat([zero, eye], 1).to(td)
    ref = oracle_full(shape, inp)
    dev = {k: v.cuda() for k, v in inp.items()}
    say("attention core on given Q, K, V (%s)" % dtype)
    out = run_layer(shape, dtype, 1, dev)
    check_against_oracle(out, ref, dtype, inp, shape)
    assert_same_bits(out, run_layer(shape, dtype, 2, dev), "U=2")


@pytest.mark.parametrize("S", [1, 33, 130])
def test_bf16_short_sequences(S):
    shape = LayerShape(S=S, D=256, H=4, G=2, d=128)
    cpu_inp = make_inputs(shape, "bf16", seed=2, device="cpu")
    ref = oracle_full(shape, cpu_inp)
    inp = {k: v.cuda() for k, v in cpu_inp.items()}
    say("bf16 short S=%d" % S)
    out = run_layer(shape, "bf16", 2, inp)
    check_against_oracle(out, ref, "bf16", cpu_inp, shape)
    if S == 1:  # one token: O is V[0] of the head's KV head (after bf16 storage)
        v0 = host(inp["X"][:1].float() @ inp["Wv"].float().T)
        for h in range(4):
            g = h // 2
            assert np.max(np.abs(host(out["O"])[0, h * 128:(h + 1) * 128] - v0[0, g * 128:(g + 1) * 128])) < 2e-2


def test_auto_u_runs_bit_identical_to_u1():
    """upipe_auto_u picks a legal U under a workspace budget; the layer run
    with that U and a workspace of exactly its size equals the U = 1 run bit
    for bit (chunking never changes results)."""
    shape = LayerShape(S=768, D=512, H=8, G=2, d=128)
    inp = {k: v.cuda() for k, v in make_inputs(shape, "bf16", seed=5, device="cpu").items()}
    budget = upipe.Plan(shape.S, shape.D, shape.H, shape.G, shape.d, 4).peak_bytes + 1000
    U = upipe.upipe_auto_u(shape.S, shape.D, shape.H, shape.G, shape.d, budget)
    say("auto U=%d for a budget of %d bytes" % (U, budget))
    assert U == 4
    plan = upipe.Plan(shape.S, shape.D, shape.H, shape.G, shape.d, U)
    assert plan.peak_bytes <= budget
    out = run(plan, inp)
    torch.cuda.synchronize()
    assert out["ws"].numel() == plan.peak_bytes
    out.pop("ws")
    assert_same_bits(run_layer(shape, "bf16", 1, inp), out, "auto U")


@pytest.mark.parametrize("S,D,H,G,d,dtype", [(768, 512, 8, 2, 128, "bf16"),
                                              (1000, 1024, 4, 1, 128, "bf16"),
                                              (320, 256, 4, 2, 64, "f32")])
def test_pipelined_plan_bit_identical(S, D, H, G, d, dtype):
    """Stage pipelining (pages' overlap suggestion; paper.rainbus.top summary,
    section 局限与改进) only moves GEMMs to a second stream with event ordering
    and alternates two copies of the stage buffers: for every legal U the
    pipelined layer equals the plain U = 1 layer bit for bit, on the default
    stream and on a side stream, and again on a later call (events reused)."""
    shape = LayerShape(S=S, D=D, H=H, G=G, d=d)
    inp = {k: v.cuda() for k, v in make_inputs(shape, dtype, seed=11, device="cpu").items()}
    ref = run_layer(shape, dtype, 1, inp)
    for U in legal_us(H, G):
        say("pipelined %s S=%d H=%d G=%d U=%d" % (dtype, S, H, G, U))
        assert_same_bits(ref, run_layer(shape, dtype, U, inp, pipeline=True), "pipelined U=%d" % U)
    say("pipelined U=1 on a side stream")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    plan = upipe.Plan(S, D, H, G, d, 1, dtype=dtype, pipeline=True)
    with torch.cuda.stream(side):
        out = run(plan, inp)
        out2 = run(plan, inp)
    torch.cuda.synchronize()
    out.pop("ws")
    out2.pop("ws")
    assert_same_bits(ref, out, "side stream")
    assert_same_bits(ref, out2, "side stream, second call")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_non_causal(dtype):
    shape = LayerShape(S=320, D=256, H=4, G=2, d=128 if dtype == "bf16" else 64)
    cpu_inp = make_inputs(shape, dtype, seed=3, device="cpu")
    ref = oracle_full(shape, cpu_inp, causal=False)
    inp = {k: v.cuda() for k, v in cpu_inp.items()}
    first = None
    for U in (1, 2, 4):
        say("non-causal %s U=%d" % (dtype, U))
        out = run_layer(shape, dtype, U, inp, causal=False)
        if first is None:
            check_against_oracle(out, ref, dtype, cpu_inp, shape, causal=False)
            first = out
        else:
            assert_same_bits(first, out, "U=%d" % U)


# ---------------------------------------------------------------- rotary embedding
# Optional rotate-half rotary embedding of queries and keys (the Llama and Qwen
# families' attention; not on the pages): the projection rotates Q and K before
# rounding, dQ and the finished dK take the transposed rotation.
ROPE_CASES = [
    # S, D, H, G, d, dtype, theta
    (1000, 1024, 4, 1, 128, "bf16", 10000.0),   # ragged
    (768, 512, 8, 2, 128, "bf16", 500000.0),    # two groups, Llama3's base
    (2048, 1024, 4, 2, 128, "bf16", 1000000.0),  # Qwen3's base; U = 1 carries dK over stages
    (320, 256, 4, 2, 64, "f32", 10000.0),
]


@pytest.mark.parametrize("S,D,H,G,d,dtype,theta", ROPE_CASES)
def test_rope_matches_oracle_and_is_U_invariant(S, D, H, G, d, dtype, theta):
    shape = LayerShape(S=S, D=D, H=H, G=G, d=d)
    cpu_inp = make_inputs(shape, dtype, seed=13, device="cpu")
    ref = oracle_full(shape, cpu_inp, rope_theta=theta)
    inp = {k: v.cuda() for k, v in cpu_inp.items()}
    first = None
    for U in legal_us(H, G):
        say("rope %s theta=%g S=%d D=%d H=%d G=%d U=%d" % (dtype, theta, S, D, H, G, U))
        out = run_layer(shape, dtype, U, inp, rope_theta=theta)
        if first is None:
            check_against_oracle(out, ref, dtype, cpu_inp, shape, rope_theta=theta)
            first = out
        else:
            assert_same_bits(first, out, "U=%d" % U)
    say("rope pipelined U=%d" % legal_us(H, G)[-1])
    assert_same_bits(first, run_layer(shape, dtype, legal_us(H, G)[-1], inp, pipeline=True,
                                      rope_theta=theta), "pipelined")
    plain = run_layer(shape, dtype, 1, inp)
    assert not torch.equal(plain["O"][1:], first["O"][1:])  # the embedding is applied


def test_rope_long_positions():
    """Rotary angles at token positions up to 2^20 (one turn fraction per
    position in fp64): forward rows near the end of a 1M-token sequence
    against the oracle.  A narrow d_model keeps the oracle's key projection
    over all positions short; the scaling identities cover the backward."""
    shape = LayerShape(S=1 << 20, D=128, H=2, G=1, d=128)
    inp = make_inputs(shape, "bf16", seed=17, device="cuda")
    say("rope S=1048576 D=128 H=2 G=1 U=2 theta=10000")
    out = run_layer(shape, "bf16", 2, inp, rope_theta=10000.0)
    S = shape.S
    sampled_rows_check(shape, inp, out, [0, 1, 4095],
                       [S - 1, S - 2, S - 1000, (1 << 19) + 3], (0, 2), rope_theta=10000.0)
    dx_tail_check(shape, inp, out, 8, rope_theta=10000.0)
    e = identities(out, inp)
    say("  identities %.2e %.2e %.2e" % e)
    assert max(e) < 1e-4
    for k in OUTS:
        assert torch.isfinite(out[k]).all(), k


# Weight gradients over token parts: from 8192 tokens on, the bf16 dW sums
# run over dw_parts(S) = min(8, S // 4096) parts of the token range, one
# workgroup each, folded in part order (a split fixed by S, so every U sums
# alike).  These cases cross 2, 3 and 4 parts, one with a ragged last k-step.
PART_CASES = [
    # S, D, H, G (d = 128)
    (8192, 256, 2, 1),    # 2 parts
    (12000, 256, 2, 1),   # 2 parts, ragged
    (12288, 384, 4, 2),   # 3 parts, two groups
    (16384, 256, 2, 1),   # 4 parts
]


@pytest.mark.parametrize("S,D,H,G", PART_CASES)
def test_bf16_weight_gradient_token_parts(S, D, H, G):
    shape = LayerShape(S=S, D=D, H=H, G=G, d=128)
    cpu_inp = make_inputs(shape, "bf16", seed=23, device="cpu")
    ref = oracle_full(shape, cpu_inp)
    inp = {k: v.cuda() for k, v in cpu_inp.items()}
    first = None
    for U in legal_us(H, G):
        say("bf16 token parts S=%d D=%d H=%d G=%d U=%d" % (S, D, H, G, U))
        out = run_layer(shape, "bf16", U, inp)
        if first is None:
            check_against_oracle(out, ref, "bf16", cpu_inp, shape)
            first = out
        else:
            assert_same_bits(first, out, "U=%d" % U)
    say("bf16 token parts pipelined U=1")
    assert_same_bits(first, run_layer(shape, "bf16", 1, inp, pipeline=True), "pipelined")


# ---------------------------------------------------------------- output projection
# Y = O Wo^T after the attention (the Llama / Qwen attention block's output map;
# not on the pages' step list): forward into Y (fp32, summed stage by stage),
# backward from dY with each stage's dO = dY Wo formed in the workspace.
OUT_KEYS = ("O", "LSE", "Y", "dX", "dWq", "dWk", "dWv", "dWo")
OUT_CASES = [
    # S, D, H, G, d, dtype, theta
    (1000, 1024, 4, 1, 128, "bf16", 0.0),       # ragged
    (768, 512, 8, 2, 128, "bf16", 500000.0),    # two groups, with the rotary embedding
    (512, 1536, 8, 8, 128, "bf16", 0.0),        # MHA, d_model (1536) wider than H*d (1024)
    (8192, 256, 2, 1, 128, "bf16", 0.0),        # dWo over 2 token parts (transposed fold)
    (320, 256, 4, 2, 64, "f32", 10000.0),
]


def run_layer_out(shape, dtype, U, inp, pipeline=False, rope_theta=0.0):
    plan = upipe.Plan(shape.S, shape.D, shape.H, shape.G, shape.d, U, dtype=dtype,
                      pipeline=pipeline, rope_theta=rope_theta, out_proj=True)
    out = run_out(plan, inp)
    torch.cuda.synchronize()
    out.pop("ws")
    return out


@pytest.mark.parametrize("S,D,H,G,d,dtype,theta", OUT_CASES)
def test_out_proj_matches_oracle_and_is_U_invariant(S, D, H, G, d, dtype, theta):
    shape = LayerShape(S=S, D=D, H=H, G=G, d=d)
    cpu_inp = make_inputs(shape, dtype, seed=19, device="cpu", out_proj=True)
    ref = oracle.backward_out(*[to_numpy_exact(cpu_inp[k]) for k in
                                ("X", "Wq", "Wk", "Wv", "Wo", "dY")],
                              H, G, d, rope_theta=theta)
    inp = {k: v.cuda() for k, v in cpu_inp.items()}
    first = None
    for U in legal_us(H, G):
        say("out-proj %s theta=%g S=%d D=%d H=%d G=%d U=%d" % (dtype, theta, S, D, H, G, U))
        out = run_layer_out(shape, dtype, U, inp, rope_theta=theta)
        if first is None:
            first = out
            if dtype == "f32":
                for k in OUT_KEYS:
                    compare(k, host(out[k]), ref[k], 2e-2, 2e-3)
            else:
                emu = bf16_path_emulation(cpu_inp, H, G, d, rope_theta=theta, out_proj=True)
                for k in OUT_KEYS:
                    got = host(out[k])
                    err = np.abs(got - ref[k])
                    floor = np.abs(emu[k].double().numpy() - ref[k])
                    fr = rel_frob(got, ref[k])
                    say("  %-4s max %.3e mean %.3e relfrob %.3e | floor max %.3e mean %.3e"
                        % (k, err.max(), err.mean(), fr, floor.max(), floor.mean()))
                    assert err.max() <= 1.25 * floor.max() + 1e-3, (k, "max above the bf16 floor")
                    assert err.mean() <= 1.25 * floor.mean() + 1e-5, (k, "mean above the floor")
                    assert fr <= 1e-2, (k, fr)
                for k in ("O", "LSE", "Y"):
                    compare(k, host(out[k]), ref[k], 2e-2, 2e-3)
        else:
            assert_same_bits(first, out, "U=%d" % U)
    say("out-proj pipelined U=%d" % legal_us(H, G)[-1])
    assert_same_bits(first, run_layer_out(shape, dtype, legal_us(H, G)[-1], inp, pipeline=True,
                                          rope_theta=theta), "pipelined")
    # the plain entry points on the same plan still give the plain layer
    plan = upipe.Plan(S, D, H, G, d, 1, dtype=dtype, rope_theta=theta, out_proj=True)
    plain = run(plan, inp, backward_pass=False)
    torch.cuda.synchronize()
    assert torch.equal(plain["O"], first["O"]) and torch.equal(plain["LSE"], first["LSE"])


# ---------------------------------------------------------------- QK-norm
# Per-head RMSNorm of the projected queries and keys before the rotary
# embedding (the Qwen3 attention; not on the pages), through upipe_fwd_ex /
# upipe_bwd_ex: every output, dgamma_q and dgamma_k included, against the
# oracle; bit-identical across U and with the pipelined plan.
QKN_KEYS = ("O", "LSE", "dX", "dWq", "dWk", "dWv", "dq_norm", "dk_norm")
QKN_CASES = [
    # S, D, H, G, d, dtype, theta, out_proj
    (1000, 1024, 4, 1, 128, "bf16", 0.0, False),      # ragged, one group (U = 1 carries dK)
    (768, 512, 8, 2, 128, "bf16", 1000000.0, False),  # two groups, Qwen3's rotary base
    (512, 1536, 8, 8, 128, "bf16", 1000000.0, True),  # MHA with the output projection
    (320, 256, 4, 2, 64, "f32", 10000.0, False),
    (256, 256, 4, 2, 64, "f32", 0.0, True),
]


def run_layer_ex(shape, dtype, U, inp, pipeline=False, rope_theta=0.0, out_proj=False):
    from headwise_chunked_context_stage_amd.layer import run_ex

    plan = upipe.Plan(shape.S, shape.D, shape.H, shape.G, shape.d, U, dtype=dtype,
                      pipeline=pipeline, rope_theta=rope_theta, out_proj=out_proj, qk_norm=True,
                      qk_norm_eps=1e-6)
    out = run_ex(plan, inp)
    torch.cuda.synchronize()
    out.pop("ws")
    return out


@pytest.mark.parametrize("S,D,H,G,d,dtype,theta,oproj", QKN_CASES)
def test_qk_norm_matches_oracle_and_is_U_invariant(S, D, H, G, d, dtype, theta, oproj):
    shape = LayerShape(S=S, D=D, H=H, G=G, d=d)
    cpu_inp = make_inputs(shape, dtype, seed=31, device="cpu", qk_norm=True, out_proj=oproj)
    ex = {k: to_numpy_exact(cpu_inp[k]) for k in cpu_inp}
    nk = dict(q_norm=ex["q_norm"], k_norm=ex["k_norm"], qk_eps=1e-6, rope_theta=theta)
    if oproj:
        ref = oracle.backward_out(ex["X"], ex["Wq"], ex["Wk"], ex["Wv"], ex["Wo"], ex["dY"],
                                  H, G, d, **nk)
    else:
        ref = oracle.backward(ex["X"], ex["Wq"], ex["Wk"], ex["Wv"], ex["dO"], H, G, d, **nk)
    keys = QKN_KEYS + (("Y", "dWo") if oproj else ())
    inp = {k: v.cuda() for k, v in cpu_inp.items()}
    emu = None
    if dtype == "bf16":
        emu = bf16_path_emulation(cpu_inp, H, G, d, rope_theta=theta, out_proj=oproj,
                                  qk_norm_eps=1e-6)
    first = None
    for U in legal_us(H, G):
        say("qk-norm %s theta=%g out_proj=%d S=%d D=%d H=%d G=%d U=%d"
            % (dtype, theta, oproj, S, D, H, G, U))
        out = run_layer_ex(shape, dtype, U, inp, rope_theta=theta, out_proj=oproj)
        if first is not None:
            assert_same_bits(first, out, "U=%d" % U)
            continue
        first = out
        for k in keys:
            got = host(out[k])
            if dtype == "f32":
                compare(k, got, ref[k], 2e-2, 2e-3)
                continue
            err = np.abs(got - ref[k])
            floor = np.abs(emu[k].double().numpy() - ref[k])
            fr = rel_frob(got, ref[k])
            say("  %-7s max %.3e mean %.3e relfrob %.3e | floor max %.3e mean %.3e"
                % (k, err.max(), err.mean(), fr, floor.max(), floor.mean()))
            assert err.max() <= 1.25 * floor.max() + 1e-3, (k, "max above the bf16 floor")
            assert err.mean() <= 1.25 * floor.mean() + 1e-5, (k, "mean above the floor")
            if k in ("O", "LSE", "Y"):
                compare(k, got, ref[k], 2e-2, 2e-3)
            elif k == "dX":
                assert err.mean() <= 2e-3, (k, err.mean())
            else:
                assert fr <= max(1e-2, 1.25 * rel_frob(emu[k].double().numpy(), ref[k])), (k, fr)
    say("qk-norm pipelined U=%d" % legal_us(H, G)[-1])
    assert_same_bits(first, run_layer_ex(shape, dtype, legal_us(H, G)[-1], inp, pipeline=True,
                                         rope_theta=theta, out_proj=oproj), "pipelined")


@pytest.mark.timeout(900)
def test_full_size_qwen32b_s64k_qk_norm_rope_U_invariant():
    """The Qwen3-32B attention block's own options at its shape (S = 65536,
    d_model 5120, 64 query heads, 8 KV heads): QK-norm and the rotary
    embedding with base 1e6, bit-identical for U in {1, 8, 64}; forward rows
    of two groups' heads against the oracle (early rows and the last ones);
    the Q/K scale invariance <dgamma_q, gamma_q> = <dgamma_k, gamma_k> (exact
    for the exact layer) and finite outputs."""
    cfg = CONFIGS["qwen32b_s64k"]
    shape = cfg["shape"]
    S, r = shape.S, shape.H // shape.G
    inp = make_inputs(shape, "bf16", seed=0, device="cuda", qk_norm=True)
    first = None
    for U in cfg["U"]:
        say("qwen32b S=65536 QK-norm + rope 1e6, U=%d" % U)
        out = run_layer_ex(shape, "bf16", U, inp, rope_theta=1e6)
        if first is not None:
            assert_same_bits(first, out, "U=%d" % U)
            del out
            torch.cuda.empty_cache()
            continue
        first = out
        n = S
        np_in = [to_numpy_exact(inp["X"][:n])] + [to_numpy_exact(inp[k]) for k in ("Wq", "Wk", "Wv")]
        nk = dict(rope_theta=1e6, q_norm=to_numpy_exact(inp["q_norm"]),
                  k_norm=to_numpy_exact(inp["k_norm"]), qk_eps=1e-6)
        rows = [0, 1, 1023, 4095, S - 1000, S - 2, S - 1]
        for heads in ((0, r), (7 * r, 8 * r)):
            say("  oracle rows %s heads %s" % (rows[:4], heads))
            Or, Lr = oracle.forward_rows(*np_in, shape.H, shape.G, shape.d, rows, heads=heads, **nk)
            c0, c1 = heads[0] * shape.d, heads[1] * shape.d
            compare("O", host(out["O"][rows])[:, c0:c1], Or[:, c0:c1], 2e-2, 2e-3)
            compare("LSE", host(out["LSE"][heads[0]:heads[1]][:, rows]), Lr[heads[0]:heads[1]], 2e-2, 2e-3)
        gq, gk = inp["q_norm"].double(), inp["k_norm"].double()
        dq, dk = out["dq_norm"].double(), out["dk_norm"].double()
        a, b = float((dq * gq).sum()), float((dk * gk).sum())
        scale = float(dq.norm() * gq.norm() + dk.norm() * gk.norm())
        say("  <dgq,gq> %.6e  <dgk,gk> %.6e  relative %.2e" % (a, b, abs(a - b) / scale))
        assert abs(a - b) <= 1e-2 * scale, (a, b, scale)
        for k in QKN_KEYS:
            assert torch.isfinite(out[k]).all(), k
    del first
    torch.cuda.empty_cache()


def test_qk_norm_entry_points_reject_mismatched_arguments():
    """A QK-norm plan refuses the entry points without gamma, and
    upipe_fwd_ex / upipe_bwd_ex refuse a missing gamma or a tensor the plan
    does not use, before anything is enqueued."""
    shape = LayerShape(S=128, D=256, H=2, G=1, d=128)
    inp = {k: v.cuda() for k, v in make_inputs(shape, "bf16", seed=2, device="cpu",
                                                qk_norm=True).items()}
    plan = upipe.Plan(128, 256, 2, 1, 128, 1, qk_norm=True)
    out = alloc_outputs(plan, inp["X"].device)
    with pytest.raises(upipe.UpipeError):
        upipe.upipe_fwd(plan.handle, inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], out["O"],
                        out["LSE"], out["ws"])
    io = dict(X=inp["X"], Wq=inp["Wq"], Wk=inp["Wk"], Wv=inp["Wv"], O=out["O"], LSE=out["LSE"])
    with pytest.raises(upipe.UpipeError):  # gamma missing
        upipe.upipe_fwd_ex(plan.handle, io, out["ws"])
    plain = upipe.Plan(128, 256, 2, 1, 128, 1)
    with pytest.raises(upipe.UpipeError):  # gamma given to a plan without QK-norm
        upipe.upipe_fwd_ex(plain.handle, dict(io, q_norm=inp["q_norm"], k_norm=inp["k_norm"]),
                           out["ws"])
    upipe.upipe_fwd_ex(plain.handle, io, out["ws"])  # the plain plan through the same entry
    torch.cuda.synchronize()
    ref = run_layer(shape, "bf16", 1, inp, backward=False)
    assert torch.equal(out["O"], ref["O"]) and torch.equal(out["LSE"], ref["LSE"])


def test_empty_sequence_zero_weight_gradients():
    shape = LayerShape(S=0, D=256, H=4, G=2, d=128)
    plan = upipe.Plan(0, 256, 4, 2, 128, 2)
    dW = [torch.full((n * 128, 256), 7.0, device="cuda") for n in (4, 2, 2)]
    say("empty sequence")
    upipe.upipe_bwd(plan.handle, 0, 0, 0, 0, 0, 0, 0, 0, dW[0], dW[1], dW[2], 0, 0)
    torch.cuda.synchronize()
    for t in dW:
        assert torch.count_nonzero(t).item() == 0
    say("empty sequence, output projection")
    plan = upipe.Plan(0, 256, 4, 2, 128, 2, out_proj=True)
    dW = [torch.full((n * 128, 256), 7.0, device="cuda") for n in (4, 2, 2)]
    dWo = torch.full((256, 4 * 128), 7.0, device="cuda")
    upipe.upipe_fwd_out(plan.handle, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    upipe.upipe_bwd_out(plan.handle, 0, 0, 0, 0, 0, 0, 0, 0, 0, dW[0], dW[1], dW[2], dWo, 0, 0)
    torch.cuda.synchronize()
    for t in dW + [dWo]:
        assert torch.count_nonzero(t).item() == 0
    del shape


def test_causal_invariance_bitwise():
    """Changing tokens after t leaves O and LSE of rows <= t bit-identical
    (masked probabilities are exactly zero)."""
    shape = LayerShape(S=1024, D=512, H=4, G=1, d=128)
    inp = make_inputs(shape, "bf16", seed=4, device="cuda", with_grad_out=False)
    say("causal invariance")
    a = run_layer(shape, "bf16", 4, inp, backward=False)
    t = 517
    inp2 = dict(inp)
    inp2["X"] = inp["X"].clone()
    inp2["X"][t + 1:] = torch.randn_like(inp2["X"][t + 1:].float()).to(torch.bfloat16)
    b = run_layer(shape, "bf16", 4, inp2, backward=False)
    assert torch.equal(a["O"][:t + 1], b["O"][:t + 1])
    assert torch.equal(a["LSE"][:, :t + 1], b["LSE"][:, :t + 1])
    assert not torch.equal(a["O"][t + 1:], b["O"][t + 1:])


# ---------------------------------------------------------------- full size
def chunked_ip(a, b, rows=1 << 16):
    """<a, b> accumulated in fp64 over row blocks (bounded temporaries at S = 1M)."""
    tot = 0.0
    for i in range(0, a.shape[0], rows):
        tot += float((a[i:i + rows].double() * b[i:i + rows].double()).sum())
    return tot


def identities(out, inp):
    """Scaling identities that hold for the exact layer at any size:
    <dWv,Wv> = <dO,O>, <dWq,Wq> = <dWk,Wk>, <dX,X> = sum <dW,W>.
    Returns the three relative discrepancies (normalised by norm products)."""
    ip = chunked_ip
    nn = lambda a, b: math.sqrt(ip(a, a) * ip(b, b))
    e1 = abs(ip(out["dWv"], inp["Wv"]) - ip(inp["dO"], out["O"])) / nn(inp["dO"], out["O"])
    e2 = abs(ip(out["dWq"], inp["Wq"]) - ip(out["dWk"], inp["Wk"])) / (
        nn(out["dWq"], inp["Wq"]) + nn(out["dWk"], inp["Wk"]))
    tot = ip(out["dWq"], inp["Wq"]) + ip(out["dWk"], inp["Wk"]) + ip(out["dWv"], inp["Wv"])
    e3 = abs(ip(out["dX"], inp["X"]) - tot) / (nn(out["dX"], inp["X"]))
    return e1, e2, e3


def sampled_rows_check(shape, inp, out, rows_all, rows_late, late_heads, rope_theta=0.0):
    """Forward rows against the oracle.  With causal masking row i depends only
    on X rows 0..i, so the oracle gets X[:max_row + 1] (a shorter sequence)."""
    n = max(rows_all + rows_late) + 1
    np_in = [to_numpy_exact(inp["X"][:n])] + [to_numpy_exact(inp[k]) for k in ("Wq", "Wk", "Wv")]
    O = out["O"]
    LSE = out["LSE"]
    for rows, heads in ((rows_all, (0, shape.H)), (rows_late, late_heads)):
        if not rows:
            continue
        say("  oracle rows %s heads %s" % (rows[:4], heads))
        Or, Lr = oracle.forward_rows(*np_in, shape.H, shape.G, shape.d, rows, heads=heads,
                                     rope_theta=rope_theta)
        c0, c1 = heads[0] * shape.d, heads[1] * shape.d
        got_o = host(O[rows])[:, c0:c1]
        got_l = host(LSE[heads[0]:heads[1]][:, rows])
        compare("O", got_o, Or[:, c0:c1], 2e-2, 2e-3)
        assert np.isfinite(Or[:, c0:c1]).all()
        compare("LSE", got_l, Lr[heads[0]:heads[1]], 2e-2, 2e-3)


def dx_tail_check(shape, inp, out, n_rows, rope_theta=0.0):
    """Backward rows against the oracle at full size: dX of the last n_rows
    tokens is cheap to compute exactly (only the last query rows see the last
    keys).  Gated on mean-abs <= 2e-3 and relative Frobenius error <= 1e-2,
    with a gross max-abs bound; the bf16 floor emulation is out of reach at
    these sizes."""
    S = shape.S
    t0 = S - n_rows
    say("  oracle dX rows %d .. %d" % (t0, S - 1))
    ref = oracle.dx_tail(*[to_numpy_exact(inp[k]) for k in ("X", "Wq", "Wk", "Wv", "dO")],
                         shape.H, shape.G, shape.d, t0, rope_theta=rope_theta)
    got = host(out["dX"][t0:])
    err = np.abs(got - ref)
    fr = rel_frob(got, ref)
    say("  dX   max %.3e mean %.3e relfrob %.3e" % (err.max(), err.mean(), fr))
    assert err.mean() <= 2e-3 and fr <= 1e-2 and err.max() <= 5e-2, (err.max(), err.mean(), fr)


def run_measured(shape, U, inp):
    """fwd + bwd with the device high-water mark taken around the calls: the
    library allocates nothing, so the only intermediate memory is the
    caller's workspace of peak_bytes()."""
    plan = upipe.Plan(shape.S, shape.D, shape.H, shape.G, shape.d, U, causal=True, dtype="bf16")
    out = alloc_outputs(plan, inp["X"].device)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    forward(plan, inp, out)
    backward(plan, inp, out)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base, "device memory allocated during the calls"
    assert out["ws"].numel() == plan.peak_bytes
    out.pop("ws")
    return out, (plan.peak_bytes_phase(0), plan.peak_bytes_phase(1))


def test_full_size_llama8b_s32k_U_invariant():
    cfg = CONFIGS["llama8b_s32k"]
    shape = cfg["shape"]
    inp = make_inputs(shape, "bf16", seed=0, device="cuda")
    first = None
    for U in cfg["U"]:
        say("llama8b S=32768 U=%d" % U)
        out = run_layer(shape, "bf16", U, inp)
        if first is None:
            first = out
            sampled_rows_check(shape, inp, out, [0, 1, 2, 63, 64, 127, 128, 129, 1000, 2047],
                               [], None)
            dx_tail_check(shape, inp, out, 16)
            e = identities(out, inp)
            say("  identities %.2e %.2e %.2e" % e)
            assert max(e) < 1e-4
        else:
            assert_same_bits(first, out, "U=%d" % U)
            del out
        torch.cuda.empty_cache()


def test_full_size_llama8b_s128k_bench_config():
    cfg = CONFIGS["llama8b_s128k"]
    shape = cfg["shape"]
    inp = make_inputs(shape, "bf16", seed=0, device="cuda")
    say("llama8b S=131072 U=4")
    out = run_layer(shape, "bf16", 4, inp)
    say("llama8b S=131072 U=4 pipelined")
    assert_same_bits(out, run_layer(shape, "bf16", 4, inp, pipeline=True), "pipelined")
    torch.cuda.empty_cache()
    S = shape.S
    sampled_rows_check(shape, inp, out, [0, 1, 100, 1023, 1024, 2047],
                       [S - 1, S - 2, S - 129, S - 4096], (0, 4))
    dx_tail_check(shape, inp, out, 8)
    e = identities(out, inp)
    say("  identities %.2e %.2e %.2e" % e)
    assert max(e) < 1e-4
    for k in OUTS:
        assert torch.isfinite(out[k]).all(), k


def test_full_size_qwen32b_s64k_U_invariant_and_peak_bytes():
    """Qwen3-32B attention shape: bit-exact across U in {1, 8, 64}, forward rows
    against the oracle, the scaling identities, and the stage workspace: the
    QKV region is 2*S*d*(U + 2*kv_s) bytes, so U = 8 needs 1/8 of U = 64 (the
    pages' 12 vs 96 S*d_head per device, 87.5% less; paper.rainbus.top summary
    of "Untied Ulysses", sections 核心方法 and 复现评估)."""
    cfg = CONFIGS["qwen32b_s64k"]
    shape = cfg["shape"]
    S, d, r = shape.S, shape.d, shape.H // shape.G
    inp = make_inputs(shape, "bf16", seed=0, device="cuda")
    first, ws = None, {}
    for U in cfg["U"]:
        say("qwen32b S=65536 U=%d" % U)
        out, ws[U] = run_measured(shape, U, inp)
        say("  workspace fwd %d bwd %d bytes" % ws[U])
        assert ws[U][0] == 2 * S * d * (U + 2 * max(1, U // r))
        if first is None:
            first = out
            sampled_rows_check(shape, inp, out, [0, 1, 100, 1023, 1024, 4095],
                               [S - 1, S - 2, S - 1000], (0, r))
            dx_tail_check(shape, inp, out, 8)
            e = identities(out, inp)
            say("  identities %.2e %.2e %.2e" % e)
            assert max(e) < 1e-4
            for k in OUTS:
                assert torch.isfinite(out[k]).all(), k
        else:
            assert_same_bits(first, out, "U=%d" % U)
            del out
        torch.cuda.empty_cache()
    assert 8 * ws[8][0] == ws[64][0]


@pytest.mark.timeout(900)
def test_full_size_llama8b_share_s1m():
    """One GPU's share of Llama3-8B at S = 1M tokens (4 query heads + 1 KV
    head, U = 1): forward rows of all heads against the oracle, early and
    past 2^19 tokens (where element offsets of X [S][4096] and O pass 2^31),
    up to the last row; dX of the last 8 tokens (offsets near 2^32) against
    the oracle's exact tail; the scaling identities, finite outputs and the
    measured workspace."""
    cfg = CONFIGS["llama8b_share_s1m"]
    shape = cfg["shape"]
    S = shape.S
    inp = make_inputs(shape, "bf16", seed=0, device="cuda")
    say("llama8b share S=1048576 U=1")
    out, ws = run_measured(shape, 1, inp)
    say("  workspace fwd %d bwd %d bytes" % ws)
    assert ws[0] == 2 * shape.S * shape.d * 3
    sampled_rows_check(shape, inp, out,
                       [0, 1, 1023, 4095, 32767, 65535, (1 << 19) + 3, 3 << 18, S - 4096,
                        S - 2, S - 1], [], None)
    dx_tail_check(shape, inp, out, 8)
    e = identities(out, inp)
    say("  identities %.2e %.2e %.2e" % e)
    assert max(e) < 1e-4
    for k in OUTS:
        assert torch.isfinite(out[k]).all(), k


# ---------------------------------------------------------------- full d_model sub-layer
@pytest.mark.parametrize("fixture", ["sublayer_s32k.npz", "sublayer_s32k_qwen3.npz"])
def test_full_dmodel_sublayer_s32k_every_output_against_oracle(fixture):
    """One KV group at full d_model and S = 32768 -- of the Llama3-8B shape (4
    query heads, 1 KV head, D = 4096) and of the Qwen3-32B shape (8 query
    heads, D = 5120): every output against the fp64 oracle's full backward,
    stored by tests/golden/make_sublayer_s32k.py -- sampled rows of dWq, dWk,
    dWv element by element (each a sum over all 32768 tokens through the split
    contraction of the weight-gradient kernel), dX, O and LSE at rows across
    the sequence -- for every legal U, bit-identical across U."""
    import os
    import sys

    golden = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, golden)
    from make_sublayer_s32k import input_hash

    fx = np.load(os.path.join(golden, fixture))
    S, D, H, G, d = (int(v) for v in fx["shape"])
    shape = LayerShape(S=S, D=D, H=H, G=G, d=d)
    cpu_inp = make_inputs(shape, "bf16", seed=int(fx["seed"]), device="cpu")
    assert input_hash(cpu_inp) == str(fx["input_sha256"]), "inputs differ from the fixture's"
    inp = {k: v.cuda() for k, v in cpu_inp.items()}
    del cpu_inp
    rows = fx["token_rows"]
    first = None
    for U in legal_us(H, G):
        say("sub-layer S=%d D=%d H=%d G=%d U=%d" % (S, D, H, G, U))
        out = run_layer(shape, "bf16", U, inp)
        if first is not None:
            assert_same_bits(first, out, "U=%d" % U)
            continue
        first = out
        compare("O", host(out["O"][rows]), fx["O"].astype(np.float64), 2e-2, 2e-3)
        compare("LSE", host(out["LSE"][:, rows]), fx["LSE"].astype(np.float64), 2e-2, 2e-3)
        got = host(out["dX"][rows])
        ref = fx["dX"].astype(np.float64)
        err = np.abs(got - ref)
        say("  dX   max %.3e mean %.3e relfrob %.3e" % (err.max(), err.mean(), rel_frob(got, ref)))
        assert err.mean() <= 2e-3 and rel_frob(got, ref) <= 1e-2 and err.max() <= 5e-2
        for k, rk in (("dWq", "dwq_rows"), ("dWk", "dwk_rows"), ("dWv", "dwv_rows")):
            got = host(out[k][fx[rk]])
            ref = fx[k].astype(np.float64)
            err = np.abs(got - ref)
            fr = rel_frob(got, ref)
            say("  %-4s max %.3e mean %.3e relfrob %.3e (literal bounds: known deviation)"
                % (k, err.max(), err.mean(), fr))
            assert fr <= 1e-2, (k, fr)
            for i in range(ref.shape[0]):  # row by row, and no single element far off
                rms = float(np.sqrt(np.mean(ref[i] ** 2)))
                assert rel_frob(got[i], ref[i]) <= 1.5e-2, (k, i, rel_frob(got[i], ref[i]))
                assert err[i].max() <= 0.1 * rms, (k, i, err[i].max(), rms)
    del first
    torch.cuda.empty_cache()
