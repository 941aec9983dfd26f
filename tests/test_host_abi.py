"""Host-side tests of the C ABI (no GPU needed): the library loads and exports
every declared symbol, plans are validated, the head schedule and the stage
buffer sizes follow the pages, and bad arguments are rejected before any
launch.

Stage schedule: paper.rainbus.top summary of "Untied Ulysses", section
方法步骤详情 (H/U stages of U consecutive heads, buffers reused by every stage)
and section 技术新颖性 (each distinct KV head moved once).
"""
import json
import os
import re

import pytest

from headwise_chunked_context_stage_amd import upipe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "upipe.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "memory_closed_forms.json")


def legal_us(H, G):
    r = H // G
    return [U for U in range(1, H + 1) if H % U == 0 and (r % U == 0 or U % r == 0)]


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    declared = set(re.findall(r"\b(upipe_[a-z_]+)\s*\(", text))
    assert declared >= set(upipe.EXPORTS)
    L = upipe.lib()
    for name in sorted(declared):
        assert hasattr(L, name), name


def test_mfma_ceiling_rejects_bad_arguments_before_any_device_call():
    import ctypes
    L = upipe.lib()
    out = ctypes.c_double(0.0)
    for w, it in ((0, 1024), (3, 1024), (1, 7), (-1, 1024)):
        assert L.upipe_mfma_ceiling(w, it, ctypes.byref(out), None) == upipe.UPIPE_ERR_ARG
    assert L.upipe_mfma_ceiling(2, 1024, None, None) == upipe.UPIPE_ERR_ARG


def test_strerror():
    assert upipe.upipe_strerror(0) == "ok"
    for c in (1, 2, 3, 4):
        assert upipe.upipe_strerror(c) not in ("ok", "unknown error")
    assert upipe.upipe_strerror(99) == "unknown error"


@pytest.mark.parametrize("args,code", [
    ((128, 256, 4, 3, 64, 1, 1, "f32"), upipe.UPIPE_ERR_ARG),   # G does not divide H
    ((128, 256, 32, 8, 128, 3, 1, "bf16"), upipe.UPIPE_ERR_ARG),  # U does not divide H
    ((128, 256, 24, 4, 128, 4, 1, "bf16"), upipe.UPIPE_ERR_ARG),  # U=4 vs group size 6
    ((128, 256, 24, 4, 128, 12, 1, "bf16"), upipe.UPIPE_OK),      # two whole groups
    ((-1, 256, 4, 2, 64, 1, 1, "f32"), upipe.UPIPE_ERR_ARG),
    ((128, 0, 4, 2, 64, 1, 1, "f32"), upipe.UPIPE_ERR_ARG),
    ((128, 256, 4, 2, 64, 1, 2, "f32"), upipe.UPIPE_ERR_ARG),     # causal flag
    ((128, 256, 4, 2, 64, 1, 1, 7), upipe.UPIPE_ERR_ARG),         # dtype
    ((128, 256, 4, 2, 96, 1, 1, "f32"), upipe.UPIPE_ERR_UNSUPPORTED),
    ((128, 256, 4, 2, 64, 1, 1, "bf16"), upipe.UPIPE_ERR_UNSUPPORTED),   # bf16 needs d=128
    ((128, 192, 4, 2, 128, 1, 1, "bf16"), upipe.UPIPE_ERR_UNSUPPORTED),  # D % 128
    ((128, 96, 4, 2, 64, 1, 1, "f32"), upipe.UPIPE_ERR_UNSUPPORTED),     # D % 64
    ((0, 256, 4, 2, 64, 2, 1, "f32"), upipe.UPIPE_OK),                   # empty sequence
])
def test_create_validation(args, code):
    if code == upipe.UPIPE_OK:
        p = upipe.upipe_create(*args)
        upipe.upipe_destroy(p)
    else:
        with pytest.raises(upipe.UpipeError) as e:
            upipe.upipe_create(*args)
        assert e.value.code == code


@pytest.mark.parametrize("theta,code", [
    (0.0, upipe.UPIPE_OK), (10000.0, upipe.UPIPE_OK), (500000.0, upipe.UPIPE_OK),
    (0.5, upipe.UPIPE_OK), (-1.0, upipe.UPIPE_ERR_ARG), (float("nan"), upipe.UPIPE_ERR_ARG),
    (float("inf"), upipe.UPIPE_ERR_ARG), (-0.0, upipe.UPIPE_OK),
])
def test_create_rope_validation(theta, code):
    """The rotary embedding's base must be 0 (off) or finite and positive."""
    if code == upipe.UPIPE_OK:
        p = upipe.upipe_create_rope(256, 256, 4, 2, 128, 2, 1, "bf16", 0, theta)
        upipe.upipe_destroy(p)
    else:
        with pytest.raises(upipe.UpipeError) as e:
            upipe.upipe_create_rope(256, 256, 4, 2, 128, 2, 1, "bf16", 0, theta)
        assert e.value.code == code


def test_rope_leaves_schedule_and_workspace_unchanged():
    for flags in (0, upipe.UPIPE_PIPELINE):
        a = upipe.upipe_create_ex(4096, 1024, 32, 8, 128, 4, 1, "bf16", flags)
        b = upipe.upipe_create_rope(4096, 1024, 32, 8, 128, 4, 1, "bf16", flags, 500000.0)
        try:
            for ph in (0, 1):
                assert upipe.upipe_peak_bytes_phase(a, ph) == upipe.upipe_peak_bytes_phase(b, ph)
            assert upipe.upipe_num_stages(a) == upipe.upipe_num_stages(b)
            for s in range(upipe.upipe_num_stages(a)):
                assert upipe.upipe_stage_info(a, s) == upipe.upipe_stage_info(b, s)
        finally:
            upipe.upipe_destroy(a)
            upipe.upipe_destroy(b)
    with pytest.raises(upipe.UpipeError):  # shape checks still apply
        upipe.upipe_create_rope(128, 256, 4, 2, 64, 1, 1, "bf16", 0, 10000.0)
    with pytest.raises(upipe.UpipeError):  # and flag checks
        upipe.upipe_create_rope(128, 256, 4, 2, 128, 1, 1, "bf16", 8, 10000.0)


@pytest.mark.parametrize("H,G", [(32, 8), (64, 8), (4, 2), (4, 1), (8, 8), (24, 4)])
def test_schedule_covers_heads_and_loads_kv_once(H, G):
    r = H // G
    for U in legal_us(H, G):
        p = upipe.Plan(1024, 1024, H, G, 128, U)
        assert p.num_stages == H // U
        seen_q, loads, dones = [], [], []
        for s in range(p.num_stages):
            st = p.stage_info(s)
            assert st["q_first"] == s * U and st["q_count"] == U
            qs = range(st["q_first"], st["q_first"] + U)
            kvs = list(range(st["kv_first"], st["kv_first"] + st["kv_count"]))
            assert sorted({h // r for h in qs}) == kvs  # exactly the KV heads it reads
            seen_q += list(qs)
            if st["kv_load"]:
                loads += kvs
                # a group is opened by the stage holding its first query head
                assert all(g * r in qs for g in kvs)
            if st["kv_done"]:
                dones += kvs
                assert all((g + 1) * r - 1 in qs for g in kvs)
        assert seen_q == list(range(H))
        assert loads == list(range(G)) and dones == list(range(G))


def test_peak_bytes_closed_forms():
    """Forward stage bytes = 2*S*d*(U + 2*kv_s) <= 6*S*U*d (the pages' per-stage
    projection bytes, which count K and V at U heads); equal for MHA; linear in
    U; independent of H."""
    g = json.load(open(GOLDEN))
    coeff, b = g["projection_coeff"], g["bytes_per_element"]
    S, d = 4096, 128
    for H, G in [(32, 8), (64, 8), (8, 8)]:
        r = H // G
        for U in legal_us(H, G):
            p = upipe.Plan(S, 1024, H, G, d, U)
            kv_s = max(1, U // r)
            fwd = p.peak_bytes_phase(0)
            assert fwd == b * S * d * (U + 2 * kv_s)
            assert fwd <= coeff * S * U * d
            if G == H:
                assert fwd == coeff * S * U * d
            assert p.peak_bytes == max(p.peak_bytes_phase(0), p.peak_bytes_phase(1))
    # independent of H for the same U and group size
    a = upipe.Plan(S, 1024, 32, 8, d, 4).peak_bytes
    c = upipe.Plan(S, 1024, 64, 16, d, 4).peak_bytes
    assert a == c
    # linear in U for group-aligned U
    p4, p8, p16 = (upipe.Plan(S, 1024, 64, 8, d, U).peak_bytes for U in (8, 16, 32))
    assert p16 - p8 == 2 * (p8 - p4)


def test_qwen3_32b_reduction_matches_pages():
    """Qwen3-32B attention (H=64, G=8): one head per device per stage (U = C = 8)
    vs all heads (U = H = 64) is 12 vs 96 (x S/C x d_head) = an 87.5% cut."""
    g = json.load(open(GOLDEN))["qwen3_32b"]
    S, D, d = 65536, 5120, 128
    u_small = upipe.Plan(S, D, g["H"], 8, d, g["C"])
    u_all = upipe.Plan(S, D, g["H"], 8, d, g["H"])
    ratio = u_small.peak_bytes_phase(0) / u_all.peak_bytes_phase(0)
    assert ratio == g["upipe_coeff"] / g["ulysses_coeff"]
    assert 100.0 * (1.0 - ratio) == g["reduction_percent"]
    # the backward's stage buffers scale the same way; the weight-gradient
    # scratch (partial sums of 7 token parts, 128 x D fp32 each) is the same
    # for every U
    # (U = 8: 10 chunks per stage, U = 64: 64 per call; both take 2 per launch)
    scratch = dw_scratch_closed_form(S, D, 10)
    assert scratch == dw_scratch_closed_form(S, D, 64) == 14 * 128 * D * 4
    ratio_b = (u_small.peak_bytes_phase(1) - scratch) / (u_all.peak_bytes_phase(1) - scratch)
    assert ratio_b == pytest.approx(1 / 8, rel=1e-3)


FAKE = 1 << 20  # a 256-aligned non-null address; never dereferenced (validation fails first)


@pytest.mark.parametrize("pipeline", [False, True])
def test_fwd_bwd_reject_before_launch(pipeline):
    p = upipe.Plan(512, 256, 4, 2, 64, 2, dtype="f32", pipeline=pipeline)
    need = p.peak_bytes
    ok = [FAKE] * 6
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_fwd(p.handle, 0, *ok[1:], FAKE, need, 0)
    assert e.value.code == upipe.UPIPE_ERR_ARG
    with pytest.raises(upipe.UpipeError) as e:  # misaligned tensor
        upipe.upipe_fwd(p.handle, FAKE + 2, *ok[1:], FAKE, need, 0)
    assert e.value.code == upipe.UPIPE_ERR_ARG
    with pytest.raises(upipe.UpipeError) as e:  # workspace too small
        upipe.upipe_fwd(p.handle, *ok, FAKE, p.peak_bytes_phase(0) - 1, 0)
    assert e.value.code == upipe.UPIPE_ERR_WORKSPACE
    with pytest.raises(upipe.UpipeError) as e:  # workspace misaligned
        upipe.upipe_fwd(p.handle, *ok, FAKE + 16, need, 0)
    assert e.value.code == upipe.UPIPE_ERR_WORKSPACE
    bw = [FAKE] * 12
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_bwd(p.handle, *bw[:7], 0, *bw[8:11], FAKE, need, 0)
    assert e.value.code == upipe.UPIPE_ERR_ARG
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_bwd(p.handle, *bw[:11], FAKE, p.peak_bytes_phase(1) - 1, 0)
    assert e.value.code == upipe.UPIPE_ERR_WORKSPACE
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_fwd(0, *ok, FAKE, need, 0)
    assert e.value.code == upipe.UPIPE_ERR_ARG


def test_empty_sequence_forward_is_a_no_op():
    p = upipe.Plan(0, 256, 4, 2, 64, 2, dtype="f32")
    assert p.peak_bytes == 0
    upipe.upipe_fwd(p.handle, 0, 0, 0, 0, 0, 0, 0, 0, 0)  # nothing to do, nothing enqueued


def test_stage_info_bad_index():
    p = upipe.Plan(128, 256, 4, 2, 64, 2, dtype="f32")
    with pytest.raises(upipe.UpipeError):
        p.stage_info(2)
    with pytest.raises(upipe.UpipeError):
        p.stage_info(-1)


def test_auto_u_is_the_largest_legal_u_that_fits():
    """upipe_auto_u: for every budget between consecutive plan sizes, the
    chosen U is legal, its workspace fits, and no larger legal U fits."""
    S, D, d = 4096, 1024, 128
    for H, G in [(32, 8), (64, 8), (8, 8), (4, 1)]:
        us = legal_us(H, G)
        peak = {U: upipe.Plan(S, D, H, G, d, U).peak_bytes for U in us}
        for budget in sorted(set(peak.values())) + [max(peak.values()) * 2]:
            for b in (budget - 1, budget):
                fits = [U for U in us if peak[U] <= b]
                if not fits:
                    with pytest.raises(upipe.UpipeError) as e:
                        upipe.upipe_auto_u(S, D, H, G, d, b)
                    assert e.value.code == upipe.UPIPE_ERR_WORKSPACE
                    continue
                U = upipe.upipe_auto_u(S, D, H, G, d, b)
                assert U == max(fits) and peak[U] <= b


def test_auto_u_longer_sequence_gets_smaller_u():
    """The pages' dynamic-chunking reading: with a fixed memory budget, U
    shrinks (never grows) as the sequence gets longer, down to no fit."""
    H, G, D, d = 32, 8, 4096, 128
    budget = upipe.Plan(262144, D, H, G, d, 16).peak_bytes
    got = {}
    for S in (16384, 65536, 131072, 262144, 524288, 1048576):
        got[S] = upipe.upipe_auto_u(S, D, H, G, d, budget)
        assert got[S] in legal_us(H, G)
    seq = [got[S] for S in sorted(got)]
    assert seq == sorted(seq, reverse=True)
    assert got[16384] == H and got[262144] == 16 and got[524288] == 8 and got[1048576] == 4
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_auto_u(4194304, D, H, G, d, budget)
    assert e.value.code == upipe.UPIPE_ERR_WORKSPACE


def test_auto_u_rejects_bad_shapes_and_null_output():
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_auto_u(4096, 1024, 30, 8, 128, 1 << 40)  # G does not divide H
    assert e.value.code == upipe.UPIPE_ERR_ARG
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_auto_u(4096, 1024, 32, 8, 64, 1 << 40)  # bf16 needs d_head = 128
    assert e.value.code == upipe.UPIPE_ERR_UNSUPPORTED
    L = upipe.lib()
    assert L.upipe_auto_u(4096, 1024, 32, 8, 128, 1, 0, 1 << 40, None) == upipe.UPIPE_ERR_ARG


def kv_sum_bytes(S, d, U, r):
    """bf16 dK/dV sums in fp32: below 512 key tiles of 128 (S <= 65408) each
    key tile's query range is split into two halves with sums of their own,
    [half][dK, dV][S][d] for one KV head at a time (they also carry the sums
    across a group's stages); from 512 key tiles on, one fp32 carry of dK and
    dV [S][d] when a group spans stages (U < r)."""
    if (S + 127) // 128 < 512:
        return 4 * 4 * S * d
    return 2 * 4 * S * d if U < r else 0


def dw_scratch_closed_form(S, D, nmax):
    """bf16 weight-gradient scratch: the token range is cut into P parts
    (P = 1 below 8192 tokens, S // 4096 up to 8 parts, 8 from 32768 tokens on);
    parts 1..P-1 of up to min(nmax, max(1, 16 // (P - 1))) chunks at a time are
    kept as 128 x D fp32 tiles (nmax: the most chunks of one call)."""
    P = 1 if S < 8192 else (8 if S >= 32768 else S // 4096)
    if P == 1:
        return 0
    return (P - 1) * min(nmax, max(1, 16 // (P - 1))) * 128 * D * 4


def test_dw_scratch_is_fixed_by_s_and_d():
    """The weight-gradient scratch is a backward-only region: the token parts
    depend on S only (so every U sums dW over the same parts), the tiles on
    d_model and on the chunks one stage passes (its heads, plus K and V of the
    group it finishes): bwd bytes(U) - the stage buffers' closed form."""
    d, D, H, G = 128, 1024, 8, 2
    r = H // G
    for S in (4096, 8191, 8192, 12288, 16384, 20480, 32768, 65536):
        for U in legal_us(H, G):
            kv_s = max(1, U // r)
            qkv = 2 * S * d * (U + 2 * kv_s)
            single = 2 * 4 * S * U + kv_sum_bytes(S, d, U, r)
            p = upipe.Plan(S, D, H, G, d, U)
            extra = p.peak_bytes_phase(1) - (2 * qkv + single)
            want = dw_scratch_closed_form(S, D, U + 2 * kv_s)
            # regions are 256-byte aligned (S = 8191 rounds up)
            assert want <= extra < want + 16 * 256, (S, U, extra, want)
            assert p.peak_bytes_phase(0) == qkv
    # fp32 plans use their own weight-gradient kernel: no scratch
    p = upipe.Plan(32768, 256, 4, 2, 64, 2, dtype="f32")
    S, d, U, kv_s = 32768, 64, 2, 1
    qkv = 4 * S * d * (U + 2 * kv_s)
    assert p.peak_bytes_phase(1) == 2 * qkv + 2 * 4 * S * U


def test_pipelined_plan_doubles_the_per_stage_buffers():
    """Stage pipelining (the pages' overlap suggestion, paper.rainbus.top summary,
    sections 局限与改进 and 独立分析的弱点) keeps two copies of the Q/K/V stage
    buffers, of the dQ/dK/dV buffers and of D and LSE*log2(e) (consecutive
    stages may run at once); the fp32 dK/dV sum regions stay single (their sums
    run in stage order).  Closed forms in element counts, every region a
    multiple of 256 bytes at these sizes."""
    S, d = 4096, 128
    for H, G in [(32, 8), (8, 2), (8, 8)]:
        r = H // G
        for U in legal_us(H, G):
            kv_s = max(1, U // r)
            plain = upipe.Plan(S, 1024, H, G, d, U)
            pipe = upipe.Plan(S, 1024, H, G, d, U, pipeline=True)
            qkv = 2 * S * d * (U + 2 * kv_s)
            stats = 2 * 4 * S * U  # D, LSE*log2 e
            single = kv_sum_bytes(S, d, U, r)  # dK/dV sums
            assert plain.peak_bytes_phase(0) == qkv
            assert pipe.peak_bytes_phase(0) == 2 * qkv
            assert plain.peak_bytes_phase(1) == 2 * qkv + stats + single
            assert pipe.peak_bytes_phase(1) == 4 * qkv + 2 * stats + single
            assert pipe.num_stages == plain.num_stages
            for s in range(plain.num_stages):
                assert pipe.stage_info(s) == plain.stage_info(s)


def test_create_ex_flags():
    h = upipe.upipe_create_ex(4096, 1024, 8, 2, 128, 2, 1, "bf16", 0)
    try:
        assert upipe.upipe_peak_bytes(h) == upipe.Plan(4096, 1024, 8, 2, 128, 2).peak_bytes
    finally:
        upipe.upipe_destroy(h)
    for bad in (4, 8, -1, 1 << 30):
        with pytest.raises(upipe.UpipeError) as e:
            upipe.upipe_create_ex(4096, 1024, 8, 2, 128, 2, 1, "bf16", bad)
        assert e.value.code == upipe.UPIPE_ERR_ARG
    # shape errors are reported as for upipe_create
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_create_ex(4096, 1024, 8, 2, 128, 3, 1, "bf16", upipe.UPIPE_PIPELINE)
    assert e.value.code == upipe.UPIPE_ERR_ARG


def test_out_proj_plan_workspace_and_validation():
    """UPIPE_OUT_PROJ adds the stage dO buffer (U*S*d elements) to the
    backward workspace only; the output-projection entry points refuse a plan
    without the flag and bad pointers, before any launch."""
    import ctypes
    S, D, H, G, d = 4096, 1024, 32, 8, 128
    for U in legal_us(H, G):
        for dtype, e in (("bf16", 2),):
            a = upipe.upipe_create_ex(S, D, H, G, d, U, 1, dtype, 0)
            b = upipe.upipe_create_ex(S, D, H, G, d, U, 1, dtype, upipe.UPIPE_OUT_PROJ)
            try:
                assert upipe.upipe_peak_bytes_phase(b, 0) == upipe.upipe_peak_bytes_phase(a, 0)
                extra = upipe.upipe_peak_bytes_phase(b, 1) - upipe.upipe_peak_bytes_phase(a, 1)
                assert U * S * d * e <= extra < U * S * d * e + 256
            finally:
                upipe.upipe_destroy(a)
                upipe.upipe_destroy(b)
    L = upipe.lib()
    plain = upipe.Plan(256, 256, 4, 2, 128, 2)
    outp = upipe.Plan(256, 256, 4, 2, 128, 2, out_proj=True)
    fake = [ctypes.c_void_p(1 << 20) for _ in range(16)]  # aligned, never dereferenced
    ws = 1 << 20
    # a plan without the flag
    assert L.upipe_fwd_out(plain.handle, *fake[:8], ws, outp.peak_bytes, None) == upipe.UPIPE_ERR_ARG
    assert L.upipe_bwd_out(plain.handle, *fake[:13], ws, outp.peak_bytes, None) == upipe.UPIPE_ERR_ARG
    # null or misaligned pointers, small workspace
    assert L.upipe_fwd_out(outp.handle, *fake[:4], None, *fake[5:8], ws, outp.peak_bytes,
                           None) == upipe.UPIPE_ERR_ARG
    assert L.upipe_fwd_out(outp.handle, *fake[:7], ctypes.c_void_p((1 << 20) + 4), ws,
                           outp.peak_bytes, None) == upipe.UPIPE_ERR_ARG
    assert L.upipe_bwd_out(outp.handle, *fake[:12], None, ws, outp.peak_bytes,
                           None) == upipe.UPIPE_ERR_ARG
    assert L.upipe_bwd_out(outp.handle, *fake[:13], ws, outp.peak_bytes - 1,
                           None) == upipe.UPIPE_ERR_WORKSPACE
    assert L.upipe_bwd_out(outp.handle, *fake[:13], ws + 8, outp.peak_bytes,
                           None) == upipe.UPIPE_ERR_WORKSPACE


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU's share; --gpus N > 1 exits with a message
    before touching any device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_binding_rejects_bad_tensors_before_calling_the_library():
    """Plan.fwd / bwd / fwd_out / bwd_out check every tensor against the plan
    (shape, element type, contiguity, GPU device, alignment, workspace size)
    and raise before any pointer reaches the library; a host tensor would
    otherwise be handed to the kernels as a device address."""
    import torch

    S, D, H, G, d = 64, 128, 2, 1, 128
    plan = upipe.Plan(S, D, H, G, d, 1, dtype="bf16", out_proj=True)
    bf, f32 = torch.bfloat16, torch.float32
    t = {"X": torch.zeros(S, D, dtype=bf), "Wq": torch.zeros(H * d, D, dtype=bf),
         "Wk": torch.zeros(G * d, D, dtype=bf), "Wv": torch.zeros(G * d, D, dtype=bf),
         "O": torch.zeros(S, H * d, dtype=bf), "LSE": torch.zeros(H, S, dtype=f32),
         "ws": torch.zeros(plan.peak_bytes, dtype=torch.uint8)}
    with pytest.raises(ValueError, match="GPU tensor"):  # host memory is never passed on
        plan.fwd(t["X"], t["Wq"], t["Wk"], t["Wv"], t["O"], t["LSE"], t["ws"])
    with pytest.raises(ValueError, match="shape"):
        plan.fwd(t["X"][:, :64], t["Wq"], t["Wk"], t["Wv"], t["O"], t["LSE"], t["ws"])
    with pytest.raises(TypeError, match="dtype"):
        plan.fwd(t["X"].float(), t["Wq"], t["Wk"], t["Wv"], t["O"], t["LSE"], t["ws"])
    with pytest.raises(ValueError, match="contiguous"):
        plan.fwd(t["X"].t().contiguous().t(), t["Wq"], t["Wk"], t["Wv"], t["O"], t["LSE"],
                 t["ws"])
    with pytest.raises(ValueError, match="bytes"):
        plan.fwd(t["X"], t["Wq"], t["Wk"], t["Wv"], t["O"], t["LSE"], t["ws"][:16])
    with pytest.raises(TypeError, match="torch tensor"):
        plan.fwd(t["X"].data_ptr(), t["Wq"], t["Wk"], t["Wv"], t["O"], t["LSE"], t["ws"])
    with pytest.raises(TypeError, match="dtype"):  # LSE is fp32
        plan.fwd(t["X"], t["Wq"], t["Wk"], t["Wv"], t["O"], t["LSE"].to(bf), t["ws"])
    with pytest.raises(ValueError, match="shape"):  # dX is [S][D] fp32
        plan.bwd(t["O"], t["X"], t["Wq"], t["Wk"], t["Wv"], t["O"], t["LSE"],
                 torch.zeros(S, D + 128, dtype=f32), torch.zeros(H * d, D, dtype=f32),
                 torch.zeros(G * d, D, dtype=f32), torch.zeros(G * d, D, dtype=f32), t["ws"])
    with pytest.raises(ValueError, match="shape"):  # Wo is [D][H*d]
        plan.fwd_out(t["X"], t["Wq"], t["Wk"], t["Wv"], torch.zeros(H * d, D, dtype=bf), t["O"],
                     t["LSE"], torch.zeros(S, D, dtype=f32), t["ws"])
