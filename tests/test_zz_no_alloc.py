"""upipe_fwd_noalloc: the forward in the library's static device array.

Through the C ABI, its O and LSE must equal upipe_fwd's (the same kernels on
the same inputs) bit for bit, on two calls in a row where the second has a
smaller input than the first (the array keeps the first call's contents),
with no device memory allocated by the calls; plans whose forward workspace
exceeds the array are rejected before anything is enqueued.
"""
import pytest
import torch

from headwise_chunked_context_stage_amd import upipe
from headwise_chunked_context_stage_amd.layer import alloc_outputs, forward
from headwise_chunked_context_stage_amd.synth import LayerShape, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    upipe.lib()


def say(*a):
    print(*a, flush=True)


def reference(shape, U, dtype, inp):
    plan = upipe.Plan(shape.S, shape.D, shape.H, shape.G, shape.d, U, dtype=dtype)
    out = alloc_outputs(plan, inp["X"].device, backward=False)
    forward(plan, inp, out)
    torch.cuda.synchronize()
    return out["O"], out["LSE"]


def noalloc(shape, U, dtype, inp):
    plan = upipe.Plan(shape.S, shape.D, shape.H, shape.G, shape.d, U, dtype=dtype)
    assert plan.peak_bytes_phase(0) <= upipe.upipe_noalloc_max_bytes()
    O = torch.full((shape.S, shape.H * shape.d), float("nan"), dtype=inp["X"].dtype, device="cuda")
    LSE = torch.full((shape.H, shape.S), float("nan"), device="cuda")
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    free0 = torch.cuda.mem_get_info()[0]
    plan.fwd_noalloc(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], O, LSE)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base  # nothing from torch's allocator
    return O, LSE, free0 - torch.cuda.mem_get_info()[0]


CASES = [
    # (S, D, H, G), U, dtype: the second call of each pair is smaller
    ((4096, 1024, 8, 2), 4, "bf16"),
    ((1000, 512, 4, 1), 2, "bf16"),
    ((640, 256, 4, 2), 2, "f32"),
    ((320, 256, 4, 2), 4, "f32"),
]


def test_noalloc_forward_equals_workspace_forward_twice_in_a_row():
    drift = []
    for (S, D, H, G), U, dtype in CASES:
        shape = LayerShape(S=S, D=D, H=H, G=G, d=128 if dtype == "bf16" else 64)
        inp = {k: v.cuda() for k, v in
               make_inputs(shape, dtype, seed=29, device="cpu", with_grad_out=False).items()}
        say("noalloc %s S=%d D=%d H=%d G=%d U=%d" % (dtype, S, D, H, G, U))
        O_ref, L_ref = reference(shape, U, dtype, inp)
        O, L, used = noalloc(shape, U, dtype, inp)
        drift.append(used)
        assert torch.equal(O, O_ref) and torch.equal(L, L_ref)
    # after the first call has set up the device's array, calls take no device memory
    say("free-memory change per call (bytes): %s" % drift)
    assert all(u == 0 for u in drift[1:]), drift


def test_noalloc_rejects_oversized_and_pipelined_plans():
    cap = upipe.upipe_noalloc_max_bytes()
    assert cap == 256 << 20
    # forward workspace 2*S*d*(U + 2): S = 2^20 with U = 1 needs 768 MiB
    big = upipe.Plan(1 << 20, 128, 1, 1, 128, 1, dtype="bf16")
    assert big.peak_bytes_phase(0) > cap
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_fwd_noalloc(big.handle, 0, 0, 0, 0, 0, 0)
    assert e.value.code == upipe.UPIPE_ERR_WORKSPACE
    pipe = upipe.Plan(256, 256, 4, 2, 128, 2, dtype="bf16", pipeline=True)
    with pytest.raises(upipe.UpipeError) as e:
        upipe.upipe_fwd_noalloc(pipe.handle, 0, 0, 0, 0, 0, 0)
    assert e.value.code == upipe.UPIPE_ERR_ARG
