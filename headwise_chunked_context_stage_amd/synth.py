"""Seeded synthetic inputs for the attention layer.

This module only draws random numbers; it holds none of the layer's
arithmetic.  Both the GPU path (tests, benchmark) and the fp64 oracle read the
same tensors produced here, so the two sides see exactly the same bits.

Recipe (the pages train Llama3-8B and Qwen3-32B on public datasets that are not
available here; Gaussian tensors of the same attention shapes stand in):
  * one generator per call, seeded with `seed`, drawing in the fixed order
    X, Wq, Wk, Wv, dO;
  * X ~ N(0, 1) [S][D]; Wq ~ N(0, 1/D) [H*d][D]; Wk, Wv ~ N(0, 1/D) [G*d][D];
    dO ~ N(0, 1) [S][H*d];
  * values are drawn in fp32 and, for bf16 runs, rounded to bf16 with
    round-to-nearest-even; the rounded tensors *are* the inputs.
  * device="cpu" uses torch's CPU generator (small shapes, bit-reproducible on
    any host); device="cuda" draws on the GPU (large shapes).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class LayerShape:
    S: int
    D: int
    H: int
    G: int
    d: int

    @property
    def Hd(self) -> int:
        return self.H * self.d


# The configurations used by the tests and the benchmark.  Shapes follow the
# attention layers of the models the pages train (Llama3-8B: d_model 4096,
# 32 query heads, 8 KV heads; Qwen3-32B: d_model 5120, 64 query heads, 8 KV
# heads; head dim 128).
CONFIGS = {
    "tiny_f32": dict(shape=LayerShape(S=512, D=256, H=4, G=2, d=64), dtype="f32",
                     U=(1, 2, 4)),
    "llama8b_s32k": dict(shape=LayerShape(S=32768, D=4096, H=32, G=8, d=128), dtype="bf16",
                         U=(1, 4, 8, 32)),
    "qwen32b_s64k": dict(shape=LayerShape(S=65536, D=5120, H=64, G=8, d=128), dtype="bf16",
                         U=(1, 8, 64)),
    "llama8b_s128k": dict(shape=LayerShape(S=131072, D=4096, H=32, G=8, d=128), dtype="bf16",
                          U=(4,)),
    "llama8b_share_s1m": dict(shape=LayerShape(S=1048576, D=4096, H=4, G=1, d=128),
                              dtype="bf16", U=(1,)),
}


def torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError("dtype must be 'bf16' or 'f32'")


def make_inputs(shape: LayerShape, dtype: str = "bf16", seed: int = 0, device: str = "cpu",
                with_grad_out: bool = True, wq_zero: bool = False, out_proj: bool = False,
                qk_norm: bool = False):
    """Draw X, Wq, Wk, Wv (and dO) for `shape`.

    Returns a dict of tensors on `device` in the storage dtype.  `wq_zero`
    replaces Wq by zeros after drawing (the draw order is unchanged).
    `out_proj` also draws, after the others, the output projection
    Wo [D][H*d] ~ N(0, 1/(H*d)) and the output gradient dY [S][D] ~ N(0, 1).
    `qk_norm` then draws the QK-norm weights q_norm, k_norm [d] ~ 1 + N(0, 0.2^2)
    (trained RMSNorm weights scatter around 1).
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    td = torch_dtype(dtype)
    S, D, H, G, d = shape.S, shape.D, shape.H, shape.G, shape.d
    wstd = 1.0 / (D ** 0.5)

    def draw(rows, cols, std):
        t = torch.randn((rows, cols), generator=gen, device=dev, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(td)

    out = {
        "X": draw(S, D, 1.0),
        "Wq": draw(H * d, D, wstd),
        "Wk": draw(G * d, D, wstd),
        "Wv": draw(G * d, D, wstd),
    }
    if with_grad_out:
        out["dO"] = draw(S, H * d, 1.0)
    if out_proj:
        out["Wo"] = draw(D, H * d, 1.0 / ((H * d) ** 0.5))
        out["dY"] = draw(S, D, 1.0)
    if qk_norm:
        for k in ("q_norm", "k_norm"):
            t = torch.randn((d,), generator=gen, device=dev, dtype=torch.float32)
            out[k] = (1.0 + 0.2 * t).to(td)
    if wq_zero:
        out["Wq"].zero_()
    return out


def to_numpy_exact(t: torch.Tensor):
    """Host copy carrying exactly the stored bits: bf16 -> uint16 patterns,
    fp32 -> float32, fp64 -> float64."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
