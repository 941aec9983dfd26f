"""Write the expected values of the full-d_model sub-layer test (fp64 oracle).

One KV group of the Llama3-8B attention shape at full d_model: S = 32768
tokens, d_model 4096, 4 query heads sharing 1 KV head, d_head 128, causal,
bf16 inputs.  Each stage of the pages' method projects its heads from X and
attends over the full sequence (paper.rainbus.top summary of "Untied
Ulysses", section 方法步骤详情); the oracle computes the unchunked layer.

With the argument `qwen3`, the same for one KV group of the Qwen3-32B
attention shape: d_model 5120, 8 query heads sharing 1 KV head (written to
sublayer_s32k_qwen3.npz).

Inputs come from the seeded CPU generator of the package's input module
(seed 0, drawn in the order X, Wq, Wk, Wv, dO), so the GPU test can draw the
same bits again.  The oracle's full forward and backward run once (minutes
on a few host cores); sampled rows of every output are stored, with the
shape, the seed and a hash of the inputs, in the .npz file.  Values are
stored as float32 (relative rounding 6e-8, far below the comparison gates).

This script calls only the oracle and the input generator:
    python tests/golden/make_sublayer_s32k.py [qwen3]
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

SEED = 0
# name -> (output file, shape, sampled dWq rows); rows are first/last rows of
# heads and blocks and a few inside
VARIANTS = {
    "llama3": ("sublayer_s32k.npz", dict(S=32768, D=4096, H=4, G=1, d=128),
               [0, 1, 126, 127, 133, 320, 484, 511]),
    "qwen3": ("sublayer_s32k_qwen3.npz", dict(S=32768, D=5120, H=8, G=1, d=128),
              [0, 1, 127, 133, 320, 575, 896, 1023]),
}
DWK_ROWS = [0, 37, 64, 127]
DWV_ROWS = [0, 50, 99, 127]
TOKEN_ROWS = [0, 1, 4095, 4096, 16383, 16391, 32766, 32767]


def input_hash(inp) -> str:
    """sha256 over the stored bits of X, Wq, Wk, Wv, dO (in that order)."""
    from headwise_chunked_context_stage_amd.synth import to_numpy_exact

    h = hashlib.sha256()
    for k in ("X", "Wq", "Wk", "Wv", "dO"):
        h.update(np.ascontiguousarray(to_numpy_exact(inp[k])).tobytes())
    return h.hexdigest()


def main(variant="llama3"):
    import torch

    import oracle
    from headwise_chunked_context_stage_amd.synth import LayerShape, make_inputs, to_numpy_exact

    fname, shape_args, DWQ_ROWS = VARIANTS[variant]
    OUT = os.path.join(HERE, fname)
    shape = LayerShape(**shape_args)
    inp = make_inputs(shape, "bf16", seed=SEED, device="cpu")
    digest = input_hash(inp)
    oracle.build(force=False)
    t0 = time.time()
    ref = oracle.backward(*[to_numpy_exact(inp[k]) for k in ("X", "Wq", "Wk", "Wv", "dO")],
                          shape.H, shape.G, shape.d)
    dt = time.time() - t0
    rows = np.array(TOKEN_ROWS, np.int64)
    np.savez_compressed(
        OUT,
        shape=np.array([shape.S, shape.D, shape.H, shape.G, shape.d], np.int64),
        seed=np.array(SEED, np.int64),
        input_sha256=np.array(digest),
        torch_version=np.array(torch.__version__),
        oracle_seconds=np.array(dt),
        dwq_rows=np.array(DWQ_ROWS, np.int64), dWq=ref["dWq"][DWQ_ROWS].astype(np.float32),
        dwk_rows=np.array(DWK_ROWS, np.int64), dWk=ref["dWk"][DWK_ROWS].astype(np.float32),
        dwv_rows=np.array(DWV_ROWS, np.int64), dWv=ref["dWv"][DWV_ROWS].astype(np.float32),
        token_rows=rows, dX=ref["dX"][rows].astype(np.float32),
        O=ref["O"][rows].astype(np.float32), LSE=ref["LSE"][:, rows].astype(np.float32),
        # whole-tensor norms, for a scale-aware report in the test
        norms=np.array([np.linalg.norm(ref[k]) for k in ("dWq", "dWk", "dWv", "dX")]),
    )
    print("wrote %s (oracle %.0f s, inputs %s)" % (OUT, dt, digest[:16]))


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "llama3")
