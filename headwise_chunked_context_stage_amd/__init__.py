"""Headwise-chunked causal GQA attention (one GPU's share), forward and
backward, for AMD Instinct MI355X (gfx950).

The compute path is the HIP library behind ``include/upipe.h``; ``upipe``
is its thin ctypes binding and ``layer`` allocates the caller-owned tensors
with torch (device memory and streams only).  ``synth`` draws the seeded
synthetic inputs.
"""
from . import upipe  # noqa: F401
