"""fp64 CPU oracle for headwise-chunked causal GQA attention (fwd + bwd).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the GPU library and never touches a GPU.

The arithmetic lives in ``upipe_oracle.cpp`` (plain fp64 loops, unchunked; see
its header for the passages of the pages on "Untied Ulysses: Memory-Efficient
Context Parallelism via Headwise Chunking" it follows).  This module only
builds that file with g++ and marshals numpy arrays to it.

Input arrays may be float64, float32, or uint16 holding bf16 bit patterns;
every element is decoded exactly into fp64 before any arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "upipe_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
               "-ffp-contract=off", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
        f64 = ctypes.c_double
        lib.oracle_forward.argtypes = [i64, i64, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp, dp,
                                       dp, i32]
        lib.oracle_forward.restype = i32
        lib.oracle_forward_rows.argtypes = [i64, i64, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp,
                                            vp, i64, i32, i32, dp, dp, i32]
        lib.oracle_forward_rows.restype = i32
        lib.oracle_backward.argtypes = [i64, i64, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp, vp,
                                        dp, dp, dp, dp, dp, dp, i32]
        lib.oracle_backward.restype = i32
        lib.oracle_dx_tail.argtypes = [i64, i64, i32, i32, i32, f64, i32, vp, vp, vp, vp, vp, i64,
                                       dp, i32]
        lib.oracle_dx_tail.restype = i32
        lib.oracle_out_proj.argtypes = [i64, i64, i64, i32, dp, vp, vp, dp, dp, dp, i32]
        lib.oracle_out_proj.restype = i32
        lib.oracle_forward_qkn.argtypes = [i64, i64, i32, i32, i32, i32, f64, f64, i32, vp, vp, vp,
                                           vp, vp, vp, dp, dp, i32]
        lib.oracle_forward_qkn.restype = i32
        lib.oracle_backward_qkn.argtypes = [i64, i64, i32, i32, i32, i32, f64, f64, i32, vp, vp, vp,
                                            vp, vp, vp, vp, dp, dp, dp, dp, dp, dp, dp, dp, i32]
        lib.oracle_backward_qkn.restype = i32
        lib.oracle_forward_rows_qkn.argtypes = [i64, i64, i32, i32, i32, i32, f64, f64, i32, vp, vp,
                                                vp, vp, vp, vp, vp, i64, i32, i32, dp, dp, i32]
        lib.oracle_forward_rows_qkn.restype = i32
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _enc(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 0
    if a.dtype == np.float32:
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError("oracle inputs must be uint16 (bf16 bits), float32 or float64, got %s" % a.dtype)


def _prep(arrs):
    arrs = [np.ascontiguousarray(a) for a in arrs]
    enc = {_enc(a) for a in arrs}
    if len(enc) != 1:
        raise TypeError("all oracle inputs must share one encoding")
    return arrs, enc.pop()


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def forward(X, Wq, Wk, Wv, H: int, G: int, d: int, causal: bool = True, nthreads: int | None = None,
            rope_theta: float = 0.0, q_norm=None, k_norm=None, qk_eps: float = 1e-6):
    """Return (O [S][H*d], LSE [H][S]) in fp64.  rope_theta > 0 applies the
    rotary embedding to queries and keys; q_norm and k_norm ([d], same
    encoding as X) apply QK-norm with qk_eps (see the C++ header)."""
    norm = q_norm is not None
    if norm != (k_norm is not None):
        raise ValueError("QK-norm needs both q_norm and k_norm")
    arrs, enc = _prep([X, Wq, Wk, Wv] + ([q_norm, k_norm] if norm else []))
    X, Wq, Wk, Wv = arrs[:4]
    S, D = X.shape
    _check_shapes(S, D, H, G, d, Wq, Wk, Wv)
    O = np.empty((S, H * d), np.float64)
    LSE = np.empty((H, S), np.float64)
    if norm:
        _check_norm(arrs[4], arrs[5], d)
        rc = _load().oracle_forward_qkn(S, D, H, G, d, int(bool(causal)), float(rope_theta),
                                        float(qk_eps), enc, _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                        _ptr(arrs[4]), _ptr(arrs[5]), _ptr(O), _ptr(LSE),
                                        nthreads or default_threads())
    else:
        rc = _load().oracle_forward(S, D, H, G, d, int(bool(causal)), float(rope_theta), enc,
                                    _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(O), _ptr(LSE),
                                    nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_forward rejected the shape")
    return O, LSE


def forward_rows(X, Wq, Wk, Wv, H: int, G: int, d: int, rows, causal: bool = True,
                 heads=None, nthreads: int | None = None, rope_theta: float = 0.0, q_norm=None,
                 k_norm=None, qk_eps: float = 1e-6):
    """Forward at the token rows `rows` only, for query heads range(*heads)
    (default: all): (O_rows [n][H*d], LSE_rows [H][n]) in fp64; entries of
    heads outside the range are NaN.  q_norm / k_norm as for forward()."""
    norm = q_norm is not None
    if norm != (k_norm is not None):
        raise ValueError("QK-norm needs both q_norm and k_norm")
    arrs, enc = _prep([X, Wq, Wk, Wv] + ([q_norm, k_norm] if norm else []))
    X, Wq, Wk, Wv = arrs[:4]
    S, D = X.shape
    _check_shapes(S, D, H, G, d, Wq, Wk, Wv)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    h0, h1 = heads if heads is not None else (0, H)
    O = np.full((n, H * d), np.nan, np.float64)
    LSE = np.full((H, n), np.nan, np.float64)
    if norm:
        _check_norm(arrs[4], arrs[5], d)
        rc = _load().oracle_forward_rows_qkn(S, D, H, G, d, int(bool(causal)), float(rope_theta),
                                             float(qk_eps), enc, _ptr(X), _ptr(Wq), _ptr(Wk),
                                             _ptr(Wv), _ptr(arrs[4]), _ptr(arrs[5]), _ptr(rows), n,
                                             int(h0), int(h1), _ptr(O), _ptr(LSE),
                                             nthreads or default_threads())
    else:
        rc = _load().oracle_forward_rows(S, D, H, G, d, int(bool(causal)), float(rope_theta), enc,
                                         _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(rows), n,
                                         int(h0), int(h1), _ptr(O), _ptr(LSE),
                                         nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_forward_rows rejected the shape or rows")
    return O, LSE


def backward(X, Wq, Wk, Wv, dO, H: int, G: int, d: int, causal: bool = True,
             nthreads: int | None = None, rope_theta: float = 0.0, q_norm=None, k_norm=None,
             qk_eps: float = 1e-6):
    """Forward + backward of L = sum(O * dO).

    Returns a dict of fp64 arrays: O, LSE, dX, dWq, dWk, dWv, and with QK-norm
    (q_norm, k_norm given) also dq_norm, dk_norm.
    """
    norm = q_norm is not None
    if norm != (k_norm is not None):
        raise ValueError("QK-norm needs both q_norm and k_norm")
    arrs, enc = _prep([X, Wq, Wk, Wv, dO] + ([q_norm, k_norm] if norm else []))
    X, Wq, Wk, Wv, dO = arrs[:5]
    S, D = X.shape
    _check_shapes(S, D, H, G, d, Wq, Wk, Wv)
    if dO.shape != (S, H * d):
        raise ValueError("dO must be [S][H*d]")
    out = {
        "O": np.empty((S, H * d), np.float64),
        "LSE": np.empty((H, S), np.float64),
        "dX": np.empty((S, D), np.float64),
        "dWq": np.empty((H * d, D), np.float64),
        "dWk": np.empty((G * d, D), np.float64),
        "dWv": np.empty((G * d, D), np.float64),
    }
    if norm:
        _check_norm(arrs[5], arrs[6], d)
        out["dq_norm"] = np.empty(d, np.float64)
        out["dk_norm"] = np.empty(d, np.float64)
        rc = _load().oracle_backward_qkn(S, D, H, G, d, int(bool(causal)), float(rope_theta),
                                         float(qk_eps), enc, _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                         _ptr(arrs[5]), _ptr(arrs[6]), _ptr(dO), _ptr(out["O"]),
                                         _ptr(out["LSE"]), _ptr(out["dX"]), _ptr(out["dWq"]),
                                         _ptr(out["dWk"]), _ptr(out["dWv"]), _ptr(out["dq_norm"]),
                                         _ptr(out["dk_norm"]), nthreads or default_threads())
    else:
        rc = _load().oracle_backward(S, D, H, G, d, int(bool(causal)), float(rope_theta), enc,
                                     _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(dO),
                                     _ptr(out["O"]), _ptr(out["LSE"]), _ptr(out["dX"]),
                                     _ptr(out["dWq"]), _ptr(out["dWk"]), _ptr(out["dWv"]),
                                     nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_backward rejected the shape")
    return out


def dx_tail(X, Wq, Wk, Wv, dO, H: int, G: int, d: int, t0: int, nthreads: int | None = None,
            rope_theta: float = 0.0):
    """Input gradient dX at rows t0 .. S-1 of the causal layer (fp64
    [S - t0][D]), exactly as oracle_backward defines it, at O((S - t0) S)
    attention cost (see the C++ source)."""
    (X, Wq, Wk, Wv, dO), enc = _prep([X, Wq, Wk, Wv, dO])
    S, D = X.shape
    _check_shapes(S, D, H, G, d, Wq, Wk, Wv)
    out = np.empty((S - t0, D), np.float64)
    rc = _load().oracle_dx_tail(S, D, H, G, d, float(rope_theta), enc, _ptr(X), _ptr(Wq), _ptr(Wk),
                                _ptr(Wv), _ptr(dO), int(t0), _ptr(out), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_dx_tail rejected the arguments")
    return out


def out_proj(O, Wo, dY=None, nthreads: int | None = None):
    """Output projection by definition (fp64): returns (Y, dO, dWo) with
    Y = O Wo^T, dO = dY Wo, dWo = dY^T O (dO and dWo are None without dY).
    O is fp64 [S][H*d]; Wo [D][H*d] and dY [S][D] share one encoding."""
    O = np.ascontiguousarray(O, dtype=np.float64)
    S, Hd = O.shape
    arrs, enc = _prep([Wo] + ([dY] if dY is not None else []))
    Wo = arrs[0]
    D = Wo.shape[0]
    if Wo.shape != (D, Hd):
        raise ValueError("Wo must be [D][H*d]")
    if dY is not None and arrs[1].shape != (S, D):
        raise ValueError("dY must be [S][D]")
    Y = np.empty((S, D), np.float64)
    dO = np.empty((S, Hd), np.float64) if dY is not None else None
    dWo = np.empty((D, Hd), np.float64) if dY is not None else None
    nul = ctypes.c_void_p(0)
    rc = _load().oracle_out_proj(S, D, Hd, enc, _ptr(O), _ptr(Wo),
                                 _ptr(arrs[1]) if dY is not None else nul, _ptr(Y),
                                 _ptr(dO) if dO is not None else nul,
                                 _ptr(dWo) if dWo is not None else nul, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_out_proj rejected the shape")
    return Y, dO, dWo


def decode_exact(a) -> np.ndarray:
    """fp64 copy of an oracle input (bf16 bit patterns, fp32 or fp64), exact."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError("unsupported oracle input dtype %s" % a.dtype)


def backward_out(X, Wq, Wk, Wv, Wo, dY, H: int, G: int, d: int, causal: bool = True,
                 nthreads: int | None = None, rope_theta: float = 0.0, q_norm=None, k_norm=None,
                 qk_eps: float = 1e-6):
    """The layer followed by its output projection, forward + backward of
    L = sum(Y * dY) with Y = O Wo^T.  Composes the definitions: attention
    forward, Y = O Wo^T, dO = dY Wo, then the attention backward with that dO
    (every input decoded exactly to fp64 first), and dWo = dY^T O.
    Returns a dict of fp64 arrays: O, LSE, Y, dX, dWq, dWk, dWv, dWo."""
    nk = dict(q_norm=q_norm, k_norm=k_norm, qk_eps=qk_eps)
    O, LSE = forward(X, Wq, Wk, Wv, H, G, d, causal=causal, nthreads=nthreads,
                     rope_theta=rope_theta, **nk)
    Y, dO, dWo = out_proj(O, Wo, dY, nthreads=nthreads)
    ex = [decode_exact(a) for a in (X, Wq, Wk, Wv)]
    if q_norm is not None:
        nk.update(q_norm=decode_exact(q_norm), k_norm=decode_exact(k_norm))
    out = backward(*ex, dO, H, G, d, causal=causal, nthreads=nthreads, rope_theta=rope_theta, **nk)
    out["Y"] = Y
    out["dWo"] = dWo
    return out


def _check_norm(gq, gk, d):
    if gq.shape != (d,) or gk.shape != (d,):
        raise ValueError("q_norm and k_norm must be [d_head]")


def _check_shapes(S, D, H, G, d, Wq, Wk, Wv):
    if H % G != 0:
        raise ValueError("G must divide H")
    if Wq.shape != (H * d, D) or Wk.shape != (G * d, D) or Wv.shape != (G * d, D):
        raise ValueError("weight shapes must be Wq [H*d][D], Wk/Wv [G*d][D]")
