"""Thin ctypes binding of the upipe C ABI (include/upipe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Tensors may be passed as torch tensors (their data_ptr is used) or as raw
integer device addresses.  The library must have been built
(``python -m headwise_chunked_context_stage_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libupipe.so")

UPIPE_BF16, UPIPE_F32 = 0, 1
UPIPE_OK, UPIPE_ERR_ARG, UPIPE_ERR_UNSUPPORTED, UPIPE_ERR_WORKSPACE, UPIPE_ERR_HIP = 0, 1, 2, 3, 4
UPIPE_PIPELINE = 1  # plan flag: stage pipelining on a second stream
UPIPE_OUT_PROJ = 2  # plan flag: workspace for upipe_bwd_out (output projection)
UPIPE_QK_NORM = 4   # plan flag: per-head RMSNorm of queries and keys (upipe_fwd_ex / upipe_bwd_ex)
KERNEL_KINDS = ("proj", "attn_fwd", "bwd_pre", "attn_dkv", "attn_dq", "dw", "dx", "fill",
                "oproj", "dout", "dwo", "norm")

EXPORTS = ("upipe_create", "upipe_create_ex", "upipe_create_rope", "upipe_destroy", "upipe_peak_bytes", "upipe_peak_bytes_phase",
           "upipe_fwd", "upipe_bwd", "upipe_strerror", "upipe_num_stages", "upipe_stage_info",
           "upipe_timing_enable", "upipe_timing_read", "upipe_kernel_name", "upipe_mfma_ceiling",
           "upipe_auto_u", "upipe_fwd_out", "upipe_bwd_out", "upipe_fwd_noalloc",
           "upipe_noalloc_max_bytes", "upipe_create_opt", "upipe_fwd_ex", "upipe_bwd_ex")

_lib = None


class Options(ctypes.Structure):
    """upipe_options"""
    _fields_ = [("flags", ctypes.c_int), ("rope_theta", ctypes.c_double),
                ("qk_norm_eps", ctypes.c_double)]


FWD_IO_FIELDS = ("X", "Wq", "Wk", "Wv", "q_norm", "k_norm", "Wo", "O", "LSE", "Y")
BWD_IO_FIELDS = ("dO", "dY", "X", "Wq", "Wk", "Wv", "q_norm", "k_norm", "Wo", "O", "LSE", "dX",
                 "dWq", "dWk", "dWv", "dq_norm", "dk_norm", "dWo")


class FwdIO(ctypes.Structure):
    """upipe_fwd_io: every member a device address (0 = NULL)."""
    _fields_ = [(n, ctypes.c_void_p) for n in FWD_IO_FIELDS]


class BwdIO(ctypes.Structure):
    """upipe_bwd_io"""
    _fields_ = [(n, ctypes.c_void_p) for n in BWD_IO_FIELDS]


class UpipeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s: %s (code %d)" % (where, strerror_text(code), code))


def lib():
    """Load libupipe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libupipe.so is not built: run `python -m "
                           "headwise_chunked_context_stage_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.upipe_create.argtypes = [ctypes.POINTER(vp), i64, i64, i32, i32, i32, i32, i32, i32]
    L.upipe_create.restype = i32
    L.upipe_create_ex.argtypes = [ctypes.POINTER(vp), i64, i64, i32, i32, i32, i32, i32, i32, i32]
    L.upipe_create_ex.restype = i32
    L.upipe_create_rope.argtypes = [ctypes.POINTER(vp), i64, i64, i32, i32, i32, i32, i32, i32, i32,
                                    ctypes.c_double]
    L.upipe_create_rope.restype = i32
    L.upipe_destroy.argtypes = [vp]
    L.upipe_destroy.restype = None
    L.upipe_peak_bytes.argtypes = [vp]
    L.upipe_peak_bytes.restype = sz
    L.upipe_peak_bytes_phase.argtypes = [vp, i32]
    L.upipe_peak_bytes_phase.restype = sz
    L.upipe_fwd.argtypes = [vp] * 8 + [sz, vp]
    L.upipe_fwd.restype = i32
    L.upipe_bwd.argtypes = [vp] * 13 + [sz, vp]
    L.upipe_bwd.restype = i32
    L.upipe_fwd_out.argtypes = [vp] * 10 + [sz, vp]
    L.upipe_fwd_out.restype = i32
    L.upipe_bwd_out.argtypes = [vp] * 15 + [sz, vp]
    L.upipe_bwd_out.restype = i32
    L.upipe_strerror.argtypes = [i32]
    L.upipe_strerror.restype = ctypes.c_char_p
    L.upipe_num_stages.argtypes = [vp]
    L.upipe_num_stages.restype = i32
    L.upipe_stage_info.argtypes = [vp, i32] + [ctypes.POINTER(i32)] * 6
    L.upipe_stage_info.restype = i32
    L.upipe_timing_enable.argtypes = [i32]
    L.upipe_timing_enable.restype = i32
    L.upipe_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), i32]
    L.upipe_timing_read.restype = i32
    L.upipe_kernel_name.argtypes = [i32]
    L.upipe_kernel_name.restype = ctypes.c_char_p
    L.upipe_mfma_ceiling.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_double), vp]
    L.upipe_mfma_ceiling.restype = i32
    L.upipe_auto_u.argtypes = [i64, i64, i32, i32, i32, i32, i32, sz, ctypes.POINTER(i32)]
    L.upipe_auto_u.restype = i32
    L.upipe_create_opt.argtypes = [ctypes.POINTER(vp), i64, i64, i32, i32, i32, i32, i32, i32,
                                   ctypes.POINTER(Options)]
    L.upipe_create_opt.restype = i32
    L.upipe_fwd_ex.argtypes = [vp, ctypes.POINTER(FwdIO), vp, sz, vp]
    L.upipe_fwd_ex.restype = i32
    L.upipe_bwd_ex.argtypes = [vp, ctypes.POINTER(BwdIO), vp, sz, vp]
    L.upipe_bwd_ex.restype = i32
    L.upipe_fwd_noalloc.argtypes = [vp] * 8
    L.upipe_fwd_noalloc.restype = i32
    L.upipe_noalloc_max_bytes.argtypes = []
    L.upipe_noalloc_max_bytes.restype = sz
    _lib = L
    return L


def strerror_text(code: int) -> str:
    try:
        return lib().upipe_strerror(code).decode()
    except Exception:  # pragma: no cover - only when the library is missing
        return "error"


def _addr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def _stream(stream, *tensors) -> int:
    if stream is not None:
        return stream if isinstance(stream, int) else int(stream.cuda_stream)
    for t in tensors:
        if hasattr(t, "is_cuda") and t.is_cuda:
            import torch

            return int(torch.cuda.current_stream(t.device).cuda_stream)
    return 0


def _check(code: int, where: str):
    if code != UPIPE_OK:
        raise UpipeError(code, where)


def _dtype_code(dtype) -> int:
    if dtype in (UPIPE_BF16, "bf16", "bfloat16"):
        return UPIPE_BF16
    if dtype in (UPIPE_F32, "f32", "fp32", "float32"):
        return UPIPE_F32
    try:
        import torch

        if dtype == torch.bfloat16:
            return UPIPE_BF16
        if dtype == torch.float32:
            return UPIPE_F32
    except ImportError:  # pragma: no cover
        pass
    return int(dtype)


def upipe_create(S, d_model, H, G, d_head, U, causal=1, dtype="bf16") -> int:
    h = ctypes.c_void_p()
    _check(lib().upipe_create(ctypes.byref(h), S, d_model, H, G, d_head, U, int(causal),
                              _dtype_code(dtype)), "upipe_create")
    return h.value


def upipe_create_ex(S, d_model, H, G, d_head, U, causal=1, dtype="bf16", flags=0) -> int:
    h = ctypes.c_void_p()
    _check(lib().upipe_create_ex(ctypes.byref(h), S, d_model, H, G, d_head, U, int(causal),
                                 _dtype_code(dtype), int(flags)), "upipe_create_ex")
    return h.value


def upipe_create_rope(S, d_model, H, G, d_head, U, causal=1, dtype="bf16", flags=0,
                      rope_theta=0.0) -> int:
    h = ctypes.c_void_p()
    _check(lib().upipe_create_rope(ctypes.byref(h), S, d_model, H, G, d_head, U, int(causal),
                                   _dtype_code(dtype), int(flags), float(rope_theta)),
           "upipe_create_rope")
    return h.value


def upipe_create_opt(S, d_model, H, G, d_head, U, causal=1, dtype="bf16", flags=0,
                     rope_theta=0.0, qk_norm_eps=0.0) -> int:
    h = ctypes.c_void_p()
    opt = Options(int(flags), float(rope_theta), float(qk_norm_eps))
    _check(lib().upipe_create_opt(ctypes.byref(h), S, d_model, H, G, d_head, U, int(causal),
                                  _dtype_code(dtype), ctypes.byref(opt)), "upipe_create_opt")
    return h.value


def upipe_fwd_ex(plan, io: dict, ws, ws_bytes=None, stream=None) -> None:
    """io: tensors (or addresses) by the names of upipe_fwd_io; missing = NULL."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    s = FwdIO(*[_addr(io.get(n)) for n in FWD_IO_FIELDS])
    _check(lib().upipe_fwd_ex(plan, ctypes.byref(s), _addr(ws), ws_bytes,
                              _stream(stream, io.get("X"), io.get("O"))), "upipe_fwd_ex")


def upipe_bwd_ex(plan, io: dict, ws, ws_bytes=None, stream=None) -> None:
    """io: tensors (or addresses) by the names of upipe_bwd_io; missing = NULL."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    s = BwdIO(*[_addr(io.get(n)) for n in BWD_IO_FIELDS])
    _check(lib().upipe_bwd_ex(plan, ctypes.byref(s), _addr(ws), ws_bytes,
                              _stream(stream, io.get("dX"), io.get("dWq"))), "upipe_bwd_ex")


def upipe_destroy(plan) -> None:
    lib().upipe_destroy(plan)


def upipe_peak_bytes(plan) -> int:
    return int(lib().upipe_peak_bytes(plan))


def upipe_peak_bytes_phase(plan, phase: int) -> int:
    return int(lib().upipe_peak_bytes_phase(plan, phase))


def upipe_fwd(plan, X, Wq, Wk, Wv, O, LSE, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().upipe_fwd(plan, _addr(X), _addr(Wq), _addr(Wk), _addr(Wv), _addr(O), _addr(LSE),
                           _addr(ws), ws_bytes, _stream(stream, X, O)), "upipe_fwd")


def upipe_bwd(plan, dO, X, Wq, Wk, Wv, O, LSE, dX, dWq, dWk, dWv, ws, ws_bytes=None,
              stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().upipe_bwd(plan, _addr(dO), _addr(X), _addr(Wq), _addr(Wk), _addr(Wv), _addr(O),
                           _addr(LSE), _addr(dX), _addr(dWq), _addr(dWk), _addr(dWv), _addr(ws),
                           ws_bytes, _stream(stream, dX, dWq)), "upipe_bwd")


def upipe_fwd_out(plan, X, Wq, Wk, Wv, Wo, O, LSE, Y, ws, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().upipe_fwd_out(plan, _addr(X), _addr(Wq), _addr(Wk), _addr(Wv), _addr(Wo), _addr(O),
                               _addr(LSE), _addr(Y), _addr(ws), ws_bytes, _stream(stream, X, Y)),
           "upipe_fwd_out")


def upipe_bwd_out(plan, dY, X, Wq, Wk, Wv, Wo, O, LSE, dX, dWq, dWk, dWv, dWo, ws, ws_bytes=None,
                  stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if hasattr(ws, "numel") else 0
    _check(lib().upipe_bwd_out(plan, _addr(dY), _addr(X), _addr(Wq), _addr(Wk), _addr(Wv),
                               _addr(Wo), _addr(O), _addr(LSE), _addr(dX), _addr(dWq), _addr(dWk),
                               _addr(dWv), _addr(dWo), _addr(ws), ws_bytes,
                               _stream(stream, dX, dWq)), "upipe_bwd_out")


def upipe_fwd_noalloc(plan, X, Wq, Wk, Wv, O, LSE, stream=None) -> None:
    """upipe_fwd without a workspace: the library's static device array holds
    the stage buffers (no allocation; calls overlapping on one GPU race)."""
    _check(lib().upipe_fwd_noalloc(plan, _addr(X), _addr(Wq), _addr(Wk), _addr(Wv), _addr(O),
                                   _addr(LSE), _stream(stream, X, O)), "upipe_fwd_noalloc")


def upipe_noalloc_max_bytes() -> int:
    return int(lib().upipe_noalloc_max_bytes())


def upipe_strerror(code: int) -> str:
    return lib().upipe_strerror(code).decode()


def upipe_num_stages(plan) -> int:
    return int(lib().upipe_num_stages(plan))


def upipe_stage_info(plan, s: int) -> dict:
    vals = [ctypes.c_int() for _ in range(6)]
    _check(lib().upipe_stage_info(plan, s, *[ctypes.byref(v) for v in vals]), "upipe_stage_info")
    keys = ("q_first", "q_count", "kv_first", "kv_count", "kv_load", "kv_done")
    return {k: v.value for k, v in zip(keys, vals)}


def upipe_timing_enable(on: bool) -> None:
    _check(lib().upipe_timing_enable(int(bool(on))), "upipe_timing_enable")


def upipe_timing_read() -> dict:
    """Per kernel kind: {"ms": total milliseconds, "launches": count}; resets."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().upipe_timing_read(ms, cnt, n), "upipe_timing_read")
    return {KERNEL_KINDS[i]: {"ms": ms[i], "launches": cnt[i]} for i in range(n)}


def upipe_kernel_name(kind: int) -> str:
    return lib().upipe_kernel_name(kind).decode()


def upipe_mfma_ceiling(waves_per_simd: int = 2, iters: int = 1 << 14, stream=None) -> float:
    """Measured dense bf16 MFMA TFLOP/s over every CU (synchronous)."""
    out = ctypes.c_double(0.0)
    _check(lib().upipe_mfma_ceiling(waves_per_simd, iters, ctypes.byref(out), _stream(stream)),
           "upipe_mfma_ceiling")
    return out.value


def upipe_auto_u(S: int, d_model: int, H: int, G: int, d_head: int, budget_bytes: int,
                 causal: bool = True, dtype="bf16") -> int:
    """Largest legal U whose workspace fits budget_bytes (host only)."""
    out = ctypes.c_int(0)
    _check(lib().upipe_auto_u(S, d_model, H, G, d_head, int(bool(causal)), _dtype_code(dtype),
                              budget_bytes, ctypes.byref(out)), "upipe_auto_u")
    return out.value


def _check_layout(t, name, shape, dtype):
    """Refuse a tensor the library would read or write out of bounds: not a
    tensor, wrong shape or element type, not contiguous."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: expected a torch tensor, got %s" % (name, type(t).__name__))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s: not contiguous" % name)


def _check_place(t, name, device, align=16):
    """... or one in host memory, on another device, or misaligned."""
    if t.device.type != "cuda" or t.device != device:
        raise ValueError("%s: on %s, expected a GPU tensor on %s" % (name, t.device, device))
    if t.numel() and t.data_ptr() % align:
        raise ValueError("%s: data pointer not %d-byte aligned" % (name, align))


class Plan:
    """Owns a plan handle; the layer's shape and stage size U are fixed here.

    The methods check every tensor against the plan (shape, element type,
    contiguity, device, alignment) before calling the library, which itself
    can only check pointers for null and alignment."""

    def __init__(self, S, d_model, H, G, d_head, U, causal=True, dtype="bf16", pipeline=False,
                 rope_theta=0.0, out_proj=False, qk_norm=False, qk_norm_eps=1e-6):
        self.S, self.D, self.H, self.G, self.d, self.U = S, d_model, H, G, d_head, U
        self.causal = bool(causal)
        self.pipeline = bool(pipeline)
        self.out_proj = bool(out_proj)
        self.qk_norm = bool(qk_norm)
        self.qk_norm_eps = float(qk_norm_eps)
        self.rope_theta = float(rope_theta)
        self.dtype = "bf16" if _dtype_code(dtype) == UPIPE_BF16 else "f32"
        flags = (UPIPE_PIPELINE if self.pipeline else 0) | (UPIPE_OUT_PROJ if self.out_proj else 0)
        if self.qk_norm:
            self.handle = upipe_create_opt(S, d_model, H, G, d_head, U, int(self.causal), dtype,
                                           flags | UPIPE_QK_NORM, self.rope_theta,
                                           self.qk_norm_eps)
        elif self.rope_theta != 0.0 or self.out_proj:
            self.handle = upipe_create_rope(S, d_model, H, G, d_head, U, int(self.causal), dtype,
                                            flags, self.rope_theta)
        elif self.pipeline:
            self.handle = upipe_create_ex(S, d_model, H, G, d_head, U, int(self.causal), dtype,
                                          UPIPE_PIPELINE)
        else:
            self.handle = upipe_create(S, d_model, H, G, d_head, U, int(self.causal), dtype)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                upipe_destroy(h)
            except Exception:  # pragma: no cover
                pass
            self.handle = None

    @property
    def peak_bytes(self) -> int:
        return upipe_peak_bytes(self.handle)

    def peak_bytes_phase(self, phase: int) -> int:
        return upipe_peak_bytes_phase(self.handle, phase)

    @property
    def num_stages(self) -> int:
        return upipe_num_stages(self.handle)

    def stage_info(self, s: int) -> dict:
        return upipe_stage_info(self.handle, s)

    def _check(self, phase, ws, ws_bytes, **tensors):
        import torch

        S, D, H, G, d = self.S, self.D, self.H, self.G, self.d
        el = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        f32 = torch.float32
        expect = {
            "X": ((S, D), el), "Wq": ((H * d, D), el), "Wk": ((G * d, D), el),
            "Wv": ((G * d, D), el), "O": ((S, H * d), el), "LSE": ((H, S), f32),
            "dO": ((S, H * d), el), "dX": ((S, D), f32), "dWq": ((H * d, D), f32),
            "dWk": ((G * d, D), f32), "dWv": ((G * d, D), f32), "Wo": ((D, H * d), el),
            "Y": ((S, D), f32), "dY": ((S, D), el), "dWo": ((D, H * d), f32),
            "q_norm": ((d,), el), "k_norm": ((d,), el), "dq_norm": ((d,), f32),
            "dk_norm": ((d,), f32),
        }
        for name, t in tensors.items():
            _check_layout(t, name, *expect[name])
        if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
            raise TypeError("ws: expected a contiguous torch tensor")
        have = ws.numel() * ws.element_size()
        need = self.peak_bytes_phase(phase)
        if (ws_bytes if ws_bytes is not None else have) > have or have < need:
            raise ValueError("ws: %d bytes, the plan needs %d" % (have, need))
        device = tensors["X"].device
        for name, t in tensors.items():
            _check_place(t, name, device)
        _check_place(ws, "ws", device, align=256)

    def fwd(self, X, Wq, Wk, Wv, O, LSE, ws, ws_bytes=None, stream=None):
        self._check(0, ws, ws_bytes, X=X, Wq=Wq, Wk=Wk, Wv=Wv, O=O, LSE=LSE)
        upipe_fwd(self.handle, X, Wq, Wk, Wv, O, LSE, ws, ws_bytes, stream)

    def bwd(self, dO, X, Wq, Wk, Wv, O, LSE, dX, dWq, dWk, dWv, ws, ws_bytes=None, stream=None):
        self._check(1, ws, ws_bytes, X=X, Wq=Wq, Wk=Wk, Wv=Wv, O=O, LSE=LSE, dO=dO, dX=dX,
                    dWq=dWq, dWk=dWk, dWv=dWv)
        upipe_bwd(self.handle, dO, X, Wq, Wk, Wv, O, LSE, dX, dWq, dWk, dWv, ws, ws_bytes, stream)

    def fwd_ex(self, io: dict, ws, ws_bytes=None, stream=None):
        """Forward of any plan; io holds the tensors of upipe_fwd_io by name
        (the ones the plan uses: q_norm, k_norm with QK-norm; Wo, Y with the
        output projection)."""
        want = ["X", "Wq", "Wk", "Wv", "O", "LSE"] + (["q_norm", "k_norm"] if self.qk_norm else []) \
            + (["Wo", "Y"] if self.out_proj else [])
        extra = set(k for k, v in io.items() if v is not None) - set(want)
        if extra:
            raise ValueError("tensors this plan does not use: %s" % sorted(extra))
        self._check(0, ws, ws_bytes, **{k: io.get(k) for k in want})
        upipe_fwd_ex(self.handle, io, ws, ws_bytes, stream)

    def bwd_ex(self, io: dict, ws, ws_bytes=None, stream=None):
        """Backward of any plan; io holds the tensors of upipe_bwd_io by name."""
        want = ["X", "Wq", "Wk", "Wv", "O", "LSE", "dX", "dWq", "dWk", "dWv"] \
            + (["q_norm", "k_norm", "dq_norm", "dk_norm"] if self.qk_norm else []) \
            + (["Wo", "dY", "dWo"] if self.out_proj else ["dO"])
        extra = set(k for k, v in io.items() if v is not None) - set(want)
        if extra:
            raise ValueError("tensors this plan does not use: %s" % sorted(extra))
        self._check(1, ws, ws_bytes, **{k: io.get(k) for k in want})
        upipe_bwd_ex(self.handle, io, ws, ws_bytes, stream)

    def fwd_noalloc(self, X, Wq, Wk, Wv, O, LSE, stream=None):
        tensors = dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv, O=O, LSE=LSE)
        import torch

        el = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        S, D, H, G, d = self.S, self.D, self.H, self.G, self.d
        expect = {"X": ((S, D), el), "Wq": ((H * d, D), el), "Wk": ((G * d, D), el),
                  "Wv": ((G * d, D), el), "O": ((S, H * d), el), "LSE": ((H, S), torch.float32)}
        for name, t in tensors.items():
            _check_layout(t, name, *expect[name])
        for name, t in tensors.items():
            _check_place(t, name, X.device)
        upipe_fwd_noalloc(self.handle, X, Wq, Wk, Wv, O, LSE, stream)

    def fwd_out(self, X, Wq, Wk, Wv, Wo, O, LSE, Y, ws, ws_bytes=None, stream=None):
        self._check(0, ws, ws_bytes, X=X, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, O=O, LSE=LSE, Y=Y)
        upipe_fwd_out(self.handle, X, Wq, Wk, Wv, Wo, O, LSE, Y, ws, ws_bytes, stream)

    def bwd_out(self, dY, X, Wq, Wk, Wv, Wo, O, LSE, dX, dWq, dWk, dWv, dWo, ws, ws_bytes=None,
                stream=None):
        self._check(1, ws, ws_bytes, X=X, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, O=O, LSE=LSE, dY=dY, dX=dX,
                    dWq=dWq, dWk=dWk, dWv=dWv, dWo=dWo)
        upipe_bwd_out(self.handle, dY, X, Wq, Wk, Wv, Wo, O, LSE, dX, dWq, dWk, dWv, dWo, ws,
                      ws_bytes, stream)
