"""ctypes binding of libmhc.so: argument marshalling only.

Each function has the name of the C entry point it calls (without the
``mhc_`` prefix).  Tensors must be CUDA (HIP) tensors, contiguous, with the
dtypes of ``include/mhc.h``; bf16 tensors are passed as their raw bits.  Work
is enqueued on torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from .params import Params

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmhc.so")

FLAG_MXFP8 = 1
FLAG_RECOMPUTE_X = 2
FLAG_DEFER_SINKHORN = 4
FLAG_MXFP8_MFMA_SCALES = 8
_STATUS = {0: "MHC_OK", 1: "MHC_ERR_NULL", 2: "MHC_ERR_SHAPE", 3: "MHC_ERR_ALIGN", 4: "MHC_ERR_ALIAS",
           5: "MHC_ERR_FLAGS", 6: "MHC_ERR_WORKSPACE", 7: "MHC_ERR_PARAM", 8: "MHC_ERR_HIP", 9: "MHC_ERR_EXPIRED",
           10: "MHC_ERR_SCRATCH"}
ERR_EXPIRED = 9
ERR_SCRATCH = 10


class MhcParams(ctypes.Structure):
    _fields_ = [("hc_norm_eps", ctypes.c_float), ("rmsnorm_eps", ctypes.c_float),
                ("hc_post_scale", ctypes.c_float), ("sinkhorn_eps", ctypes.c_float),
                ("sinkhorn_iters", ctypes.c_int32)]

    @classmethod
    def of(cls, p: Params) -> "MhcParams":
        return cls(p.hc_norm_eps, p.rmsnorm_eps, p.hc_post_scale, p.sinkhorn_eps, p.sinkhorn_iters)


class MhcError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        msg = f"{what}: {self.name}"
        if _LIB is not None:
            msg += " (" + _LIB.mhc_strerror(status).decode() + ")"
            if status == 8:
                msg += f", hipError {_LIB.mhc_last_hip_error()}"
        super().__init__(msg)


_LIB = None
_LOCK = threading.Lock()

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIG = {
    "mhc_abi_version": ([], ctypes.c_int),
    "mhc_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "mhc_last_hip_error": ([], ctypes.c_int),
    "mhc_workspace_bytes": ([_I64, _I64, ctypes.c_uint], ctypes.c_size_t),
    "mhc_workspace_init": ([_P, ctypes.c_size_t, _P], ctypes.c_int),
    "mhc_workspace_check": ([_P, _P], ctypes.c_int),
    "mhc_sinkhorn": ([_P, _I64, ctypes.POINTER(MhcParams), _P], ctypes.c_int),
    "mhc_phi_packed_bytes": ([_I64], ctypes.c_size_t),
    "mhc_schedule": ([_I64, _I64, ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    "mhc_pack_phi": ([_P, _I64, _P, _P], ctypes.c_int),
    "mhc_coeffs": ([_P, _I64, _I64, _P, _P, ctypes.POINTER(MhcParams), _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "mhc_coeffs_prepacked": ([_P, _I64, _I64, _P, _P, ctypes.POINTER(MhcParams), _P, _P, ctypes.c_size_t, _P],
                             ctypes.c_int),
    "mhc_pre": ([_P, _P, _P, _I64, _I64, ctypes.POINTER(MhcParams), _P, _P], ctypes.c_int),
    "mhc_pre_broadcast": ([_P, _I64, _I64, _P, _P, _P, ctypes.POINTER(MhcParams), _P, _P, _P, ctypes.c_size_t, _P],
                          ctypes.c_int),
    "mhc_pre_broadcast_prepacked": ([_P, _I64, _I64, _P, _P, _P, ctypes.POINTER(MhcParams), _P, _P, _P,
                                     ctypes.c_size_t, _P], ctypes.c_int),
    "mhc_post": ([_P, _P, _P, _I64, _I64, _P, _P], ctypes.c_int),
    "mhc_post_int8": ([_P, _P, _P, _P, _I64, _I64, _P, _P], ctypes.c_int),
    "mhc_post_int8_pre_fused": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.POINTER(MhcParams), ctypes.c_uint,
                                 _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "mhc_post_int8_pre_fused_prepacked": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.POINTER(MhcParams),
                                           ctypes.c_uint, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "mhc_post_pre_fused": ([_P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.POINTER(MhcParams), ctypes.c_uint,
                            _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "mhc_post_pre_fused_prepacked": ([_P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.POINTER(MhcParams),
                                      ctypes.c_uint, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "mhc_post_pre_fused_prepacked_static": ([_P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.POINTER(MhcParams),
                                             ctypes.c_uint, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """Load libmhc.so (once).  Raises if it has not been built."""
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m manifold_constrained_hyper_mhc_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in _SIG.items():
                fn = getattr(L, name)
                fn.argtypes = args
                fn.restype = res
            _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != 0:
        raise MhcError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(x):
    if not isinstance(x, torch.Tensor) or x.dim() != 3 or x.shape[1] != 4:
        raise ValueError("x must have shape [T, 4, C]")
    return int(x.shape[0]), int(x.shape[2])


# workspaces cached per (device, stream): a workspace must not be shared by
# calls that can run concurrently
_WS = {}


def workspace(T: int, C: int, device=None, *, fresh: bool = False) -> torch.Tensor:
    """A cleared workspace of at least mhc_workspace_bytes(T, C) bytes."""
    L = lib()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    need = int(L.mhc_workspace_bytes(T, C, 0))
    if need == 0:
        raise MhcError(2, "mhc_workspace_bytes")
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = None if fresh else _WS.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _check(L.mhc_workspace_init(_ptr(ws), ws.numel(), _stream(dev)), "mhc_workspace_init")
        if not fresh:
            _WS[key] = ws
    return ws


def schedule(T: int, C: int) -> str:
    """"persistent" or "staged": the kernel mhc_coeffs and mhc_post_pre_fused
    run for this shape on the current device (MHC_SCHEDULE=staged forces the
    staged one)."""
    out = ctypes.c_int(-1)
    _check(lib().mhc_schedule(T, C, ctypes.byref(out)), "mhc_schedule")
    return "persistent" if out.value == 1 else "staged"


def check(ws: torch.Tensor) -> None:
    """Raise MhcError (MHC_ERR_EXPIRED) if a bounded wait of any call that used
    the workspace ``ws`` has expired since it was cleared: those calls'
    outputs are invalid.  Synchronises torch's current stream
    (mhc_workspace_check), so it belongs after the calls, not between them."""
    _check(lib().mhc_workspace_check(_ptr(ws), _stream(ws.device)), "mhc_workspace_check")


def workspace_error(ws: torch.Tensor) -> int:
    """The workspace's error word (its first 4 bytes): nonzero once a bounded
    wait of a kernel that used it expired.  Synchronises with the device."""
    return int(ws[:4].cpu().view(torch.int32).item())


def pack_phi(phi: torch.Tensor) -> torch.Tensor:
    L = lib()
    C = phi.shape[0] // 4
    _need(phi, "phi", torch.float32, (4 * C, 24))
    out = torch.empty(int(L.mhc_phi_packed_bytes(C)), dtype=torch.uint8, device=phi.device)
    _check(L.mhc_pack_phi(_ptr(phi), C, _ptr(out), _stream(phi.device)), "mhc_pack_phi")
    return out


def coeffs(x, phi, bias, params: Params = Params(), *, ws=None, out=None) -> torch.Tensor:
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(phi, "phi", torch.float32, (4 * C, 24), dev)
    _need(bias, "bias", torch.float32, (24,), dev)
    out = torch.empty((T, 24), dtype=torch.float32, device=dev) if out is None else out
    _need(out, "coeffs", torch.float32, (T, 24), dev)
    ws = workspace(T, C, dev) if ws is None else ws
    p = MhcParams.of(params)
    _check(L.mhc_coeffs(_ptr(x), T, C, _ptr(phi), _ptr(bias), ctypes.byref(p), _ptr(out), _ptr(ws), ws.numel(),
                        _stream(dev)), "mhc_coeffs")
    return out


def coeffs_prepacked(x, phi_packed, bias, params: Params = Params(), *, ws=None, out=None) -> torch.Tensor:
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(phi_packed, "phi_packed", torch.uint8, (int(L.mhc_phi_packed_bytes(C)),), dev)
    _need(bias, "bias", torch.float32, (24,), dev)
    out = torch.empty((T, 24), dtype=torch.float32, device=dev) if out is None else out
    _need(out, "coeffs", torch.float32, (T, 24), dev)
    ws = workspace(T, C, dev) if ws is None else ws
    p = MhcParams.of(params)
    _check(L.mhc_coeffs_prepacked(_ptr(x), T, C, _ptr(phi_packed), _ptr(bias), ctypes.byref(p), _ptr(out),
                                  _ptr(ws), ws.numel(), _stream(dev)), "mhc_coeffs_prepacked")
    return out


def pre_broadcast(x0, phi, bias, gamma, params: Params = Params(), *, ws=None, coeffs_out=None,
                  h_out=None, phi_packed=None):
    """Coefficients and pre of the [T, C] stream x0 broadcast to the 4 routes
    (mhc_pre_broadcast, or mhc_pre_broadcast_prepacked when phi_packed is
    given and phi is None).  Returns (coeffs [T, 24], h [T, C])."""
    L = lib()
    if not isinstance(x0, torch.Tensor) or x0.dim() != 2:
        raise ValueError("x0 must have shape [T, C]")
    T, C = int(x0.shape[0]), int(x0.shape[1])
    dev = x0.device
    _need(x0, "x0", torch.bfloat16, (T, C))
    if phi is not None:
        _need(phi, "phi", torch.float32, (4 * C, 24), dev)
    else:
        _need(phi_packed, "phi_packed", torch.uint8, (int(L.mhc_phi_packed_bytes(C)),), dev)
    _need(bias, "bias", torch.float32, (24,), dev)
    _need(gamma, "gamma", torch.float32, (C,), dev)
    cf = torch.empty((T, 24), dtype=torch.float32, device=dev) if coeffs_out is None else coeffs_out
    h = _placed_empty((T, C), torch.bfloat16, dev, x0) if h_out is None else h_out
    _need(cf, "coeffs", torch.float32, (T, 24), dev)
    _need(h, "h", torch.bfloat16, (T, C), dev)
    ws = workspace(T, C, dev) if ws is None else ws
    p = MhcParams.of(params)
    if phi is not None:
        _check(L.mhc_pre_broadcast(_ptr(x0), T, C, _ptr(phi), _ptr(bias), _ptr(gamma), ctypes.byref(p), _ptr(cf),
                                   _ptr(h), _ptr(ws), ws.numel(), _stream(dev)), "mhc_pre_broadcast")
    else:
        _check(L.mhc_pre_broadcast_prepacked(_ptr(x0), T, C, _ptr(phi_packed), _ptr(bias), _ptr(gamma),
                                             ctypes.byref(p), _ptr(cf), _ptr(h), _ptr(ws), ws.numel(),
                                             _stream(dev)), "mhc_pre_broadcast_prepacked")
    return cf, h


def pre(x, coeffs_t, gamma, params: Params = Params(), *, out=None) -> torch.Tensor:
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(coeffs_t, "coeffs", torch.float32, (T, 24), dev)
    _need(gamma, "gamma", torch.float32, (C,), dev)
    out = _placed_empty((T, C), torch.bfloat16, dev, x) if out is None else out
    _need(out, "h", torch.bfloat16, (T, C), dev)
    p = MhcParams.of(params)
    _check(L.mhc_pre(_ptr(x), _ptr(coeffs_t), _ptr(gamma), T, C, ctypes.byref(p), _ptr(out), _stream(dev)),
           "mhc_pre")
    return out


def post(x, y, coeffs_t, *, out=None) -> torch.Tensor:
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(y, "y", torch.bfloat16, (T, C), dev)
    _need(coeffs_t, "coeffs", torch.float32, (T, 24), dev)
    out = _placed_empty((T, 4, C), torch.bfloat16, dev, x) if out is None else out
    _need(out, "x_out", torch.bfloat16, (T, 4, C), dev)
    _check(L.mhc_post(_ptr(x), _ptr(y), _ptr(coeffs_t), T, C, _ptr(out), _stream(dev)), "mhc_post")
    return out


def post_int8(x, y_q, y_scale, coeffs_t, *, out=None) -> torch.Tensor:
    """Post of an int8 sublayer output y_q [T, C] with per-token fp32 scales
    y_scale [T] (mhc_post_int8)."""
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(y_q, "y_q", torch.int8, (T, C), dev)
    _need(y_scale, "y_scale", torch.float32, (T,), dev)
    _need(coeffs_t, "coeffs", torch.float32, (T, 24), dev)
    out = _placed_empty((T, 4, C), torch.bfloat16, dev, x) if out is None else out
    _need(out, "x_out", torch.bfloat16, (T, 4, C), dev)
    _check(L.mhc_post_int8(_ptr(x), _ptr(y_q), _ptr(y_scale), _ptr(coeffs_t), T, C, _ptr(out), _stream(dev)),
           "mhc_post_int8")
    return out


def _flags(mxfp8, recompute_x: bool, defer_sinkhorn: bool = False) -> int:
    """mxfp8: False, True (linear scale layout) or "mfma" (the MX matrix-core
    operand order of the scales, MHC_FLAG_MXFP8_MFMA_SCALES)."""
    return ((FLAG_MXFP8 if mxfp8 else 0) | (FLAG_MXFP8_MFMA_SCALES if mxfp8 == "mfma" else 0) |
            (FLAG_RECOMPUTE_X if recompute_x else 0) | (FLAG_DEFER_SINKHORN if defer_sinkhorn else 0))


def scale_shape(T: int, C: int, mxfp8) -> tuple:
    """Shape of h_scale: [T, C/32] (linear), or the flat bytes of the MX
    matrix-core operand order, ceil(T/16)*16 * C/32 (mxfp8 == "mfma")."""
    if mxfp8 == "mfma":
        return ((T + 15) // 16 * 16 * (C // 32),)
    return (T, C // 32)


def sinkhorn(coeffs_t, params: Params = Params(), *, stream=None) -> torch.Tensor:
    """mhc_sinkhorn: finish the deferred Sinkhorn of a fused call made with
    ``defer_sinkhorn=True``, in place on coeffs_t [T, 24] (slots 8..23), on
    ``stream`` (a torch.cuda.Stream; default: the current one)."""
    L = lib()
    T = int(coeffs_t.shape[0]) if isinstance(coeffs_t, torch.Tensor) else -1
    _need(coeffs_t, "coeffs", torch.float32, (T, 24))
    st = ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream(coeffs_t.device)).cuda_stream)
    p = MhcParams.of(params)
    _check(L.mhc_sinkhorn(_ptr(coeffs_t), T, ctypes.byref(p), st), "mhc_sinkhorn")
    return coeffs_t


# Placement of the stream outputs the binding allocates: x_out (and the h of
# mhc_pre) starts this many bytes past x modulo 1 KiB, and the fused pass's h
# past y.  A workgroup reads x and writes x_out at the same offsets within
# their rows; with the two buffers equally aligned modulo 1 KiB those reads
# and writes meet in the same memory channels, and the fused pass measured
# 3-4% slower (the splits whose slice sits 256-511 bytes into each KiB fell
# behind the others).  Offsets of 256, 512 and 768 bytes measured within 1%
# of each other.  (A caller of the C functions that allocates its own
# outputs can place them the same way.)
PLACE_OFFSET = 768


def _placed_empty(shape, dtype, dev, ref):
    """An empty tensor whose first byte sits PLACE_OFFSET bytes past ref's
    modulo 1 KiB: a view into a slightly larger allocation."""
    n = 1
    for k in shape:
        n *= k
    if ref is None or not PLACE_OFFSET:
        return torch.empty(shape, dtype=dtype, device=dev)
    es = torch.empty(0, dtype=dtype).element_size()
    big = torch.empty(n + 1024 // es, dtype=dtype, device=dev)
    skip = ((ref.data_ptr() + PLACE_OFFSET - big.data_ptr()) % 1024) // es
    return big[skip: skip + n].view(shape)


def fused_outputs(x, y, *, mxfp8=False, want_h: bool = True) -> dict:
    """The outputs of a fused call on x [T, 4, C] and y [T, C], allocated
    the way the fused functions allocate the ones a caller leaves out: x_out
    and h placed PLACE_OFFSET bytes past x and y modulo 1 KiB.  For callers
    that keep their output buffers across calls."""
    T, C = _dims(x)
    return _fused_outputs(T, C, x.device, mxfp8, want_h, None, x=x, y=y)


def _fused_outputs(T, C, dev, mxfp8, want_h, outs, x=None, y=None):
    # outputs the caller did not pass are allocated here (only those); x_out
    # and h placed relative to x and y (PLACE_OFFSET)
    o = dict(outs or {})

    def need(key, shape, dtype, ref=None):
        if o.get(key) is None:
            o[key] = _placed_empty(shape, dtype, dev, ref)

    need("x_out", (T, 4, C), torch.bfloat16, x)
    need("coeffs_next", (T, 24), torch.float32)
    if want_h:
        need("h", (T, C), torch.bfloat16, y)
    else:
        o["h"] = None
    if mxfp8:
        need("h_fp8", (T, C), torch.uint8)
        need("h_scale", scale_shape(T, C, mxfp8), torch.uint8)
    else:
        o["h_fp8"] = o["h_scale"] = None
    _need(o["x_out"], "x_out", torch.bfloat16, (T, 4, C), dev)
    _need(o["coeffs_next"], "coeffs_next", torch.float32, (T, 24), dev)
    if o["h"] is not None:
        _need(o["h"], "h", torch.bfloat16, (T, C), dev)
    if mxfp8:
        _need(o["h_fp8"], "h_fp8", torch.uint8, (T, C), dev)
        _need(o["h_scale"], "h_scale", torch.uint8, scale_shape(T, C, mxfp8), dev)
    return o


def post_pre_fused(x, y, coeffs_t, phi_next, bias_next, gamma_next, params: Params = Params(), *,
                   mxfp8=False, want_h: bool = True, ws=None, outs=None,
                   recompute_x: bool = False, defer_sinkhorn: bool = False) -> dict:
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(y, "y", torch.bfloat16, (T, C), dev)
    _need(coeffs_t, "coeffs", torch.float32, (T, 24), dev)
    _need(phi_next, "phi_next", torch.float32, (4 * C, 24), dev)
    _need(bias_next, "bias_next", torch.float32, (24,), dev)
    _need(gamma_next, "gamma_next", torch.float32, (C,), dev)
    o = _fused_outputs(T, C, dev, mxfp8, want_h, outs, x=x, y=y)
    ws = workspace(T, C, dev) if ws is None else ws
    p = MhcParams.of(params)
    _check(L.mhc_post_pre_fused(_ptr(x), _ptr(y), _ptr(coeffs_t), _ptr(phi_next), _ptr(bias_next), _ptr(gamma_next),
                                T, C, ctypes.byref(p), _flags(mxfp8, recompute_x, defer_sinkhorn), _ptr(o["x_out"]),
                                _ptr(o["coeffs_next"]), _ptr(o["h"]), _ptr(o["h_fp8"]), _ptr(o["h_scale"]),
                                _ptr(ws), ws.numel(), _stream(dev)), "mhc_post_pre_fused")
    return o


def post_int8_pre_fused(x, y_q, y_scale, coeffs_t, phi_next, bias_next, gamma_next, params: Params = Params(), *,
                        mxfp8=False, want_h: bool = True, ws=None, outs=None, recompute_x: bool = False,
                        phi_packed=None) -> dict:
    """post_pre_fused of an int8 sublayer output y_q [T, C] with per-token
    fp32 scales y_scale [T] (mhc_post_int8_pre_fused, or its _prepacked
    form when ``phi_packed`` is given and ``phi_next`` is None)."""
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(y_q, "y_q", torch.int8, (T, C), dev)
    _need(y_scale, "y_scale", torch.float32, (T,), dev)
    _need(coeffs_t, "coeffs", torch.float32, (T, 24), dev)
    if phi_packed is not None:
        _need(phi_packed, "phi_packed", torch.uint8, (int(L.mhc_phi_packed_bytes(C)),), dev)
        fn, phi_arg, name = L.mhc_post_int8_pre_fused_prepacked, _ptr(phi_packed), "mhc_post_int8_pre_fused_prepacked"
    else:
        _need(phi_next, "phi_next", torch.float32, (4 * C, 24), dev)
        fn, phi_arg, name = L.mhc_post_int8_pre_fused, _ptr(phi_next), "mhc_post_int8_pre_fused"
    _need(bias_next, "bias_next", torch.float32, (24,), dev)
    _need(gamma_next, "gamma_next", torch.float32, (C,), dev)
    o = _fused_outputs(T, C, dev, mxfp8, want_h, outs, x=x, y=y_q)
    ws = workspace(T, C, dev) if ws is None else ws
    p = MhcParams.of(params)
    _check(fn(_ptr(x), _ptr(y_q), _ptr(y_scale), _ptr(coeffs_t), phi_arg, _ptr(bias_next), _ptr(gamma_next), T, C,
              ctypes.byref(p), _flags(mxfp8, recompute_x), _ptr(o["x_out"]), _ptr(o["coeffs_next"]), _ptr(o["h"]),
              _ptr(o["h_fp8"]), _ptr(o["h_scale"]), _ptr(ws), ws.numel(), _stream(dev)), name)
    return o


class Prepared:
    """One library call whose arguments were checked and marshalled once:
    calling it enqueues the same work again, on the stream that was current
    when it was prepared (for a serving loop that would otherwise pay the
    per-call checks).  The tensors it was prepared with must stay alive and
    keep their storage; ``outputs`` holds the output tensors."""

    def __init__(self, fn, args, what, keep, outputs=None):
        self._fn, self._args, self._what, self._keep = fn, args, what, keep
        self.outputs = outputs

    def __call__(self):
        status = self._fn(*self._args)
        if status != 0:
            raise MhcError(status, self._what)
        return self.outputs


def prepare_pack_phi(phi: torch.Tensor, out: torch.Tensor) -> Prepared:
    L = lib()
    C = phi.shape[0] // 4
    _need(phi, "phi", torch.float32, (4 * C, 24))
    _need(out, "phi_packed", torch.uint8, (int(L.mhc_phi_packed_bytes(C)),), phi.device)
    return Prepared(L.mhc_pack_phi, (_ptr(phi), C, _ptr(out), _stream(phi.device)), "mhc_pack_phi", (phi, out), out)


def prepare_post_pre_fused_prepacked(x, y, coeffs_t, phi_next_packed, bias_next, gamma_next,
                                     params: Params = Params(), *, mxfp8=False, want_h: bool = True,
                                     ws=None, outs=None, recompute_x: bool = False,
                                     defer_sinkhorn: bool = False) -> Prepared:
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(y, "y", torch.bfloat16, (T, C), dev)
    _need(coeffs_t, "coeffs", torch.float32, (T, 24), dev)
    _need(phi_next_packed, "phi_next_packed", torch.uint8, (int(L.mhc_phi_packed_bytes(C)),), dev)
    _need(bias_next, "bias_next", torch.float32, (24,), dev)
    _need(gamma_next, "gamma_next", torch.float32, (C,), dev)
    o = _fused_outputs(T, C, dev, mxfp8, want_h, outs, x=x, y=y)
    ws = workspace(T, C, dev) if ws is None else ws
    p = MhcParams.of(params)
    args = (_ptr(x), _ptr(y), _ptr(coeffs_t), _ptr(phi_next_packed), _ptr(bias_next), _ptr(gamma_next), T, C,
            ctypes.byref(p), _flags(mxfp8, recompute_x, defer_sinkhorn), _ptr(o["x_out"]), _ptr(o["coeffs_next"]),
            _ptr(o["h"]), _ptr(o["h_fp8"]), _ptr(o["h_scale"]), _ptr(ws), ws.numel(), _stream(dev))
    keep = (x, y, coeffs_t, phi_next_packed, bias_next, gamma_next, ws, p, o)
    return Prepared(L.mhc_post_pre_fused_prepacked, args, "mhc_post_pre_fused_prepacked", keep, o)


def post_pre_fused_prepacked(x, y, coeffs_t, phi_next_packed, bias_next, gamma_next, params: Params = Params(), *,
                             mxfp8=False, want_h: bool = True, ws=None, outs=None,
                             recompute_x: bool = False, defer_sinkhorn: bool = False) -> dict:
    return prepare_post_pre_fused_prepacked(x, y, coeffs_t, phi_next_packed, bias_next, gamma_next, params,
                                            mxfp8=mxfp8, want_h=want_h, ws=ws, outs=outs,
                                            recompute_x=recompute_x, defer_sinkhorn=defer_sinkhorn)()


def prepare_sinkhorn(coeffs_t, params: Params = Params(), *, stream=None) -> Prepared:
    """mhc_sinkhorn checked and marshalled once (see Prepared)."""
    L = lib()
    T = int(coeffs_t.shape[0]) if isinstance(coeffs_t, torch.Tensor) else -1
    _need(coeffs_t, "coeffs", torch.float32, (T, 24))
    st = ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream(coeffs_t.device)).cuda_stream)
    p = MhcParams.of(params)
    return Prepared(L.mhc_sinkhorn, (_ptr(coeffs_t), T, ctypes.byref(p), st), "mhc_sinkhorn", (coeffs_t, p),
                    coeffs_t)


def post_pre_fused_prepacked_static(x, y, coeffs_t, phi_next_packed, bias_next, gamma_next, params: Params = Params(),
                                    *, error_word, mxfp8=False, want_h: bool = True, outs=None,
                                    recompute_x: bool = False) -> dict:
    """mhc_post_pre_fused_prepacked_static: the fused pass on the library's
    static scratch (no workspace argument).  ``error_word`` is a one-element
    int32 GPU tensor that a bounded wait which expires sets nonzero."""
    L = lib()
    T, C = _dims(x)
    dev = x.device
    _need(x, "x", torch.bfloat16, (T, 4, C))
    _need(y, "y", torch.bfloat16, (T, C), dev)
    _need(coeffs_t, "coeffs", torch.float32, (T, 24), dev)
    _need(phi_next_packed, "phi_next_packed", torch.uint8, (int(L.mhc_phi_packed_bytes(C)),), dev)
    _need(bias_next, "bias_next", torch.float32, (24,), dev)
    _need(gamma_next, "gamma_next", torch.float32, (C,), dev)
    _need(error_word, "error_word", torch.int32, (1,), dev)
    o = _fused_outputs(T, C, dev, mxfp8, want_h, outs, x=x, y=y)
    p = MhcParams.of(params)
    _check(L.mhc_post_pre_fused_prepacked_static(
        _ptr(x), _ptr(y), _ptr(coeffs_t), _ptr(phi_next_packed), _ptr(bias_next), _ptr(gamma_next), T, C,
        ctypes.byref(p), _flags(mxfp8, recompute_x), _ptr(o["x_out"]), _ptr(o["coeffs_next"]), _ptr(o["h"]),
        _ptr(o["h_fp8"]), _ptr(o["h_scale"]), _ptr(error_word), _stream(dev)), "mhc_post_pre_fused_prepacked_static")
    return o
