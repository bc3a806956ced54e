"""RMSNorm and fused residual-Add + RMSNorm on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/addrms.h`` (library
``libaddrms.so`` next to this file).  It only marshals arguments: torch
supplies device memory and the current stream; every step of the computation
runs in the library's HIP kernels.  There is no fallback: if the library is
missing, importing this package raises.  The two latency-bound forwards
(rmsnorm_fwd, add_rmsnorm_fwd) are bound natively (module _native, built
beside the library) when it is built, with the same arguments, checks,
results and errors; rmsnorm_fwd_ctypes and add_rmsnorm_fwd_ctypes stay
available.

Operations (same names as the C ABI):
    rmsnorm_fwd(x, w, eps)            -> y (and rstd)
    add_rmsnorm_fwd(x, r, w, eps)     -> y, residual_out (and rstd)
    rmsnorm_bwd(dy, x, w, rstd)       -> dx, dw
    add_rmsnorm_bwd(dy, dres, h, w, rstd) -> dh (gradient of x and of r), dw
    layernorm_fwd(x, w, b, eps)       -> y (and mean, rstd)
    add_layernorm_fwd(x, r, w, b, eps) -> y, residual_out (and mean, rstd)
    layernorm_bwd(dy, x, w, mean, rstd) -> dx, dw, db
    add_layernorm_bwd(dy, dres, h, w, mean, rstd) -> dh, dw, db
    rmsnorm_fwd_fp8(x, w, eps)        -> y_fp8 (float8_e4m3fn), per-row scale
    add_rmsnorm_fwd_fp8(x, r, w, eps) -> y_fp8, scale, residual_out
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["rmsnorm_fwd", "add_rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_noalloc", "add_rmsnorm_bwd",
           "rmsnorm_bwd_workspace_bytes", "layernorm_fwd", "add_layernorm_fwd", "layernorm_bwd",
           "layernorm_bwd_workspace_bytes", "add_layernorm_bwd", "rmsnorm_fwd_fp8",
           "add_rmsnorm_fwd_fp8", "rmsnorm_fwd_mxfp4", "add_rmsnorm_fwd_mxfp4", "rmsnorm_rope_qk",
           "AddRmsError", "LIB_PATH", "lib", "KNOBS", "set_knob", "tuning", "plan",
           "rmsnorm_fwd_ctypes", "add_rmsnorm_fwd_ctypes"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaddrms.so")

F32, BF16, F16 = 0, 1, 2
_CODES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class AddRmsError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = _lib.addrms_status_str(status).decode()
        if status == -7:
            msg += f" (hipError {_lib.addrms_last_hip_error()})"
        super().__init__(f"{what}: {msg} [{status}]")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python add_rmsnorm_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.rmsnorm_fwd.restype = i32
    lib.rmsnorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.add_rmsnorm_fwd.restype = i32
    lib.add_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.rmsnorm_bwd_workspace_bytes.restype = sz
    lib.rmsnorm_bwd_workspace_bytes.argtypes = [i64, i64]
    lib.rmsnorm_bwd.restype = i32
    lib.rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, i32, vp]
    lib.rmsnorm_bwd_noalloc.restype = i32
    lib.rmsnorm_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, vp]
    lib.add_rmsnorm_bwd.restype = i32
    lib.add_rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, i32, vp]
    lib.rmsnorm_fwd_fp8.restype = i32
    lib.rmsnorm_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.add_rmsnorm_fwd_fp8.restype = i32
    lib.add_rmsnorm_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.layernorm_fwd.restype = i32
    lib.layernorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.add_layernorm_fwd.restype = i32
    lib.add_layernorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.layernorm_bwd_workspace_bytes.restype = sz
    lib.layernorm_bwd_workspace_bytes.argtypes = [i64, i64]
    lib.layernorm_bwd.restype = i32
    lib.layernorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, i32, vp]
    lib.add_layernorm_bwd.restype = i32
    lib.add_layernorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32,
                                      i32, vp]
    lib.rmsnorm_fwd_fp8_grouped.restype = i32
    lib.rmsnorm_fwd_fp8_grouped.argtypes = [vp, vp, vp, vp, i64, vp, i64, i64, f32, i32, i32, vp]
    lib.add_rmsnorm_fwd_fp8_grouped.restype = i32
    lib.add_rmsnorm_fwd_fp8_grouped.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, i64, i64, f32,
                                                i32, i32, vp]
    lib.rmsnorm_fwd_mxfp4.restype = i32
    lib.rmsnorm_fwd_mxfp4.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.add_rmsnorm_fwd_mxfp4.restype = i32
    lib.add_rmsnorm_fwd_mxfp4.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.rmsnorm_rope_qk.restype = i32
    lib.rmsnorm_rope_qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, i64, i64, i64, i64,
                                    i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.addrms_status_str.restype = ctypes.c_char_p
    lib.addrms_status_str.argtypes = [i32]
    lib.addrms_last_hip_error.restype = i32
    lib.addrms_last_hip_error.argtypes = []
    lib.addrms_tune.restype = i32
    lib.addrms_tune.argtypes = [i32, i32]
    lib.addrms_plan.restype = i32
    lib.addrms_plan.argtypes = [i32, i32, i32, i32, i64, i64, i64, i32, i32, i32,
                                ctypes.POINTER(_Plan)]
    return lib


class _Plan(ctypes.Structure):
    """addrms_plan_t of addrms.h."""
    _fields_ = [(n, ctypes.c_int) for n in ("vector", "waves_per_row", "vectors_per_lane",
                                            "prefetch", "wide", "blocks_per_cu")]


_lib = _load()
lib = _lib


# Tuning knobs of the library's dispatcher (ADDRMS_KNOB_* in addrms.h).
KNOBS = {"FWD_WPR": 0, "FWD_VPL": 1, "BWD_WPR": 2, "BWD_WIDE": 3, "BWD_PREFETCH": 4,
         "FORCE_ELEM": 5, "MAX_PARTIALS": 6, "BLOCKS_PER_CU": 7, "ROPE_BLOCKS_PER_CU": 8,
         "ROPE_HPL": 9}


def set_knob(name: str, value: int) -> int:
    """Set a tuning knob of the library (0: the default choice) for the whole
    process and return its previous value."""
    k = KNOBS.get(name.upper().removeprefix("ADDRMS_"))
    if k is None:
        raise KeyError(f"unknown tuning knob {name!r}; known: {sorted(KNOBS)}")
    prev = _lib.addrms_tune(k, int(value))
    if prev < 0:
        raise AddRmsError(prev, "addrms_tune")
    return prev


_QMODES = {None: 0, "fp8": 1, "fp8_group": 2, "mxfp4": 3}


def plan(op: str, M: int, N: int, dtype=torch.bfloat16, w_dtype=None, *, norm: str = "rms",
         fused: bool = True, qmode=None, group: int = 0, cus: int = 256) -> dict:
    """The kernel variant a call would take (addrms_plan in addrms.h): op
    "fwd" or "bwd"; norm "rms" or "layer"; qmode None, "fp8", "fp8_group"
    (with `group` columns per scale) or "mxfp4"; for aligned contiguous
    tensors on a device of `cus` compute units, with the current knobs.
    Returns the fields of addrms_plan_t as a dict.  No GPU needed."""
    if op not in ("fwd", "bwd") or norm not in ("rms", "layer") or qmode not in _QMODES:
        raise ValueError(f"plan: op {op!r}, norm {norm!r}, qmode {qmode!r}")
    out = _Plan()
    rc = _lib.addrms_plan(0 if op == "fwd" else 1, 0 if norm == "rms" else 1, int(fused),
                          _QMODES[qmode], int(group), int(M), int(N), _dtype_code(dtype, "dtype"),
                          _dtype_code(w_dtype or dtype, "w_dtype"), int(cus), ctypes.byref(out))
    if rc != 0:
        raise AddRmsError(rc, "addrms_plan")
    return {n: getattr(out, n) for n, _ in _Plan._fields_}


class tuning:
    """Context manager: `with tuning(BWD_WPR=2, BWD_WIDE=1): ...` sets the
    knobs for its body and restores their previous values after."""

    def __init__(self, **knobs):
        self.knobs = knobs
        self.prev = {}

    def __enter__(self):
        for name, v in self.knobs.items():
            self.prev[name] = set_knob(name, v)
        return self

    def __exit__(self, *exc):
        for name, v in self.prev.items():
            set_knob(name, v)


def _dtype_code(dtype, what: str) -> int:
    c = _CODES.get(dtype)
    if c is None:
        raise TypeError(f"{what}: dtype {dtype} not supported (float32, bfloat16, float16)")
    return c


def _code(t: torch.Tensor, what: str) -> int:
    return _dtype_code(t.dtype, what)


def _dev(t: torch.Tensor, what: str, dtype=None, shape=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _rows(x: torch.Tensor):
    if x.dim() < 1 or x.shape[-1] == 0:
        raise ValueError("input must have a non-empty last dimension")
    N = x.shape[-1]
    return x.numel() // N, N


# The raw handle of the current stream (cheap internal accessor when present).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev: int) -> int:
    if _raw_stream is not None:
        return _raw_stream(dev)
    return torch.cuda.current_stream(dev).cuda_stream


class _OnDevice:
    """Make `dev` current for the call only when it is not already."""
    __slots__ = ("dev", "prev")

    def __init__(self, dev: int):
        self.dev = dev
        self.prev = -1

    def __enter__(self):
        cur = torch.cuda.current_device()
        if cur != self.dev:
            self.prev = cur
            torch.cuda.set_device(self.dev)

    def __exit__(self, *exc):
        if self.prev >= 0:
            torch.cuda.set_device(self.prev)


def _p(t):
    return t.data_ptr() if t is not None else None


_get_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device


def _ok(t, dtype, shape) -> bool:
    """The checks of _dev in one expression (the per-call fast path of the
    latency-bound forwards); on False the caller runs _dev for the message."""
    return t.is_cuda and t.dtype == dtype and t.shape == shape and t.is_contiguous()


def _call(dev: int, fn, *args) -> int:
    """fn(*args) with `dev` the current device (switched only when needed)."""
    cur = _get_device()
    if cur == dev:
        return fn(*args)
    torch.cuda.set_device(dev)
    try:
        return fn(*args)
    finally:
        torch.cuda.set_device(cur)


def rmsnorm_fwd(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, *, y=None, rstd=None,
                return_rstd: bool = False):
    """y = x / sqrt(mean(x^2, -1) + eps) * w, normalising the last dimension.
    `y` may be `x` (in place).  Returns y, or (y, rstd) with float32 rstd."""
    _dev(x, "x")
    M, N = _rows(x)
    if not _ok(w, w.dtype, (N,)):
        _dev(w, "w", shape=(N,))
    if y is None:
        y = torch.empty_like(x)
    elif not _ok(y, x.dtype, x.shape):
        _dev(y, "y", x.dtype, x.shape)
    if rstd is None and return_rstd:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    elif rstd is not None:
        _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dev = x.get_device()
    st = _call(dev, _lib.rmsnorm_fwd, x.data_ptr(), w.data_ptr(), y.data_ptr(), _p(rstd), M, N,
               float(eps), _code(x, "x"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "rmsnorm_fwd")
    return (y, rstd) if (return_rstd or rstd is not None) else y


def add_rmsnorm_fwd(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, *,
                    y=None, residual_out=None, rstd=None, return_rstd: bool = False):
    """residual_out = x + r (float32 add, stored in x's dtype);
    y = residual_out / sqrt(mean(residual_out^2, -1) + eps) * w.
    `residual_out` may be `r` or `x` (in-place residual update), `y` may be
    `x` or `r`.  Returns (y, residual_out) or (y, residual_out, rstd)."""
    _dev(x, "x")
    M, N = _rows(x)
    dt, shp = x.dtype, x.shape
    if not _ok(r, dt, shp):
        _dev(r, "r", dt, shp)
    if not _ok(w, w.dtype, (N,)):
        _dev(w, "w", shape=(N,))
    if y is None:
        y = torch.empty_like(x)
    elif not _ok(y, dt, shp):
        _dev(y, "y", dt, shp)
    if residual_out is None:
        residual_out = torch.empty_like(x)
    elif not _ok(residual_out, dt, shp):
        _dev(residual_out, "residual_out", dt, shp)
    if rstd is None and return_rstd:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    elif rstd is not None:
        _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dev = x.get_device()
    st = _call(dev, _lib.add_rmsnorm_fwd, x.data_ptr(), r.data_ptr(), w.data_ptr(), y.data_ptr(),
               residual_out.data_ptr(), _p(rstd), M, N, float(eps), _code(x, "x"), _code(w, "w"),
               _stream(dev))
    if st != 0:
        raise AddRmsError(st, "add_rmsnorm_fwd")
    if return_rstd or rstd is not None:
        return y, residual_out, rstd
    return y, residual_out


def rmsnorm_bwd_workspace_bytes(M: int, N: int) -> int:
    """Device scratch bytes rmsnorm_bwd needs for M rows of N."""
    return int(_lib.rmsnorm_bwd_workspace_bytes(M, N))


_ws_cache: dict = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A per-device scratch buffer, grown on demand and reused across calls on
    the current stream (calls on other streams must pass their own).  Under
    graph capture every call gets its own buffer from the capture's memory
    pool instead: a replay then writes only memory the graph owns, and the
    cache is left alone (replacing a cached buffer would free memory that a
    captured graph still writes)."""
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    key = (device.index, _stream(device.index))
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def rmsnorm_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor, *,
                dx=None, dw=None, workspace: torch.Tensor | None = None):
    """Gradients of y = x * rstd * w given dy and the forward's saved float32
    rstd: returns (dx, dw) with dw float32.  `dx` may be `dy` or `x`."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(dy, "dy", x.dtype, x.shape)
    _dev(w, "w", shape=(N,))
    _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dx = torch.empty_like(x) if dx is None else _dev(dx, "dx", x.dtype, x.shape)
    dw = (torch.empty(N, dtype=torch.float32, device=x.device) if dw is None
          else _dev(dw, "dw", torch.float32, (N,)))
    need = rmsnorm_bwd_workspace_bytes(M, N)
    if workspace is None:
        workspace = _workspace(x.device, need)
    else:
        _dev(workspace, "workspace")
    dev = x.get_device()
    with _OnDevice(dev):
        st = _lib.rmsnorm_bwd(_p(dy), _p(x), _p(w), _p(rstd), _p(dx), _p(dw), _p(workspace),
                              workspace.numel() * workspace.element_size(), M, N,
                              _code(x, "x"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "rmsnorm_bwd")
    return dx, dw


def rmsnorm_bwd_noalloc(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor,
                        *, dx=None, dw=None):
    """rmsnorm_bwd without a workspace: the library keeps the dw partial sums
    in a fixed device scratch of its own (16 MiB per GPU), so the library call
    allocates nothing (pass dx and dw to allocate nothing at all).  Calls that
    may overlap on one GPU share that scratch and must be serialised.
    Returns (dx, dw)."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(dy, "dy", x.dtype, x.shape)
    _dev(w, "w", shape=(N,))
    _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dx = torch.empty_like(x) if dx is None else _dev(dx, "dx", x.dtype, x.shape)
    dw = (torch.empty(N, dtype=torch.float32, device=x.device) if dw is None
          else _dev(dw, "dw", torch.float32, (N,)))
    dev = x.get_device()
    with _OnDevice(dev):
        st = _lib.rmsnorm_bwd_noalloc(_p(dy), _p(x), _p(w), _p(rstd), _p(dx), _p(dw), M, N,
                                      _code(x, "x"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "rmsnorm_bwd_noalloc")
    return dx, dw


def add_rmsnorm_bwd(dy: torch.Tensor, dres, h: torch.Tensor, w: torch.Tensor,
                    rstd: torch.Tensor, *, dh=None, dw=None,
                    workspace: torch.Tensor | None = None):
    """Backward of add_rmsnorm_fwd: from the gradients of y (dy) and of
    residual_out (dres, or None for zero), the saved residual_out h and rstd,
    returns (dh, dw): dh is the gradient of both x and r.  `dh` may be `dy`,
    `dres` or `h`."""
    _dev(h, "h")
    M, N = _rows(h)
    _dev(dy, "dy", h.dtype, h.shape)
    if dres is not None:
        _dev(dres, "dres", h.dtype, h.shape)
    _dev(w, "w", shape=(N,))
    _dev(rstd, "rstd", torch.float32, h.shape[:-1])
    dh = torch.empty_like(h) if dh is None else _dev(dh, "dh", h.dtype, h.shape)
    dw = (torch.empty(N, dtype=torch.float32, device=h.device) if dw is None
          else _dev(dw, "dw", torch.float32, (N,)))
    need = rmsnorm_bwd_workspace_bytes(M, N)
    if workspace is None:
        workspace = _workspace(h.device, need)
    else:
        _dev(workspace, "workspace")
    dev = h.get_device()
    with _OnDevice(dev):
        st = _lib.add_rmsnorm_bwd(_p(dy), _p(dres), _p(h), _p(w), _p(rstd), _p(dh), _p(dw),
                                  _p(workspace), workspace.numel() * workspace.element_size(),
                                  M, N, _code(h, "h"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "add_rmsnorm_bwd")
    return dh, dw


def _stats(x, mean, rstd, want):
    if want:
        mean = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if mean is None else mean
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if rstd is None else rstd
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        if t is not None:
            _dev(t, n, torch.float32, x.shape[:-1])
    return mean, rstd


def layernorm_fwd(x: torch.Tensor, w: torch.Tensor, b=None, eps: float = 1e-5, *, y=None,
                  mean=None, rstd=None, return_stats: bool = False):
    """y = (x - mean) / sqrt(var + eps) * w (+ b) over the last dimension.
    Returns y, or (y, mean, rstd) with float32 statistics."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(w, "w", shape=(N,))
    if b is not None:
        _dev(b, "b", w.dtype, (N,))
    y = torch.empty_like(x) if y is None else _dev(y, "y", x.dtype, x.shape)
    mean, rstd = _stats(x, mean, rstd, return_stats)
    dev = x.get_device()
    with _OnDevice(dev):
        st = _lib.layernorm_fwd(_p(x), _p(w), _p(b), _p(y), _p(mean), _p(rstd), M, N, float(eps),
                                _code(x, "x"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "layernorm_fwd")
    return (y, mean, rstd) if (return_stats or rstd is not None) else y


def add_layernorm_fwd(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor, b=None,
                      eps: float = 1e-5, *, y=None, residual_out=None, mean=None, rstd=None,
                      return_stats: bool = False):
    """residual_out = x + r (float32 add, stored in x's dtype);
    y = LayerNorm(residual_out) * w (+ b).  Returns (y, residual_out) or
    (y, residual_out, mean, rstd)."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(r, "r", x.dtype, x.shape)
    _dev(w, "w", shape=(N,))
    if b is not None:
        _dev(b, "b", w.dtype, (N,))
    y = torch.empty_like(x) if y is None else _dev(y, "y", x.dtype, x.shape)
    residual_out = (torch.empty_like(x) if residual_out is None
                    else _dev(residual_out, "residual_out", x.dtype, x.shape))
    mean, rstd = _stats(x, mean, rstd, return_stats)
    dev = x.get_device()
    with _OnDevice(dev):
        st = _lib.add_layernorm_fwd(_p(x), _p(r), _p(w), _p(b), _p(y), _p(residual_out),
                                    _p(mean), _p(rstd), M, N, float(eps), _code(x, "x"),
                                    _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "add_layernorm_fwd")
    if return_stats or rstd is not None:
        return y, residual_out, mean, rstd
    return y, residual_out


def layernorm_bwd_workspace_bytes(M: int, N: int) -> int:
    """Device scratch bytes layernorm_bwd needs for M rows of N."""
    return int(_lib.layernorm_bwd_workspace_bytes(M, N))


def layernorm_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, mean: torch.Tensor,
                  rstd: torch.Tensor, *, dx=None, dw=None, db=None, with_db: bool = True,
                  workspace: torch.Tensor | None = None):
    """Gradients of LayerNorm from the saved float32 mean and rstd: returns
    (dx, dw, db) with dw and db float32 (db None when with_db is False and no
    db buffer is given).  `dx` may be `dy` or `x`."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(dy, "dy", x.dtype, x.shape)
    _dev(w, "w", shape=(N,))
    _dev(mean, "mean", torch.float32, x.shape[:-1])
    _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dx = torch.empty_like(x) if dx is None else _dev(dx, "dx", x.dtype, x.shape)
    dw = (torch.empty(N, dtype=torch.float32, device=x.device) if dw is None
          else _dev(dw, "dw", torch.float32, (N,)))
    if db is None and with_db:
        db = torch.empty(N, dtype=torch.float32, device=x.device)
    elif db is not None:
        _dev(db, "db", torch.float32, (N,))
    need = layernorm_bwd_workspace_bytes(M, N)
    if workspace is None:
        workspace = _workspace(x.device, need)
    else:
        _dev(workspace, "workspace")
    dev = x.get_device()
    with _OnDevice(dev):
        st = _lib.layernorm_bwd(_p(dy), _p(x), _p(w), _p(mean), _p(rstd), _p(dx), _p(dw), _p(db),
                                _p(workspace), workspace.numel() * workspace.element_size(), M,
                                N, _code(x, "x"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "layernorm_bwd")
    return dx, dw, db


def add_layernorm_bwd(dy: torch.Tensor, dres, h: torch.Tensor, w: torch.Tensor,
                      mean: torch.Tensor, rstd: torch.Tensor, *, dh=None, dw=None, db=None,
                      with_db: bool = True, workspace: torch.Tensor | None = None):
    """Backward of add_layernorm_fwd: from dy, the residual_out gradient dres
    (None for zero), the saved residual_out h, mean and rstd, returns
    (dh, dw, db); dh is the gradient of both x and r."""
    _dev(h, "h")
    M, N = _rows(h)
    _dev(dy, "dy", h.dtype, h.shape)
    if dres is not None:
        _dev(dres, "dres", h.dtype, h.shape)
    _dev(w, "w", shape=(N,))
    _dev(mean, "mean", torch.float32, h.shape[:-1])
    _dev(rstd, "rstd", torch.float32, h.shape[:-1])
    dh = torch.empty_like(h) if dh is None else _dev(dh, "dh", h.dtype, h.shape)
    dw = (torch.empty(N, dtype=torch.float32, device=h.device) if dw is None
          else _dev(dw, "dw", torch.float32, (N,)))
    if db is None and with_db:
        db = torch.empty(N, dtype=torch.float32, device=h.device)
    elif db is not None:
        _dev(db, "db", torch.float32, (N,))
    need = layernorm_bwd_workspace_bytes(M, N)
    if workspace is None:
        workspace = _workspace(h.device, need)
    else:
        _dev(workspace, "workspace")
    dev = h.get_device()
    with _OnDevice(dev):
        st = _lib.add_layernorm_bwd(_p(dy), _p(dres), _p(h), _p(w), _p(mean), _p(rstd), _p(dh),
                                    _p(dw), _p(db), _p(workspace),
                                    workspace.numel() * workspace.element_size(), M, N,
                                    _code(h, "h"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "add_layernorm_bwd")
    return dh, dw, db


_FP8 = getattr(torch, "float8_e4m3fn", None)


def _fp8_out(x, y_fp8, y_scale, group=None):
    """Output buffers of the FP8 variants: codes like x; scales [..] (one per
    row) or, with a group, [.., ceil(N / group)]."""
    N = x.shape[-1]
    sshape = x.shape[:-1] if group is None else x.shape[:-1] + ((N + min(group, N) - 1) //
                                                                min(group, N),)
    if y_fp8 is None:
        y_fp8 = torch.empty(x.shape, dtype=_FP8 if _FP8 is not None else torch.uint8,
                            device=x.device)
    else:
        _dev(y_fp8, "y_fp8", shape=x.shape)
        if y_fp8.element_size() != 1:
            raise TypeError("y_fp8 must have 1-byte elements (float8_e4m3fn or uint8)")
    if y_scale is None:
        y_scale = torch.empty(sshape, dtype=torch.float32, device=x.device)
    else:
        _dev(y_scale, "y_scale", torch.float32, sshape)
    return y_fp8, y_scale


def _group(group):
    if group is None:
        return None
    g = int(group)
    if g < 1:
        raise ValueError(f"group must be >= 1, got {group}")
    return g


def rmsnorm_fwd_fp8(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, *, group=None,
                    y_fp8=None, y_scale=None, rstd=None):
    """RMSNorm with an OCP E4M3 output (torch.float8_e4m3fn) and dynamic
    float32 scales: one per row (y ~= y_fp8.float() * y_scale[..., None]) or,
    with group=G, one per G consecutive columns (y_scale [..., ceil(N/G)]).
    Returns (y_fp8, y_scale)."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(w, "w", shape=(N,))
    g = _group(group)
    y_fp8, y_scale = _fp8_out(x, y_fp8, y_scale, g)
    if rstd is not None:
        _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dev = x.get_device()
    with _OnDevice(dev):
        if g is None:
            st = _lib.rmsnorm_fwd_fp8(_p(x), _p(w), _p(y_fp8), _p(y_scale), _p(rstd), M, N,
                                      float(eps), _code(x, "x"), _code(w, "w"), _stream(dev))
        else:
            st = _lib.rmsnorm_fwd_fp8_grouped(_p(x), _p(w), _p(y_fp8), _p(y_scale), g, _p(rstd),
                                              M, N, float(eps), _code(x, "x"), _code(w, "w"),
                                              _stream(dev))
    if st != 0:
        raise AddRmsError(st, "rmsnorm_fwd_fp8")
    return y_fp8, y_scale


def add_rmsnorm_fwd_fp8(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                        *, group=None, y_fp8=None, y_scale=None, residual_out=None, rstd=None):
    """Fused residual add + RMSNorm with an E4M3 output and dynamic scales (per
    row, or per `group` columns as rmsnorm_fwd_fp8).
    Returns (y_fp8, y_scale, residual_out)."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(r, "r", x.dtype, x.shape)
    _dev(w, "w", shape=(N,))
    g = _group(group)
    y_fp8, y_scale = _fp8_out(x, y_fp8, y_scale, g)
    residual_out = (torch.empty_like(x) if residual_out is None
                    else _dev(residual_out, "residual_out", x.dtype, x.shape))
    if rstd is not None:
        _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dev = x.get_device()
    with _OnDevice(dev):
        if g is None:
            st = _lib.add_rmsnorm_fwd_fp8(_p(x), _p(r), _p(w), _p(y_fp8), _p(y_scale),
                                          _p(residual_out), _p(rstd), M, N, float(eps),
                                          _code(x, "x"), _code(w, "w"), _stream(dev))
        else:
            st = _lib.add_rmsnorm_fwd_fp8_grouped(_p(x), _p(r), _p(w), _p(y_fp8), _p(y_scale), g,
                                                  _p(residual_out), _p(rstd), M, N, float(eps),
                                                  _code(x, "x"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "add_rmsnorm_fwd_fp8")
    return y_fp8, y_scale, residual_out


_FP4X2 = getattr(torch, "float4_e2m1fn_x2", None)
_E8M0 = getattr(torch, "float8_e8m0fnu", None)


def _mx_out(x, y_fp4, y_scale):
    """MXFP4 output buffers: codes [.., N/2] (two per byte), E8M0 scales
    [.., ceil(N/32)]; 1-byte element types (packed FP4 / E8M0, or uint8)."""
    N = x.shape[-1]
    if N % 2:
        raise ValueError(f"MXFP4 needs an even last dimension, got {N}")
    cshape = x.shape[:-1] + (N // 2,)
    sshape = x.shape[:-1] + ((N + 31) // 32,)
    if y_fp4 is None:
        y_fp4 = torch.empty(cshape, dtype=_FP4X2 or torch.uint8, device=x.device)
    else:
        _dev(y_fp4, "y_fp4", shape=cshape)
    if y_scale is None:
        y_scale = torch.empty(sshape, dtype=_E8M0 or torch.uint8, device=x.device)
    else:
        _dev(y_scale, "y_scale", shape=sshape)
    for t, n in ((y_fp4, "y_fp4"), (y_scale, "y_scale")):
        if t.element_size() != 1:
            raise TypeError(f"{n} must have 1-byte elements")
    return y_fp4, y_scale


def rmsnorm_fwd_mxfp4(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, *, y_fp4=None,
                      y_scale=None, rstd=None):
    """RMSNorm with an MXFP4 output (OCP MX): E2M1 codes two per byte
    (torch.float4_e2m1fn_x2 [.., N/2], element 2i in the low nibble) and one
    E8M0 scale per 32 values (torch.float8_e8m0fnu [.., ceil(N/32)]):
    y ~= E2M1(code) * 2^(scale - 127).  Returns (y_fp4, y_scale)."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(w, "w", shape=(N,))
    y_fp4, y_scale = _mx_out(x, y_fp4, y_scale)
    if rstd is not None:
        _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dev = x.get_device()
    with _OnDevice(dev):
        st = _lib.rmsnorm_fwd_mxfp4(_p(x), _p(w), _p(y_fp4), _p(y_scale), _p(rstd), M, N,
                                    float(eps), _code(x, "x"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "rmsnorm_fwd_mxfp4")
    return y_fp4, y_scale


def add_rmsnorm_fwd_mxfp4(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                          *, y_fp4=None, y_scale=None, residual_out=None, rstd=None):
    """Fused residual add + RMSNorm with an MXFP4 output, as rmsnorm_fwd_mxfp4.
    Returns (y_fp4, y_scale, residual_out)."""
    _dev(x, "x")
    M, N = _rows(x)
    _dev(r, "r", x.dtype, x.shape)
    _dev(w, "w", shape=(N,))
    y_fp4, y_scale = _mx_out(x, y_fp4, y_scale)
    residual_out = (torch.empty_like(x) if residual_out is None
                    else _dev(residual_out, "residual_out", x.dtype, x.shape))
    if rstd is not None:
        _dev(rstd, "rstd", torch.float32, x.shape[:-1])
    dev = x.get_device()
    with _OnDevice(dev):
        st = _lib.add_rmsnorm_fwd_mxfp4(_p(x), _p(r), _p(w), _p(y_fp4), _p(y_scale),
                                        _p(residual_out), _p(rstd), M, N, float(eps),
                                        _code(x, "x"), _code(w, "w"), _stream(dev))
    if st != 0:
        raise AddRmsError(st, "add_rmsnorm_fwd_mxfp4")
    return y_fp4, y_scale, residual_out


def _heads(t: torch.Tensor, what: str, dtype=None, T=None, D=None) -> int:
    """Check a [T, H, D] GPU tensor whose heads of one token are contiguous
    (any token stride, e.g. a view into a packed projection output) and
    return its token stride in elements."""
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if t.dim() != 3:
        raise ValueError(f"{what} must be [T, H, D], got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    Tt, H, Dd = t.shape
    if (T is not None and Tt != T) or (D is not None and Dd != D):
        raise ValueError(f"{what}: shape {tuple(t.shape)} does not match T={T}, D={D}")
    if Dd > 0 and (t.stride(2) != 1 or (H > 1 and t.stride(1) != Dd)):
        raise ValueError(f"{what}: the heads of one token must be contiguous")
    return t.stride(0) if Tt > 1 else H * Dd


def rmsnorm_rope_qk(q: torch.Tensor, k, wq: torch.Tensor, wk, cos: torch.Tensor,
                    sin: torch.Tensor, pos: torch.Tensor, eps: float = 1e-6, *,
                    interleaved: bool = False, q_out=None, k_out=None):
    """Per-head RMSNorm (weights wq, wk [D]) then RoPE at each token's
    position, for query heads q [T, Hq, D] and key heads k [T, Hk, D] (k may
    be None).  q and k may be views with any token stride.  cos, sin: float32
    [P, D/2]; pos: int64 [T].  interleaved selects pairs (2i, 2i+1) instead of
    (i, i + D/2).  q_out=q, k_out=k update in place (e.g. a packed qkv
    buffer).  Returns (q_out, k_out); a position outside [0, P) gives NaN
    heads."""
    T, Hq, D = q.shape if q.dim() == 3 else (None, None, None)
    qs = _heads(q, "q")
    Hk, ks = 0, 0
    if k is not None:
        ks = _heads(k, "k", q.dtype, T, D)
        Hk = k.shape[1]
    _dev(wq, "wq", shape=(D,))
    if k is not None:
        if wk is None:
            raise ValueError("wk is required with k")
        _dev(wk, "wk", wq.dtype, (D,))
    _dev(cos, "cos", torch.float32)
    if cos.dim() != 2 or cos.shape[1] != D // 2:
        raise ValueError(f"cos must be [P, D/2], got {tuple(cos.shape)}")
    _dev(sin, "sin", torch.float32, cos.shape)
    _dev(pos, "pos", torch.int64, (T,))
    q_out = torch.empty((T, Hq, D), dtype=q.dtype, device=q.device) if q_out is None else q_out
    qos = _heads(q_out, "q_out", q.dtype, T, D)
    kos = 0
    if k is not None:
        k_out = torch.empty((T, Hk, D), dtype=q.dtype, device=q.device) if k_out is None else k_out
        kos = _heads(k_out, "k_out", q.dtype, T, D)
    dev = q.get_device()
    with _OnDevice(dev):
        st = _lib.rmsnorm_rope_qk(_p(q), _p(k), _p(wq), _p(wk) if k is not None else None,
                                  _p(cos), _p(sin), _p(pos), cos.shape[0], _p(q_out), _p(k_out),
                                  T, Hq, Hk, D, qs, ks, qos, kos, float(eps),
                                  1 if interleaved else 0, _code(q, "q"), _code(wq, "wq"),
                                  _stream(dev))
    if st != 0:
        raise AddRmsError(st, "rmsnorm_rope_qk")
    return q_out, k_out


# The native binding of the latency-bound forwards (csrc/binding.cpp, built
# beside the library as _native*.so): the same arguments, checks and results
# as rmsnorm_fwd and add_rmsnorm_fwd above, with the tensor checks in C++
# (at decode sizes the call is launch-bound and the Python checks cost about
# as much as the launch).  When it is built it replaces them; if it is built
# but cannot load, the import fails.  The ctypes versions stay available as
# rmsnorm_fwd_ctypes and add_rmsnorm_fwd_ctypes.
rmsnorm_fwd_ctypes, add_rmsnorm_fwd_ctypes = rmsnorm_fwd, add_rmsnorm_fwd
native = None
if any(f.startswith("_native") and f.endswith(".so")
       for f in os.listdir(os.path.dirname(os.path.abspath(__file__)))):
    import importlib
    native = importlib.import_module(__name__ + "._native")
    rmsnorm_fwd = native.rmsnorm_fwd
    add_rmsnorm_fwd = native.add_rmsnorm_fwd
