"""CPU oracle for RMSNorm / fused residual-Add + RMSNorm (forward, backward).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import this module.  The GPU library never
loads it.

The arithmetic lives in ``addrms_oracle.c`` (plain C, binary64, one rounding
per output); this module only marshals torch CPU tensors into it.  The
definitions it follows are stated in that file's header: the operations are
the RMSNorm op of the "Machete" README ("Built-In Areas") and the fused
Add + RMSNorm of KernelAgent-Oink (KernelAgent repository digest, opening
summary), with the textbook RMSNorm formula.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "addrms_oracle.c")
# A test may point the wrapper at another build of the oracle source (the
# mutation test builds deliberately broken copies to show the pins catch them).
_LIB_PATH = os.environ.get("ADDRMS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32, BF16, F64, F16 = 0, 1, 2, 3
_CODES = {torch.float32: F32, torch.bfloat16: BF16, torch.float64: F64, torch.float16: F16}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: no fast-math, no FMA contraction, so that
    every operation is the IEEE operation written in the source."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Werror", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_bf16_round.argtypes = [dbl]
        lib.oracle_bf16_round_array.restype = None
        lib.oracle_bf16_round_array.argtypes = [vp, vp, i64]
        lib.oracle_f16_round.restype = ctypes.c_uint16
        lib.oracle_f16_round.argtypes = [dbl]
        lib.oracle_f16_round_array.restype = None
        lib.oracle_f16_round_array.argtypes = [vp, vp, i64]
        lib.oracle_f16_decode_array.restype = None
        lib.oracle_f16_decode_array.argtypes = [vp, vp, i64]
        lib.oracle_rmsnorm_fwd.restype = i32
        lib.oracle_rmsnorm_fwd.argtypes = [vp, i32, vp, i32, vp, i32, vp, i32, i64, i64, dbl]
        lib.oracle_add_rmsnorm_fwd.restype = i32
        lib.oracle_add_rmsnorm_fwd.argtypes = [vp, vp, i32, vp, i32, vp, i32, vp, i32, vp, i32,
                                               i64, i64, dbl]
        lib.oracle_rmsnorm_bwd.restype = i32
        lib.oracle_rmsnorm_bwd.argtypes = [vp, vp, i32, vp, i32, vp, i32, vp, i32, vp, i32, vp,
                                           i64, i64]
        lib.oracle_layernorm_fwd.restype = i32
        lib.oracle_layernorm_fwd.argtypes = [vp, i32, vp, vp, i32, vp, i32, vp, vp, i32, i64,
                                             i64, dbl]
        lib.oracle_add_layernorm_fwd.restype = i32
        lib.oracle_add_layernorm_fwd.argtypes = [vp, vp, i32, vp, vp, i32, vp, i32, vp, i32, vp,
                                                 vp, i32, i64, i64, dbl]
        lib.oracle_add_layernorm_bwd.restype = i32
        lib.oracle_add_layernorm_bwd.argtypes = [vp, vp, vp, i32, vp, i32, vp, vp, i32, vp, i32,
                                                 vp, vp, i32, vp, vp, i64, i64]
        lib.oracle_layernorm_bwd.restype = i32
        lib.oracle_layernorm_bwd.argtypes = [vp, vp, i32, vp, i32, vp, vp, i32, vp, i32, vp, vp,
                                             i32, vp, vp, i64, i64]
        lib.oracle_fp8e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_fp8e4m3_encode.argtypes = [dbl]
        lib.oracle_fp8e4m3_decode.restype = dbl
        lib.oracle_fp8e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8e4m3_encode_array.restype = None
        lib.oracle_fp8e4m3_encode_array.argtypes = [vp, vp, i64]
        lib.oracle_rmsnorm_fwd_fp8.restype = i32
        lib.oracle_rmsnorm_fwd_fp8.argtypes = [vp, i32, vp, i32, vp, vp, vp, i32, i64, i64, dbl]
        lib.oracle_add_rmsnorm_fwd_fp8.restype = i32
        lib.oracle_add_rmsnorm_fwd_fp8.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, i32, vp, i32,
                                                   i64, i64, dbl]
        lib.oracle_add_rmsnorm_bwd.restype = i32
        lib.oracle_add_rmsnorm_bwd.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, vp, i32, vp,
                                               i32, vp, i64, i64]
        lib.oracle_rmsnorm_fwd_fp8_grouped.restype = i32
        lib.oracle_rmsnorm_fwd_fp8_grouped.argtypes = [vp, i32, vp, i32, vp, vp, i64, vp, i32, i64,
                                                       i64, dbl]
        lib.oracle_add_rmsnorm_fwd_fp8_grouped.restype = i32
        lib.oracle_add_rmsnorm_fwd_fp8_grouped.argtypes = [vp, vp, i32, vp, i32, vp, vp, i64, vp,
                                                           i32, vp, i32, i64, i64, dbl]
        lib.oracle_fp4e2m1_encode.restype = ctypes.c_uint8
        lib.oracle_fp4e2m1_encode.argtypes = [dbl]
        lib.oracle_fp4e2m1_decode.restype = dbl
        lib.oracle_fp4e2m1_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_fp4e2m1_encode_array.restype = None
        lib.oracle_fp4e2m1_encode_array.argtypes = [vp, vp, i64]
        lib.oracle_rmsnorm_fwd_mxfp4.restype = i32
        lib.oracle_rmsnorm_fwd_mxfp4.argtypes = [vp, i32, vp, i32, vp, vp, vp, i32, i64, i64, dbl]
        lib.oracle_add_rmsnorm_fwd_mxfp4.restype = i32
        lib.oracle_add_rmsnorm_fwd_mxfp4.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, i32, vp, i32,
                                                     i64, i64, dbl]
        lib.oracle_rmsnorm_rope.restype = i32
        lib.oracle_rmsnorm_rope.argtypes = [vp, i32, i64, vp, i32, vp, vp, vp, i64, vp, i32, i64,
                                            i64, i64, i64, i32, dbl]
        _lib = lib
    return _lib


def _code(t: torch.Tensor) -> int:
    if t.dtype not in _CODES:
        raise TypeError(f"oracle: unsupported dtype {t.dtype}")
    return _CODES[t.dtype]


def _cpu(t: torch.Tensor) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError("oracle: CPU tensors only")
    return t.contiguous()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def eps_as_float32(eps: float) -> float:
    """The eps value the GPU library sees: the binary32 nearest to eps."""
    return float(np.float32(eps))


def f16_round(v) -> np.ndarray:
    """binary64 values -> IEEE binary16 bit patterns (uint16), one RNE rounding."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_f16_round_array(a.ctypes.data, out.ctypes.data, a.size)
    return out


def f16_decode(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> their exact binary64 values."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_f16_decode_array(b.ctypes.data, out.ctypes.data, b.size)
    return out


def bf16_round(v) -> np.ndarray:
    """binary64 values -> bfloat16 bit patterns (uint16), one RNE rounding."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_bf16_round_array(a.ctypes.data, out.ctypes.data, a.size)
    return out


def rmsnorm_fwd(x: torch.Tensor, w: torch.Tensor, eps: float, *, y_dtype=None,
                rstd_dtype=torch.float32, eps_exact: bool = False):
    """y = x * rstd * w over the last dim; returns (y, rstd).  By default eps is
    first rounded to binary32, as the library's float argument is."""
    x, w = _cpu(x), _cpu(w)
    N = x.shape[-1]
    M = x.numel() // N
    y = torch.empty(x.shape, dtype=y_dtype or x.dtype)
    rstd = torch.empty(x.shape[:-1], dtype=rstd_dtype)
    e = float(eps) if eps_exact else eps_as_float32(eps)
    _check(_load().oracle_rmsnorm_fwd(_ptr(x), _code(x), _ptr(w), _code(w), _ptr(y), _code(y),
                                      _ptr(rstd), _code(rstd), M, N, e), "rmsnorm_fwd")
    return y, rstd


def add_rmsnorm_fwd(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor, eps: float, *,
                    y_dtype=None, res_dtype=None, rstd_dtype=torch.float32,
                    eps_exact: bool = False):
    """residual_out = stored(x + r); y = RMSNorm(residual_out) * w.
    Returns (y, residual_out, rstd)."""
    x, r, w = _cpu(x), _cpu(r), _cpu(w)
    if x.dtype != r.dtype or x.shape != r.shape:
        raise ValueError("oracle: x and r must share dtype and shape")
    N = x.shape[-1]
    M = x.numel() // N
    y = torch.empty(x.shape, dtype=y_dtype or x.dtype)
    res = torch.empty(x.shape, dtype=res_dtype or x.dtype)
    rstd = torch.empty(x.shape[:-1], dtype=rstd_dtype)
    e = float(eps) if eps_exact else eps_as_float32(eps)
    _check(_load().oracle_add_rmsnorm_fwd(_ptr(x), _ptr(r), _code(x), _ptr(w), _code(w),
                                          _ptr(y), _code(y), _ptr(res), _code(res),
                                          _ptr(rstd), _code(rstd), M, N, e), "add_rmsnorm_fwd")
    return y, res, rstd


def rmsnorm_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor, *,
                dx_dtype=None, dw_dtype=torch.float32):
    """dx, dw from the saved rstd.  Returns (dx, dw, dw_abs) where dw_abs[j] is
    sum_i |dy_ij * x_ij * rstd_i| in binary64."""
    dy, x, w, rstd = _cpu(dy), _cpu(x), _cpu(w), _cpu(rstd)
    if dy.dtype != x.dtype or dy.shape != x.shape:
        raise ValueError("oracle: dy and x must share dtype and shape")
    N = x.shape[-1]
    M = x.numel() // N
    dx = torch.empty(x.shape, dtype=dx_dtype or x.dtype)
    dw = torch.empty((N,), dtype=dw_dtype)
    dw_abs = torch.empty((N,), dtype=torch.float64)
    _check(_load().oracle_rmsnorm_bwd(_ptr(dy), _ptr(x), _code(x), _ptr(w), _code(w),
                                      _ptr(rstd), _code(rstd), _ptr(dx), _code(dx), _ptr(dw),
                                      _code(dw), _ptr(dw_abs), M, N), "rmsnorm_bwd")
    return dx, dw, dw_abs


def add_rmsnorm_bwd(dy: torch.Tensor, dres, h: torch.Tensor, w: torch.Tensor,
                    rstd: torch.Tensor, *, dh_dtype=None, dw_dtype=torch.float32):
    """Backward of the fused op: dh (the gradient of x and of r) and dw, from
    the gradients of y (dy) and of residual_out (dres, None for zero), the
    saved residual h and rstd.  Returns (dh, dw, dw_abs)."""
    dy, h, w, rstd = _cpu(dy), _cpu(h), _cpu(w), _cpu(rstd)
    if dres is not None:
        dres = _cpu(dres)
        if dres.dtype != h.dtype or dres.shape != h.shape:
            raise ValueError("oracle: dres must match h")
    if dy.dtype != h.dtype or dy.shape != h.shape:
        raise ValueError("oracle: dy and h must share dtype and shape")
    N = h.shape[-1]
    M = h.numel() // N
    dh = torch.empty(h.shape, dtype=dh_dtype or h.dtype)
    dw = torch.empty((N,), dtype=dw_dtype)
    dw_abs = torch.empty((N,), dtype=torch.float64)
    _check(_load().oracle_add_rmsnorm_bwd(_ptr(dy), _ptr(dres), _ptr(h), _code(h), _ptr(w),
                                          _code(w), _ptr(rstd), _code(rstd), _ptr(dh), _code(dh),
                                          _ptr(dw), _code(dw), _ptr(dw_abs), M, N),
           "add_rmsnorm_bwd")
    return dh, dw, dw_abs


def layernorm_fwd(x: torch.Tensor, w: torch.Tensor, b, eps: float, *, y_dtype=None,
                  stat_dtype=torch.float32, eps_exact: bool = False):
    """LayerNorm over the last dim: y = (x - mean) * rstd * w (+ b).
    Returns (y, mean, rstd)."""
    x, w = _cpu(x), _cpu(w)
    if b is not None:
        b = _cpu(b)
        if b.dtype != w.dtype:
            raise ValueError("oracle: b must have w's dtype")
    N = x.shape[-1]
    M = x.numel() // N
    y = torch.empty(x.shape, dtype=y_dtype or x.dtype)
    mean = torch.empty(x.shape[:-1], dtype=stat_dtype)
    rstd = torch.empty(x.shape[:-1], dtype=stat_dtype)
    e = float(eps) if eps_exact else eps_as_float32(eps)
    _check(_load().oracle_layernorm_fwd(_ptr(x), _code(x), _ptr(w), _ptr(b), _code(w), _ptr(y),
                                        _code(y), _ptr(mean), _ptr(rstd), _code(mean), M, N, e),
           "layernorm_fwd")
    return y, mean, rstd


def add_layernorm_fwd(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor, b, eps: float, *,
                      y_dtype=None, res_dtype=None, stat_dtype=torch.float32,
                      eps_exact: bool = False):
    """residual_out = stored(x + r); y = LayerNorm(residual_out) * w (+ b).
    Returns (y, residual_out, mean, rstd)."""
    x, r, w = _cpu(x), _cpu(r), _cpu(w)
    if b is not None:
        b = _cpu(b)
    if x.dtype != r.dtype or x.shape != r.shape:
        raise ValueError("oracle: x and r must share dtype and shape")
    N = x.shape[-1]
    M = x.numel() // N
    y = torch.empty(x.shape, dtype=y_dtype or x.dtype)
    res = torch.empty(x.shape, dtype=res_dtype or x.dtype)
    mean = torch.empty(x.shape[:-1], dtype=stat_dtype)
    rstd = torch.empty(x.shape[:-1], dtype=stat_dtype)
    e = float(eps) if eps_exact else eps_as_float32(eps)
    _check(_load().oracle_add_layernorm_fwd(_ptr(x), _ptr(r), _code(x), _ptr(w), _ptr(b),
                                            _code(w), _ptr(y), _code(y), _ptr(res), _code(res),
                                            _ptr(mean), _ptr(rstd), _code(mean), M, N, e),
           "add_layernorm_fwd")
    return y, res, mean, rstd


def layernorm_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, mean: torch.Tensor,
                  rstd: torch.Tensor, *, dx_dtype=None, dwb_dtype=torch.float32):
    """dx, dw, db from the saved mean and rstd.  Returns
    (dx, dw, db, dw_abs, db_abs)."""
    dy, x, w, mean, rstd = _cpu(dy), _cpu(x), _cpu(w), _cpu(mean), _cpu(rstd)
    if mean.dtype != rstd.dtype:
        raise ValueError("oracle: mean and rstd must share dtype")
    N = x.shape[-1]
    M = x.numel() // N
    dx = torch.empty(x.shape, dtype=dx_dtype or x.dtype)
    dw = torch.empty((N,), dtype=dwb_dtype)
    db = torch.empty((N,), dtype=dwb_dtype)
    dw_abs = torch.empty((N,), dtype=torch.float64)
    db_abs = torch.empty((N,), dtype=torch.float64)
    _check(_load().oracle_layernorm_bwd(_ptr(dy), _ptr(x), _code(x), _ptr(w), _code(w),
                                        _ptr(mean), _ptr(rstd), _code(mean), _ptr(dx), _code(dx),
                                        _ptr(dw), _ptr(db), _code(dw), _ptr(dw_abs),
                                        _ptr(db_abs), M, N), "layernorm_bwd")
    return dx, dw, db, dw_abs, db_abs


def add_layernorm_bwd(dy: torch.Tensor, dres, h: torch.Tensor, w: torch.Tensor,
                      mean: torch.Tensor, rstd: torch.Tensor, *, dh_dtype=None,
                      dwb_dtype=torch.float32):
    """Backward of the fused Add + LayerNorm: dh (the gradient of x and of r),
    dw, db from dy, the residual_out gradient dres (None for zero), the saved
    residual h, mean and rstd.  Returns (dh, dw, db, dw_abs, db_abs)."""
    dy, h, w, mean, rstd = _cpu(dy), _cpu(h), _cpu(w), _cpu(mean), _cpu(rstd)
    if dres is not None:
        dres = _cpu(dres)
    N = h.shape[-1]
    M = h.numel() // N
    dh = torch.empty(h.shape, dtype=dh_dtype or h.dtype)
    dw = torch.empty((N,), dtype=dwb_dtype)
    db = torch.empty((N,), dtype=dwb_dtype)
    dw_abs = torch.empty((N,), dtype=torch.float64)
    db_abs = torch.empty((N,), dtype=torch.float64)
    _check(_load().oracle_add_layernorm_bwd(_ptr(dy), _ptr(dres), _ptr(h), _code(h), _ptr(w),
                                            _code(w), _ptr(mean), _ptr(rstd), _code(mean),
                                            _ptr(dh), _code(dh), _ptr(dw), _ptr(db), _code(dw),
                                            _ptr(dw_abs), _ptr(db_abs), M, N),
           "add_layernorm_bwd")
    return dh, dw, db, dw_abs, db_abs


def fp8e4m3_encode(v) -> np.ndarray:
    """binary64 values -> E4M3 codes (uint8): RNE, saturating to +-448."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint8)
    _load().oracle_fp8e4m3_encode_array(a.ctypes.data, out.ctypes.data, a.size)
    return out


def fp8e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes -> exact binary64 values."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_fp8e4m3_decode(int(b)) for b in c.ravel()]).reshape(c.shape)


def rmsnorm_fwd_fp8(x: torch.Tensor, w: torch.Tensor, eps: float, *, residual=None,
                    group: int = 0, eps_exact: bool = False):
    """RMSNorm with an E4M3 output and dynamic scales: one per row (group=0)
    or one per `group` consecutive columns (scale shape [M, ceil(N/group)]).
    With residual=r, the fused form: x + r is stored first and normalised.
    Returns (q uint8, scale float32, rstd float32) or, fused,
    (q, scale, residual_out, rstd)."""
    x, w = _cpu(x), _cpu(w)
    N = x.shape[-1]
    M = x.numel() // N
    g = max(0, int(group))
    ng = (N + min(g, N) - 1) // min(g, N) if g else 0   # group >= N: one group per row
    q = torch.empty(x.shape, dtype=torch.uint8)
    scale = torch.empty(x.shape[:-1] + (ng,) if g else x.shape[:-1], dtype=torch.float32)
    rstd = torch.empty(x.shape[:-1], dtype=torch.float32)
    e = float(eps) if eps_exact else eps_as_float32(eps)
    if residual is None:
        _check(_load().oracle_rmsnorm_fwd_fp8_grouped(_ptr(x), _code(x), _ptr(w), _code(w),
                                                      _ptr(q), _ptr(scale), g, _ptr(rstd),
                                                      _code(rstd), M, N, e), "rmsnorm_fwd_fp8")
        return q, scale, rstd
    r = _cpu(residual)
    res = torch.empty(x.shape, dtype=x.dtype)
    _check(_load().oracle_add_rmsnorm_fwd_fp8_grouped(_ptr(x), _ptr(r), _code(x), _ptr(w),
                                                      _code(w), _ptr(q), _ptr(scale), g,
                                                      _ptr(res), _code(res), _ptr(rstd),
                                                      _code(rstd), M, N, e),
           "add_rmsnorm_fwd_fp8")
    return q, scale, res, rstd


def rmsnorm_rope(x: torch.Tensor, w: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                 pos: torch.Tensor, eps: float, *, interleaved: bool = False, y_dtype=None,
                 eps_exact: bool = False) -> torch.Tensor:
    """Per-head RMSNorm (weight w[D]) then RoPE by position, for heads x[T, H, D].

    x may be a view with any token stride (e.g. the query or key part of a
    packed projection output) as long as each token's H*D values are
    contiguous.  cos, sin: float32 [P, D/2]; pos: int64 [T].  Returns a
    contiguous [T, H, D] tensor in y_dtype (default x's dtype).  A position
    outside [0, P) gives NaN heads."""
    if x.device.type != "cpu" or x.dim() != 3:
        raise ValueError("oracle: x must be a CPU [T, H, D] tensor")
    T, H, D = x.shape
    if x.stride(2) != 1 or (H > 1 and x.stride(1) != D):
        x = x.contiguous()
    w, cos, sin = _cpu(w), _cpu(cos), _cpu(sin)
    pos = _cpu(pos)
    if pos.dtype != torch.int64 or cos.dtype != torch.float32 or sin.dtype != torch.float32:
        raise TypeError("oracle: pos int64, cos/sin float32")
    y = torch.empty((T, H, D), dtype=y_dtype or x.dtype)
    e = float(eps) if eps_exact else eps_as_float32(eps)
    _check(_load().oracle_rmsnorm_rope(_ptr(x), _code(x), x.stride(0) if T > 1 else H * D,
                                       _ptr(w), _code(w), _ptr(cos), _ptr(sin), _ptr(pos),
                                       cos.shape[0], _ptr(y), _code(y), H * D, T, H, D,
                                       int(bool(interleaved)), e), "rmsnorm_rope")
    return y


def fp4e2m1_encode(v) -> np.ndarray:
    """E2M1 codes (uint8, 0..15) of binary64 values: nearest, ties to the even
    code, saturating at +-6, sign kept."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint8)
    _load().oracle_fp4e2m1_encode_array(a.ctypes.data_as(ctypes.c_void_p),
                                        out.ctypes.data_as(ctypes.c_void_p), a.size)
    return out


def fp4e2m1_decode(c) -> np.ndarray:
    """Exact binary64 values of E2M1 codes (the low 4 bits of each entry)."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    c = np.asarray(c, dtype=np.uint8)
    return np.where(c & 0x8, -1.0, 1.0) * grid[c & 0x7]


def unpack_fp4(q: torch.Tensor) -> np.ndarray:
    """[.., N/2] packed bytes (element 2i in the low nibble) -> [.., N] codes."""
    b = q.numpy() if isinstance(q, torch.Tensor) else np.asarray(q)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def rmsnorm_fwd_mxfp4(x: torch.Tensor, w: torch.Tensor, eps: float, *, residual=None,
                      eps_exact: bool = False):
    """RMSNorm with an MXFP4 output: E2M1 codes packed two per byte
    (q uint8 [M, N/2]), one E8M0 scale byte per 32 columns (scale uint8
    [M, ceil(N/32)]).  Returns (q, scale, rstd) or, with residual=r, the fused
    form (q, scale, residual_out, rstd)."""
    x, w = _cpu(x), _cpu(w)
    N = x.shape[-1]
    M = x.numel() // N
    q = torch.empty(x.shape[:-1] + (N // 2,), dtype=torch.uint8)
    scale = torch.empty(x.shape[:-1] + ((N + 31) // 32,), dtype=torch.uint8)
    rstd = torch.empty(x.shape[:-1], dtype=torch.float32)
    e = float(eps) if eps_exact else eps_as_float32(eps)
    if residual is None:
        _check(_load().oracle_rmsnorm_fwd_mxfp4(_ptr(x), _code(x), _ptr(w), _code(w), _ptr(q),
                                                _ptr(scale), _ptr(rstd), _code(rstd), M, N, e),
               "rmsnorm_fwd_mxfp4")
        return q, scale, rstd
    r = _cpu(residual)
    res = torch.empty(x.shape, dtype=x.dtype)
    _check(_load().oracle_add_rmsnorm_fwd_mxfp4(_ptr(x), _ptr(r), _code(x), _ptr(w), _code(w),
                                                _ptr(q), _ptr(scale), _ptr(res), _code(res),
                                                _ptr(rstd), _code(rstd), M, N, e),
           "add_rmsnorm_fwd_mxfp4")
    return q, scale, res, rstd
