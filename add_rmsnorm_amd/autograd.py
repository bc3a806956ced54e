"""PyTorch custom ops with autograd for RMSNorm, LayerNorm and their fused
residual-Add forms.

The KernelAgent digest describes KernelAgent-Oink's RMSNorm and fused
Add + RMSNorm as PyTorch custom operators, and the Machete README ("Built-In
Areas") lists autograd helpers for composing kernel-backed modules.  This
module registers the library's calls as ``torch.library`` custom ops
(``addrms::*``) with fake (shape) implementations and autograd formulas, so
they work in eager mode and under graph capture.  Every numeric step runs in
the HIP library; these functions only allocate outputs and marshal.

    y = rms_norm(x, w, eps)                    # differentiable in x and w
    y, residual = add_rms_norm(x, r, w, eps)   # differentiable in x, r and w
    RMSNorm(hidden, eps), AddRMSNorm(hidden, eps)   # nn.Module forms

Gradients: dx (and dr, equal to it for the fused op) in x's dtype; dw is
computed in float32 and returned in w's dtype.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch
from torch import Tensor

from . import (add_layernorm_bwd, add_layernorm_fwd, add_rmsnorm_bwd, add_rmsnorm_fwd,
               add_rmsnorm_fwd_fp8, add_rmsnorm_fwd_mxfp4, layernorm_bwd, layernorm_fwd,
               rmsnorm_bwd, rmsnorm_fwd, rmsnorm_fwd_fp8, rmsnorm_fwd_mxfp4, rmsnorm_rope_qk)

__all__ = ["rms_norm", "add_rms_norm", "layer_norm", "add_layer_norm", "rms_norm_fp8",
           "add_rms_norm_fp8", "rms_norm_mxfp4", "add_rms_norm_mxfp4", "rms_norm_rope_qk",
           "RMSNorm", "AddRMSNorm", "LayerNorm", "AddLayerNorm"]


# ---- forward / backward ops -------------------------------------------------
# The ops take inputs of any strides (they run on contiguous copies) and
# return contiguous outputs; the fake implementations say the same.

def _like(t: Tensor, dtype=None) -> Tensor:
    """An empty contiguous tensor of t's shape (and dtype unless given)."""
    return torch.empty(t.shape, dtype=dtype or t.dtype, device=t.device)


@torch.library.custom_op("addrms::rms_norm_fwd", mutates_args=())
def _rms_norm_fwd(x: Tensor, w: Tensor, eps: float) -> Tuple[Tensor, Tensor]:
    return rmsnorm_fwd(x.contiguous(), w.contiguous(), eps, return_rstd=True)


@_rms_norm_fwd.register_fake
def _(x, w, eps):
    return _like(x), x.new_empty(x.shape[:-1], dtype=torch.float32)


@torch.library.custom_op("addrms::rms_norm_bwd", mutates_args=())
def _rms_norm_bwd(dy: Tensor, x: Tensor, w: Tensor, rstd: Tensor) -> Tuple[Tensor, Tensor]:
    return rmsnorm_bwd(dy.contiguous(), x.contiguous(), w.contiguous(), rstd.contiguous())


@_rms_norm_bwd.register_fake
def _(dy, x, w, rstd):
    return _like(x), w.new_empty(w.shape, dtype=torch.float32)


@torch.library.custom_op("addrms::add_rms_norm_fwd", mutates_args=())
def _add_rms_norm_fwd(x: Tensor, r: Tensor, w: Tensor, eps: float) -> Tuple[Tensor, Tensor, Tensor]:
    return add_rmsnorm_fwd(x.contiguous(), r.contiguous(), w.contiguous(), eps, return_rstd=True)


@_add_rms_norm_fwd.register_fake
def _(x, r, w, eps):
    return _like(x), _like(x), x.new_empty(x.shape[:-1], dtype=torch.float32)


@torch.library.custom_op("addrms::add_rms_norm_bwd", mutates_args=())
def _add_rms_norm_bwd(dy: Tensor, dres: Optional[Tensor], h: Tensor, w: Tensor,
                      rstd: Tensor) -> Tuple[Tensor, Tensor]:
    return add_rmsnorm_bwd(dy.contiguous(), None if dres is None else dres.contiguous(),
                           h.contiguous(), w.contiguous(), rstd.contiguous())


@_add_rms_norm_bwd.register_fake
def _(dy, dres, h, w, rstd):
    return _like(h), w.new_empty(w.shape, dtype=torch.float32)


# ---- autograd ----------------------------------------------------------------

def _rms_setup(ctx, inputs, output):
    x, w, _ = inputs
    _, rstd = output
    ctx.save_for_backward(x, w, rstd)
    ctx.mark_non_differentiable(rstd)


def _rms_backward(ctx, dy, _drstd):
    x, w, rstd = ctx.saved_tensors
    if dy is None:
        dy = torch.zeros(x.shape, dtype=x.dtype, device=x.device)
    dx, dw = _rms_norm_bwd(dy, x, w, rstd)
    return dx, dw.to(w.dtype), None


_rms_norm_fwd.register_autograd(_rms_backward, setup_context=_rms_setup)


def _add_setup(ctx, inputs, output):
    _, _, w, _ = inputs
    _, res, rstd = output
    ctx.save_for_backward(res, w, rstd)
    ctx.mark_non_differentiable(rstd)


def _add_backward(ctx, dy, dres, _drstd):
    h, w, rstd = ctx.saved_tensors
    if dy is None:
        dy = torch.zeros(h.shape, dtype=h.dtype, device=h.device)
    dh, dw = _add_rms_norm_bwd(dy, dres, h, w, rstd)
    return dh, dh, dw.to(w.dtype), None


_add_rms_norm_fwd.register_autograd(_add_backward, setup_context=_add_setup)


# ---- LayerNorm ------------------------------------------------------------------

@torch.library.custom_op("addrms::layer_norm_fwd", mutates_args=())
def _layer_norm_fwd(x: Tensor, w: Tensor, b: Optional[Tensor],
                    eps: float) -> Tuple[Tensor, Tensor, Tensor]:
    return layernorm_fwd(x.contiguous(), w.contiguous(), None if b is None else b.contiguous(),
                         eps, return_stats=True)


@_layer_norm_fwd.register_fake
def _(x, w, b, eps):
    st = x.new_empty(x.shape[:-1], dtype=torch.float32)
    return _like(x), st, torch.empty_like(st)


@torch.library.custom_op("addrms::add_layer_norm_fwd", mutates_args=())
def _add_layer_norm_fwd(x: Tensor, r: Tensor, w: Tensor, b: Optional[Tensor],
                        eps: float) -> Tuple[Tensor, Tensor, Tensor, Tensor]:
    return add_layernorm_fwd(x.contiguous(), r.contiguous(), w.contiguous(),
                             None if b is None else b.contiguous(), eps, return_stats=True)


@_add_layer_norm_fwd.register_fake
def _(x, r, w, b, eps):
    st = x.new_empty(x.shape[:-1], dtype=torch.float32)
    return _like(x), _like(x), st, torch.empty_like(st)


@torch.library.custom_op("addrms::layer_norm_bwd", mutates_args=())
def _layer_norm_bwd(dy: Tensor, x: Tensor, w: Tensor, mean: Tensor,
                    rstd: Tensor) -> Tuple[Tensor, Tensor, Tensor]:
    return layernorm_bwd(dy.contiguous(), x.contiguous(), w.contiguous(), mean.contiguous(),
                         rstd.contiguous(), with_db=True)


@_layer_norm_bwd.register_fake
def _(dy, x, w, mean, rstd):
    return (_like(x), w.new_empty(w.shape, dtype=torch.float32),
            w.new_empty(w.shape, dtype=torch.float32))


@torch.library.custom_op("addrms::add_layer_norm_bwd", mutates_args=())
def _add_layer_norm_bwd(dy: Tensor, dres: Optional[Tensor], h: Tensor, w: Tensor, mean: Tensor,
                        rstd: Tensor) -> Tuple[Tensor, Tensor, Tensor]:
    return add_layernorm_bwd(dy.contiguous(), None if dres is None else dres.contiguous(),
                             h.contiguous(), w.contiguous(), mean.contiguous(), rstd.contiguous(),
                             with_db=True)


@_add_layer_norm_bwd.register_fake
def _(dy, dres, h, w, mean, rstd):
    return (_like(h), w.new_empty(w.shape, dtype=torch.float32),
            w.new_empty(w.shape, dtype=torch.float32))


def _ln_setup(ctx, inputs, output):
    x, w, b, _ = inputs
    _, mean, rstd = output
    ctx.has_b = b is not None
    ctx.save_for_backward(x, w, mean, rstd)
    ctx.mark_non_differentiable(mean, rstd)


def _ln_backward(ctx, dy, _dmean, _drstd):
    x, w, mean, rstd = ctx.saved_tensors
    if dy is None:
        dy = torch.zeros(x.shape, dtype=x.dtype, device=x.device)
    dx, dw, db = _layer_norm_bwd(dy, x, w, mean, rstd)
    return dx, dw.to(w.dtype), (db.to(w.dtype) if ctx.has_b else None), None


_layer_norm_fwd.register_autograd(_ln_backward, setup_context=_ln_setup)


def _add_ln_setup(ctx, inputs, output):
    _, _, w, b, _ = inputs
    _, res, mean, rstd = output
    ctx.has_b = b is not None
    ctx.save_for_backward(res, w, mean, rstd)
    ctx.mark_non_differentiable(mean, rstd)


def _add_ln_backward(ctx, dy, dres, _dmean, _drstd):
    h, w, mean, rstd = ctx.saved_tensors
    if dy is None:
        dy = torch.zeros(h.shape, dtype=h.dtype, device=h.device)
    dh, dw, db = _add_layer_norm_bwd(dy, dres, h, w, mean, rstd)
    return dh, dh, dw.to(w.dtype), (db.to(w.dtype) if ctx.has_b else None), None


_add_layer_norm_fwd.register_autograd(_add_ln_backward, setup_context=_add_ln_setup)


# ---- forward-only ops: quantised output, RMSNorm + RoPE ---------------------------
# Quantisation has no useful gradient and the composed norm + rotation has no
# backward here; these ops are registered (with fake implementations) so that
# they can sit in a traced or compiled graph.

_FP8 = torch.float8_e4m3fn


def _scale_shape(x: Tensor, group: int):
    N = x.shape[-1]
    if group <= 0:
        return x.shape[:-1]
    g = min(group, N)
    return x.shape[:-1] + ((N + g - 1) // g,)


@torch.library.custom_op("addrms::rms_norm_fp8", mutates_args=())
def _rms_norm_fp8(x: Tensor, w: Tensor, eps: float, group: int) -> Tuple[Tensor, Tensor]:
    return rmsnorm_fwd_fp8(x.contiguous(), w.contiguous(), eps,
                           group=group if group > 0 else None)


@_rms_norm_fp8.register_fake
def _(x, w, eps, group):
    return x.new_empty(x.shape, dtype=_FP8), x.new_empty(_scale_shape(x, group),
                                                          dtype=torch.float32)


@torch.library.custom_op("addrms::add_rms_norm_fp8", mutates_args=())
def _add_rms_norm_fp8(x: Tensor, r: Tensor, w: Tensor, eps: float,
                      group: int) -> Tuple[Tensor, Tensor, Tensor]:
    return add_rmsnorm_fwd_fp8(x.contiguous(), r.contiguous(), w.contiguous(), eps,
                               group=group if group > 0 else None)


@_add_rms_norm_fp8.register_fake
def _(x, r, w, eps, group):
    return (x.new_empty(x.shape, dtype=_FP8),
            x.new_empty(_scale_shape(x, group), dtype=torch.float32), _like(x))


def _mx_shapes(x: Tensor):
    N = x.shape[-1]
    return x.shape[:-1] + (N // 2,), x.shape[:-1] + ((N + 31) // 32,)


@torch.library.custom_op("addrms::rms_norm_mxfp4", mutates_args=())
def _rms_norm_mxfp4(x: Tensor, w: Tensor, eps: float) -> Tuple[Tensor, Tensor]:
    return rmsnorm_fwd_mxfp4(x.contiguous(), w.contiguous(), eps)


@_rms_norm_mxfp4.register_fake
def _(x, w, eps):
    cs, ss = _mx_shapes(x)
    return x.new_empty(cs, dtype=torch.float4_e2m1fn_x2), x.new_empty(ss, dtype=torch.float8_e8m0fnu)


@torch.library.custom_op("addrms::add_rms_norm_mxfp4", mutates_args=())
def _add_rms_norm_mxfp4(x: Tensor, r: Tensor, w: Tensor, eps: float) -> Tuple[Tensor, Tensor, Tensor]:
    return add_rmsnorm_fwd_mxfp4(x.contiguous(), r.contiguous(), w.contiguous(), eps)


@_add_rms_norm_mxfp4.register_fake
def _(x, r, w, eps):
    cs, ss = _mx_shapes(x)
    return (x.new_empty(cs, dtype=torch.float4_e2m1fn_x2),
            x.new_empty(ss, dtype=torch.float8_e8m0fnu), _like(x))


@torch.library.custom_op("addrms::rms_norm_rope_qk", mutates_args=())
def _rms_norm_rope_qk(q: Tensor, k: Tensor, wq: Tensor, wk: Tensor, cos: Tensor, sin: Tensor,
                      pos: Tensor, eps: float, interleaved: bool) -> Tuple[Tensor, Tensor]:
    return rmsnorm_rope_qk(q, k, wq, wk, cos, sin, pos, eps, interleaved=interleaved)


@_rms_norm_rope_qk.register_fake
def _(q, k, wq, wk, cos, sin, pos, eps, interleaved):
    return q.new_empty(q.shape), k.new_empty(k.shape)


@torch.library.custom_op("addrms::rms_norm_rope_qk_", mutates_args=("q", "k"))
def _rms_norm_rope_qk_(q: Tensor, k: Tensor, wq: Tensor, wk: Tensor, cos: Tensor, sin: Tensor,
                       pos: Tensor, eps: float, interleaved: bool) -> None:
    rmsnorm_rope_qk(q, k, wq, wk, cos, sin, pos, eps, interleaved=interleaved, q_out=q, k_out=k)


@_rms_norm_rope_qk_.register_fake
def _(q, k, wq, wk, cos, sin, pos, eps, interleaved):
    return None


# ---- user-facing functions and modules ----------------------------------------

def rms_norm_fp8(x: Tensor, w: Tensor, eps: float = 1e-6,
                 group: Optional[int] = None) -> Tuple[Tensor, Tensor]:
    """RMSNorm with an E4M3 output: (codes float8_e4m3fn, float32 scales), one
    scale per row or per `group` columns.  Not differentiable."""
    return _rms_norm_fp8(x, w, eps, int(group or 0))


def add_rms_norm_fp8(x: Tensor, r: Tensor, w: Tensor, eps: float = 1e-6,
                     group: Optional[int] = None) -> Tuple[Tensor, Tensor, Tensor]:
    """Fused residual add + RMSNorm with an E4M3 output: (codes, scales,
    residual).  Not differentiable."""
    return _add_rms_norm_fp8(x, r, w, eps, int(group or 0))


def rms_norm_mxfp4(x: Tensor, w: Tensor, eps: float = 1e-6) -> Tuple[Tensor, Tensor]:
    """RMSNorm with an MXFP4 output: (codes float4_e2m1fn_x2 [.., N/2], scales
    float8_e8m0fnu [.., ceil(N/32)]).  Not differentiable."""
    return _rms_norm_mxfp4(x, w, eps)


def add_rms_norm_mxfp4(x: Tensor, r: Tensor, w: Tensor,
                       eps: float = 1e-6) -> Tuple[Tensor, Tensor, Tensor]:
    """Fused residual add + RMSNorm with an MXFP4 output: (codes, scales,
    residual).  Not differentiable."""
    return _add_rms_norm_mxfp4(x, r, w, eps)


def rms_norm_rope_qk(q: Tensor, k: Tensor, wq: Tensor, wk: Tensor, cos: Tensor, sin: Tensor,
                     pos: Tensor, eps: float = 1e-6, interleaved: bool = False,
                     inplace: bool = False):
    """Per-head RMSNorm then RoPE of query heads q [T, Hq, D] and key heads
    k [T, Hk, D] (views of a packed projection output are fine).  Returns
    (q_out, k_out), or, with inplace=True, updates q and k and returns them.
    Not differentiable."""
    if inplace:
        _rms_norm_rope_qk_(q, k, wq, wk, cos, sin, pos, eps, interleaved)
        return q, k
    return _rms_norm_rope_qk(q, k, wq, wk, cos, sin, pos, eps, interleaved)


def rms_norm(x: Tensor, w: Tensor, eps: float = 1e-6) -> Tensor:
    """RMSNorm over the last dimension, differentiable in x and w."""
    return _rms_norm_fwd(x, w, eps)[0]


def add_rms_norm(x: Tensor, r: Tensor, w: Tensor, eps: float = 1e-6) -> Tuple[Tensor, Tensor]:
    """Fused residual add + RMSNorm: returns (RMSNorm(x + r) * w, x + r),
    differentiable in x, r and w (the residual output carries its own
    gradient into dx and dr)."""
    y, res, _ = _add_rms_norm_fwd(x, r, w, eps)
    return y, res


class RMSNorm(torch.nn.Module):
    """y = RMSNorm(x) * weight, weight initialised to ones."""

    def __init__(self, hidden: int, eps: float = 1e-6, dtype=torch.bfloat16, device=None):
        super().__init__()
        self.eps = eps
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=dtype, device=device))

    def forward(self, x: Tensor) -> Tensor:
        return rms_norm(x, self.weight, self.eps)


class AddRMSNorm(torch.nn.Module):
    """(y, residual) = (RMSNorm(x + residual) * weight, x + residual): the
    pre-norm transformer's residual update and normalisation in one pass."""

    def __init__(self, hidden: int, eps: float = 1e-6, dtype=torch.bfloat16, device=None):
        super().__init__()
        self.eps = eps
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=dtype, device=device))

    def forward(self, x: Tensor, residual: Tensor) -> Tuple[Tensor, Tensor]:
        return add_rms_norm(x, residual, self.weight, self.eps)


def layer_norm(x: Tensor, w: Tensor, b: Optional[Tensor] = None, eps: float = 1e-5) -> Tensor:
    """LayerNorm over the last dimension, differentiable in x, w and b."""
    return _layer_norm_fwd(x, w, b, eps)[0]


def add_layer_norm(x: Tensor, r: Tensor, w: Tensor, b: Optional[Tensor] = None,
                   eps: float = 1e-5) -> Tuple[Tensor, Tensor]:
    """Fused residual add + LayerNorm: (LayerNorm(x + r) * w + b, x + r)."""
    y, res, _, _ = _add_layer_norm_fwd(x, r, w, b, eps)
    return y, res


class LayerNorm(torch.nn.Module):
    """y = LayerNorm(x) * weight + bias (weight ones, bias zeros)."""

    def __init__(self, hidden: int, eps: float = 1e-5, bias: bool = True, dtype=torch.bfloat16,
                 device=None):
        super().__init__()
        self.eps = eps
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=dtype, device=device))
        self.bias = (torch.nn.Parameter(torch.zeros(hidden, dtype=dtype, device=device))
                     if bias else None)

    def forward(self, x: Tensor) -> Tensor:
        return layer_norm(x, self.weight, self.bias, self.eps)


class AddLayerNorm(LayerNorm):
    """(y, residual) = (LayerNorm(x + residual) * weight + bias, x + residual)."""

    def forward(self, x: Tensor, residual: Tensor) -> Tuple[Tensor, Tensor]:
        return add_layer_norm(x, residual, self.weight, self.bias, self.eps)
