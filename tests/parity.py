"""Comparison helpers for the GPU parity tests.

Tolerances (floating-point outputs, |gpu - oracle| <= atol + rtol * |oracle|):
    bfloat16 y, dx : atol 1e-2, rtol 1.6e-2
    float32  y, dx : atol 1e-6, rtol 1e-5
    float32  rstd  : rtol 1e-5 (bf16 inputs) -- one float32 rounding of the
                     sum of squares and of 1/sqrt
    float32  dw    : rtol 1e-3 plus atol 1e-5 * sum_i |dy_ij x_ij rstd_i|
                     (the magnitude that bounds any summation order's error)
Residuals are compared bit for bit; NaN must sit where the oracle has NaN.
"""
import numpy as np
import torch

TOL = {torch.bfloat16: (1e-2, 1.6e-2), torch.float32: (1e-6, 1e-5)}


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


def assert_bits_equal(gpu: torch.Tensor, ref: torch.Tensor, what: str):
    g, r = bits(gpu), bits(ref)
    gf = gpu.detach().cpu().float().numpy()
    rf = ref.detach().cpu().float().numpy()
    nan = np.isnan(rf)
    assert np.array_equal(np.isnan(gf), nan), f"{what}: NaN positions differ"
    bad = np.nonzero((g != r) & ~nan)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} elements differ, first at "
                              f"{tuple(b[0] for b in bad)}: gpu {g[bad][0]:#x} ref {r[bad][0]:#x}")


def assert_close(gpu: torch.Tensor, ref: torch.Tensor, what: str, atol=None, rtol=None):
    dt = ref.dtype
    a0, r0 = TOL[dt]
    atol = a0 if atol is None else atol
    rtol = r0 if rtol is None else rtol
    g = gpu.detach().cpu().double().numpy()
    r = ref.detach().cpu().double().numpy()
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(g), nan), f"{what}: NaN positions differ"
    inf = np.isinf(r)
    assert np.array_equal(g[inf], r[inf]), f"{what}: Inf values differ"
    ok = nan | inf | (np.abs(g - r) <= atol + rtol * np.abs(r))
    if not ok.all():
        bad = np.nonzero(~ok)
        i = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} of {ok.size} outside tolerance "
                             f"(atol {atol}, rtol {rtol}); first at {i}: gpu {g[i]!r} ref {r[i]!r}")


def assert_dw_close(gpu: torch.Tensor, ref: torch.Tensor, mag: torch.Tensor, what="dw"):
    g = gpu.detach().cpu().double().numpy()
    r = ref.detach().cpu().double().numpy()
    m = mag.detach().cpu().double().numpy()
    ok = np.abs(g - r) <= 1e-3 * np.abs(r) + 1e-5 * m
    if not ok.all():
        i = np.nonzero(~ok)[0][0]
        raise AssertionError(f"{what}: {int((~ok).sum())} columns outside tolerance; "
                             f"first col {i}: gpu {g[i]!r} ref {r[i]!r} mag {m[i]!r}")
