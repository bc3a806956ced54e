"""Comparison helpers for the GPU parity tests.

Tolerances (floating-point outputs, |gpu - oracle| <= atol + rtol * |oracle|):
    bfloat16 y, dx : atol 1e-2, rtol 1.6e-2
    float16  y, dx : atol 1e-4, rtol 2e-3 (two float16 ulps relative; the
                     absolute term covers float32 cancellation near zero)
    float32  y, dx : atol 1e-6, rtol 1e-5
    float32  rstd  : rtol 1e-5 (bf16 inputs) -- one float32 rounding of the
                     sum of squares and of 1/sqrt
    float32  dw    : rtol 1e-3 plus atol 1e-5 * sum_i |dy_ij x_ij rstd_i|
                     (a multiple of the error the library's summation order
                     can reach); columns with |dw| >= 1e-2 of that magnitude
                     also meet rtol 1e-3 alone
    bf16 y, dx, dh : also within half a bf16 ulp of the binary64 value plus
                     float32 noise (one rounding; assert_correctly_rounded),
                     and float16 outputs within half a float16 ulp
Residuals are compared bit for bit; NaN must sit where the oracle has NaN.
"""
import numpy as np
import torch

TOL = {torch.bfloat16: (1e-2, 1.6e-2), torch.float32: (1e-6, 1e-5), torch.float16: (1e-4, 2e-3)}


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
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
    with np.errstate(invalid="ignore"):  # inf - inf where both are infinite
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
    # columns whose sum is not dominated by cancellation (|dw| >= 1e-2 of the
    # magnitude of its terms) must also meet rtol 1e-3 alone
    strong = np.abs(r) >= 1e-2 * m
    ok = ~strong | (np.abs(g - r) <= 1e-3 * np.abs(r))
    if not ok.all():
        i = np.nonzero(~ok)[0][0]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {int(strong.sum())} columns without "
                             f"cancellation outside rtol 1e-3; first col {i}: gpu {g[i]!r} "
                             f"ref {r[i]!r}")


def assert_correctly_rounded(gpu: torch.Tensor, ref64: torch.Tensor, mag, what: str,
                             noise: float = 2.0 ** -18):
    """bfloat16 or float16 outputs rounded once (reading R5): every finite
    element lies within half an ulp of its storage type from the oracle's
    binary64 value plus the float32 arithmetic's own error, noise * mag,
    where mag (a tensor, or None for |ref64|) bounds the magnitude of the
    terms the element was computed from.  Rounding the float32 result once
    stays within half an ulp of its float32 value; an extra rounding on the
    way (of h * rstd, or of the row terms of dx) adds up to another half ulp,
    2^-9 (bf16) or 2^-12 (float16) relative, hundreds of times the noise
    term."""
    g = gpu.detach().cpu().float().numpy().astype(np.float64)
    r = ref64.detach().cpu().numpy().astype(np.float64)
    m = np.abs(r) if mag is None else np.asarray(mag.detach().cpu().numpy() if hasattr(mag, "detach")
                                                 else mag, dtype=np.float64)
    m = np.broadcast_to(m, r.shape)
    fin = np.isfinite(r)
    if gpu.dtype == torch.float16:   # 11 significant bits; subnormal spacing 2^-24
        a = np.maximum(np.abs(r[fin]), 2.0 ** -14)
        half_ulp = 2.0 ** (np.floor(np.log2(a)) - 11)
        name, floor_ = "float16", 2.0 ** -25
    else:                            # bf16 keeps 8 significant bits
        a = np.maximum(np.abs(r[fin]), 2.0 ** -126)
        half_ulp = 2.0 ** (np.floor(np.log2(a)) - 8)
        name, floor_ = "bf16", 2.0 ** -133
    err = np.abs(g[fin] - r[fin])
    lim = half_ulp + noise * m[fin] + floor_
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements more than half a "
                           f"{name} ulp (+ float32 noise) from the binary64 value; worst excess "
                           f"{float((err - lim).max())}")
