"""Pins for the oracle's backward (CPU only).

Checked against: torch.autograd through torch's float64 rms_norm (a library
routine), central finite differences of the oracle's own binary64 forward on
tiny shapes (brute force), hand-derived worked examples, the exact identity
sum_j x_j dx_j = eps rstd^3 sum_j g_j x_j (g = dy w), and linearity of dw in dy.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _case(M, N, seed):
    x = synth.store(synth.normal(seed, "x", (M, N)), torch.float64)
    dy = synth.store(synth.normal(seed, "dy", (M, N)), torch.float64)
    w = synth.weight(seed, N, torch.float64)
    return x, dy, w


@pytest.mark.parametrize("M,N", [(1, 1), (2, 2), (3, 17), (9, 64), (4, 300)])
@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_matches_torch_autograd_float64(M, N, eps):
    x, dy, w = _case(M, N, 41)
    _, rstd = oracle.rmsnorm_fwd(x, w, eps, eps_exact=True, rstd_dtype=torch.float64)
    dx, dw, _ = oracle.rmsnorm_bwd(dy, x, w, rstd, dw_dtype=torch.float64)
    xr, wr = x.clone().requires_grad_(True), w.clone().requires_grad_(True)
    F.rms_norm(xr, (N,), wr, eps).backward(dy)
    torch.testing.assert_close(dx, xr.grad, rtol=1e-11, atol=1e-13)
    torch.testing.assert_close(dw, wr.grad, rtol=1e-11, atol=1e-13)


def _loss(x, w, dy, eps):
    y, _ = oracle.rmsnorm_fwd(x, w, eps, eps_exact=True)
    return float((y * dy).sum())


@pytest.mark.parametrize("M,N", [(1, 1), (1, 2), (3, 3), (1, 8), (3, 17)])
def test_finite_differences(M, N):
    eps, h = 1e-3, 1e-6
    x, dy, w = _case(M, N, 43)
    _, rstd = oracle.rmsnorm_fwd(x, w, eps, eps_exact=True, rstd_dtype=torch.float64)
    dx, dw, _ = oracle.rmsnorm_bwd(dy, x, w, rstd, dw_dtype=torch.float64)
    fd_x = torch.empty_like(x)
    for i in range(M):
        for j in range(N):
            xp, xm = x.clone(), x.clone()
            xp[i, j] += h
            xm[i, j] -= h
            fd_x[i, j] = (_loss(xp, w, dy, eps) - _loss(xm, w, dy, eps)) / (2 * h)
    fd_w = torch.empty_like(w)
    for j in range(N):
        wp, wm = w.clone(), w.clone()
        wp[j] += h
        wm[j] -= h
        fd_w[j] = (_loss(x, wp, dy, eps) - _loss(x, wm, dy, eps)) / (2 * h)
    scale = max(1.0, float(dx.abs().max()))
    assert float((fd_x - dx).abs().max()) < 1e-7 * scale
    assert float((fd_w - dw).abs().max()) < 1e-7 * max(1.0, float(dw.abs().max()))


def test_golden_backward_cases():
    for c in json.load(open(GOLDEN))["backward"]:
        x = torch.tensor([c["x"]], dtype=torch.float64)
        w = torch.tensor(c["w"], dtype=torch.float64)
        dy = torch.tensor([c["dy"]], dtype=torch.float64)
        _, rstd = oracle.rmsnorm_fwd(x, w, c["eps"], eps_exact=True, rstd_dtype=torch.float64)
        assert rstd.item() == float(Fraction(c["rstd"])), c["name"]
        dx, dw, _ = oracle.rmsnorm_bwd(dy, x, w, rstd, dw_dtype=torch.float64)
        assert dx[0].tolist() == pytest.approx([float(Fraction(v)) for v in c["dx"]],
                                               rel=1e-14, abs=1e-16), c["name"]
        assert dw.tolist() == pytest.approx([float(Fraction(v)) for v in c["dw"]],
                                            rel=1e-14, abs=1e-16), c["name"]


@pytest.mark.parametrize("eps", [0.0, 1e-4, 0.5])
def test_radial_identity(eps):
    """sum_j x dx = eps rstd^3 sum_j (dy w) x: the gradient along x itself only
    comes from eps (RMSNorm is scale-invariant when eps = 0)."""
    M, N = 6, 50
    x, dy, w = _case(M, N, 47)
    _, rstd = oracle.rmsnorm_fwd(x, w, eps, eps_exact=True, rstd_dtype=torch.float64)
    dx, _, _ = oracle.rmsnorm_bwd(dy, x, w, rstd, dw_dtype=torch.float64)
    lhs = (x * dx).sum(-1)
    rhs = eps * rstd ** 3 * (dy * w * x).sum(-1)
    torch.testing.assert_close(lhs, rhs, rtol=1e-9, atol=1e-12)


def test_dw_linear_in_dy_and_abs_bound():
    M, N = 7, 40
    x, dy, w = _case(M, N, 53)
    dy2 = synth.store(synth.normal(54, "dy", (M, N)), torch.float64)
    _, rstd = oracle.rmsnorm_fwd(x, w, 1e-6, eps_exact=True, rstd_dtype=torch.float64)
    _, dwa, absa = oracle.rmsnorm_bwd(dy, x, w, rstd, dw_dtype=torch.float64)
    _, dwb, _ = oracle.rmsnorm_bwd(dy2, x, w, rstd, dw_dtype=torch.float64)
    _, dwab, _ = oracle.rmsnorm_bwd(2 * dy - 3 * dy2, x, w, rstd, dw_dtype=torch.float64)
    torch.testing.assert_close(dwab, 2 * dwa - 3 * dwb, rtol=1e-12, atol=1e-12)
    assert torch.all(absa >= dwa.abs())


def test_bf16_storage_uses_saved_fp32_rstd():
    """dx/dw for bf16 tensors are one rounding of the binary64 values computed
    from the saved float32 rstd, and agree with autograd of the float64 op to
    the rounding of rstd."""
    M, N = 16, 256
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.bfloat16, seed=59)
    x, dy, w = inp["x"], inp["dy"], inp["w"]
    _, rstd32 = oracle.rmsnorm_fwd(x, w, 1e-6)
    dx64, dw64, _ = oracle.rmsnorm_bwd(dy, x, w, rstd32, dx_dtype=torch.float64,
                                       dw_dtype=torch.float64)
    dxb, dw32, _ = oracle.rmsnorm_bwd(dy, x, w, rstd32)
    assert np.array_equal(dxb.view(torch.int16).numpy().view(np.uint16),
                          oracle.bf16_round(dx64.numpy()))
    assert torch.equal(dw32, dw64.float())
    xr = x.double().requires_grad_(True)
    wr = w.double().requires_grad_(True)
    F.rms_norm(xr, (N,), wr, oracle.eps_as_float32(1e-6)).backward(dy.double())
    torch.testing.assert_close(dx64, xr.grad, rtol=1e-6, atol=1e-6)
    torch.testing.assert_close(dw64, wr.grad, rtol=1e-6, atol=1e-6)


# ---- backward of the fused op ------------------------------------------------

@pytest.mark.parametrize("M,N", [(1, 1), (3, 17), (9, 64), (4, 300)])
@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_fused_matches_torch_autograd_float64(M, N, eps):
    """dh is the gradient of both x and r of L = sum(dy * y) + sum(dres * res)
    with res = x + r, y = rms_norm(res) * w."""
    x, dy, w = _case(M, N, 61)
    r = synth.store(synth.normal(61, "r", (M, N)), torch.float64)
    dres = synth.store(synth.normal(62, "dy", (M, N)), torch.float64)
    _, res, rstd = oracle.add_rmsnorm_fwd(x, r, w, eps, eps_exact=True, rstd_dtype=torch.float64)
    dh, dw, _ = oracle.add_rmsnorm_bwd(dy, dres, res, w, rstd, dw_dtype=torch.float64)
    xr, rr, wr = (t.clone().requires_grad_(True) for t in (x, r, w))
    s = xr + rr
    (F.rms_norm(s, (N,), wr, eps) * dy).sum().add((s * dres).sum()).backward()
    torch.testing.assert_close(dh, xr.grad, rtol=1e-11, atol=1e-13)
    torch.testing.assert_close(dh, rr.grad, rtol=1e-11, atol=1e-13)
    torch.testing.assert_close(dw, wr.grad, rtol=1e-11, atol=1e-13)


def test_fused_special_cases():
    M, N = 5, 40
    x, dy, w = _case(M, N, 67)
    dres = synth.store(synth.normal(68, "dy", (M, N)), torch.float64)
    _, rstd = oracle.rmsnorm_fwd(x, w, 1e-6, eps_exact=True, rstd_dtype=torch.float64)
    # no residual gradient: the plain backward
    dh0, dw0, _ = oracle.add_rmsnorm_bwd(dy, None, x, w, rstd, dw_dtype=torch.float64)
    dx, dw, _ = oracle.rmsnorm_bwd(dy, x, w, rstd, dw_dtype=torch.float64)
    assert torch.equal(dh0, dx) and torch.equal(dw0, dw)
    # no gradient of y: dh is the residual gradient exactly, dw = 0
    dh1, dw1, _ = oracle.add_rmsnorm_bwd(torch.zeros_like(dy), dres, x, w, rstd,
                                         dw_dtype=torch.float64)
    assert torch.equal(dh1, dres) and torch.all(dw1 == 0)


@pytest.mark.parametrize("M,N", [(1, 2), (3, 5)])
def test_fused_finite_differences(M, N):
    eps, h = 1e-3, 1e-6
    x, dy, w = _case(M, N, 71)
    r = synth.store(synth.normal(71, "r", (M, N)), torch.float64)
    dres = synth.store(synth.normal(72, "dy", (M, N)), torch.float64)

    def loss(xx):
        y, res, _ = oracle.add_rmsnorm_fwd(xx, r, w, eps, eps_exact=True)
        return float((y * dy).sum() + (res * dres).sum())

    _, res, rstd = oracle.add_rmsnorm_fwd(x, r, w, eps, eps_exact=True, rstd_dtype=torch.float64)
    dh, _, _ = oracle.add_rmsnorm_bwd(dy, dres, res, w, rstd, dw_dtype=torch.float64)
    fd = torch.empty_like(x)
    for i in range(M):
        for j in range(N):
            xp, xm = x.clone(), x.clone()
            xp[i, j] += h
            xm[i, j] -= h
            fd[i, j] = (loss(xp) - loss(xm)) / (2 * h)
    assert float((fd - dh).abs().max()) < 1e-7 * max(1.0, float(dh.abs().max()))
