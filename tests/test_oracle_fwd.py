"""Pins for the oracle's forward (CPU only).

Each test checks the oracle against something other than itself: torch's
float64 rms_norm (a library routine), hand-derived worked examples with exact
rational answers, closed forms (constant rows, zero rows, N = 1, the unit-RMS
property for w = 1), the exact power-of-two scale identity, torch's binary32
add + bfloat16 conversion for the fused residual, and the special cases of the
add (r = 0, r = -x, x <-> r)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _f64(a):
    return torch.tensor(np.asarray(a, dtype=np.float64))


@pytest.mark.parametrize("M,N", [(1, 1), (3, 2), (5, 3), (7, 64), (4, 257), (2, 1000)])
@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_matches_torch_rms_norm_float64(M, N, eps):
    x = synth.store(synth.normal(3, "x", (M, N)), torch.float64)
    w = synth.weight(3, N, torch.float64)
    y, rstd = oracle.rmsnorm_fwd(x, w, eps, rstd_dtype=torch.float64, eps_exact=True)
    ref = F.rms_norm(x, (N,), w, eps)
    torch.testing.assert_close(y, ref, rtol=1e-13, atol=1e-15)
    ref_rstd = torch.rsqrt(x.pow(2).mean(-1) + eps)
    torch.testing.assert_close(rstd, ref_rstd, rtol=1e-14, atol=0)


def test_golden_forward_cases():
    for c in json.load(open(GOLDEN))["forward"]:
        x = _f64([c["x"]])
        w = _f64(c["w"])
        y, rstd = oracle.rmsnorm_fwd(x, w, c["eps"], rstd_dtype=torch.float64, eps_exact=True)
        assert rstd.item() == float(Fraction(c["rstd"])), c["name"]
        want = [float(Fraction(v)) for v in c["y"]]
        assert y[0].tolist() == pytest.approx(want, rel=1e-15, abs=0), c["name"]


def test_golden_fused_cases():
    for c in json.load(open(GOLDEN))["fused_forward"]:
        x = _f64([[float(Fraction(v)) for v in c["x"]]])
        r = _f64([[float(Fraction(v)) for v in c["r"]]])
        w = _f64(c["w"])
        y, res, _ = oracle.add_rmsnorm_fwd(x, r, w, c["eps"], eps_exact=True)
        assert res[0].tolist() == [float(Fraction(v)) for v in c["residual"]]
        assert y[0].tolist() == pytest.approx([float(Fraction(v)) for v in c["y"]], rel=1e-15)


@pytest.mark.parametrize("c", [1.0, -3.5, 1e-3, 250.0])
@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_constant_row_closed_form(c, eps):
    N = 37
    x = torch.full((2, N), c, dtype=torch.float64)
    w = synth.weight(5, N, torch.float64)
    y, _ = oracle.rmsnorm_fwd(x, w, eps, eps_exact=True, rstd_dtype=torch.float64)
    want = c / math.sqrt(c * c + eps) * w
    torch.testing.assert_close(y[0], want, rtol=1e-14, atol=0)
    torch.testing.assert_close(y[1], want, rtol=1e-14, atol=0)


def test_unit_weight_gives_unit_rms():
    """With w = 1, mean_j y_j^2 = ms / (ms + eps) exactly in real arithmetic."""
    M, N, eps = 6, 513, 1e-3
    x = synth.store(synth.normal(7, "x", (M, N), std=0.05), torch.float64)
    w = torch.ones(N, dtype=torch.float64)
    y, _ = oracle.rmsnorm_fwd(x, w, eps, eps_exact=True)
    ms = x.pow(2).mean(-1)
    torch.testing.assert_close(y.pow(2).mean(-1), ms / (ms + eps), rtol=1e-13, atol=0)


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32, torch.bfloat16])
def test_power_of_two_scale_identity_is_exact(dtype):
    """y(k x; eps) == y(x; eps / k^2) bit for bit for k = 4: every step scales
    by a power of two exactly, and sqrt is correctly rounded."""
    M, N, k = 5, 96, 4.0
    x = synth.store(synth.normal(11, "x", (M, N)), dtype)
    w = synth.weight(11, N, dtype)
    y1, _ = oracle.rmsnorm_fwd((x.double() * k).to(dtype), w, 1e-6, eps_exact=True)
    y2, _ = oracle.rmsnorm_fwd(x, w, 1e-6 / (k * k), eps_exact=True)
    assert torch.equal(y1.view(-1).double(), y2.view(-1).double())


def test_zero_row_and_single_column():
    w = torch.tensor([2.0, -1.0, 0.5], dtype=torch.float64)
    y, rstd = oracle.rmsnorm_fwd(torch.zeros(1, 3, dtype=torch.float64), w, 0.01,
                                 eps_exact=True, rstd_dtype=torch.float64)
    assert torch.equal(y, torch.zeros(1, 3, dtype=torch.float64))
    assert rstd.item() == pytest.approx(10.0, rel=1e-15)
    xs = torch.tensor([[3.0], [-0.2], [7.0]], dtype=torch.float64)
    y1, _ = oracle.rmsnorm_fwd(xs, torch.tensor([1.5], dtype=torch.float64), 1e-4, eps_exact=True)
    want = xs / torch.sqrt(xs * xs + 1e-4) * 1.5
    torch.testing.assert_close(y1, want, rtol=1e-15, atol=0)


def test_outputs_are_one_rounding_of_the_binary64_result():
    M, N = 4, 200
    x = synth.store(synth.normal(13, "x", (M, N)), torch.bfloat16)
    w = synth.weight(13, N, torch.bfloat16)
    y64, r64 = oracle.rmsnorm_fwd(x, w, 1e-6, y_dtype=torch.float64, rstd_dtype=torch.float64)
    yb, r32 = oracle.rmsnorm_fwd(x, w, 1e-6)
    y32, _ = oracle.rmsnorm_fwd(x, w, 1e-6, y_dtype=torch.float32)
    assert np.array_equal(yb.view(torch.int16).numpy().view(np.uint16),
                          oracle.bf16_round(y64.numpy()))
    assert torch.equal(y32, y64.to(torch.float32))
    assert torch.equal(r32, r64.to(torch.float32))
    # and the binary64 result agrees with torch's float64 routine on the same data
    ref = F.rms_norm(x.double(), (N,), w.double(), oracle.eps_as_float32(1e-6))
    torch.testing.assert_close(y64, ref, rtol=1e-13, atol=1e-15)


# ---- fused residual add ---------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_residual_is_binary32_add_rounded_to_storage(dtype):
    M, N = 64, 333
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, seed=21, r_std=0.5)
    x, r, w = inp["x"], inp["r"], inp["w"]
    y, res, _ = oracle.add_rmsnorm_fwd(x, r, w, 1e-6)
    want = (x.float() + r.float()).to(dtype)
    assert torch.equal(res.view(-1).view(torch.uint8), want.view(-1).view(torch.uint8))
    # y is RMSNorm of the stored residual (torch float64 routine on it)
    ref = F.rms_norm(want.double(), (N,), w.double(), oracle.eps_as_float32(1e-6))
    y64, _, _ = oracle.add_rmsnorm_fwd(x, r, w, 1e-6, y_dtype=torch.float64)
    torch.testing.assert_close(y64, ref, rtol=1e-13, atol=1e-15)


def test_residual_wide_exponent_gaps():
    """Sums whose binary32 rounding then bfloat16 rounding differs from a
    single rounding of the exact sum: the residual must follow the binary32
    add (torch's float add is IEEE binary32)."""
    rng = np.random.default_rng(5)
    xb = rng.integers(0, 1 << 16, size=200000, dtype=np.uint32).astype(np.uint16)
    rb = rng.integers(0, 1 << 16, size=200000, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).reshape(-1, 1000)
    r = torch.from_numpy(rb.view(np.int16)).view(torch.bfloat16).reshape(-1, 1000)
    w = torch.ones(1000, dtype=torch.bfloat16)
    _, res, _ = oracle.add_rmsnorm_fwd(x, r, w, 1e-6)
    want = (x.float() + r.float()).to(torch.bfloat16)
    a = res.view(torch.int16).numpy().view(np.uint16)
    b = want.view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(want.float().numpy())
    assert np.array_equal(a[~nan], b[~nan])
    assert np.all(((a[nan] & 0x7F80) == 0x7F80) & ((a[nan] & 0x7F) != 0))


def test_residual_special_cases():
    M, N = 8, 128
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=31)
    x, r, w = inp["x"], inp["r"], inp["w"]
    # r = 0: residual is x, output equals the plain op on x
    y0, res0, s0 = oracle.add_rmsnorm_fwd(x, torch.zeros_like(x), w, 1e-6)
    yp, sp = oracle.rmsnorm_fwd(x, w, 1e-6)
    assert torch.equal(res0.view(torch.int16), x.view(torch.int16))
    assert torch.equal(y0.view(torch.int16), yp.view(torch.int16)) and torch.equal(s0, sp)
    # r = -x: residual is +0 everywhere, y = 0
    yn, resn, _ = oracle.add_rmsnorm_fwd(x, -x, w, 1e-6)
    assert torch.all(resn.view(torch.int16) == 0)
    assert torch.all(yn.float() == 0)
    # x <-> r: bit-identical outputs
    ya, ra, sa = oracle.add_rmsnorm_fwd(x, r, w, 1e-6)
    yb, rb, sb = oracle.add_rmsnorm_fwd(r, x, w, 1e-6)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    assert torch.equal(ra.view(torch.int16), rb.view(torch.int16)) and torch.equal(sa, sb)
    # fused == plain op on the stored residual
    yr, sr = oracle.rmsnorm_fwd(ra, w, 1e-6)
    assert torch.equal(ya.view(torch.int16), yr.view(torch.int16)) and torch.equal(sa, sr)


def test_eps_is_rounded_to_binary32_by_default():
    assert oracle.eps_as_float32(1e-6) == float(np.float32(1e-6)) != 1e-6
