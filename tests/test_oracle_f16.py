"""Pins of the oracle's IEEE binary16 (float16) storage (CPU only).

The converter is written from IEEE 754's definition of binary16 (1 sign bit,
5 exponent bits with bias 15, 10 fraction bits; subnormals below 2^-14;
round to nearest, ties to even).  It is checked against independent
implementations of the same definition (numpy's float16 and torch's
float32 -> float16 conversions), every representable value, every midpoint
between neighbours, and the overflow and special cases; then the oracle's
float16 forwards against the same definitions composed by hand."""
import numpy as np
import pytest
import torch

import oracle
import synth

FINITE = np.array([b for b in range(1 << 16) if (b & 0x7C00) != 0x7C00], dtype=np.uint16)


def test_decode_every_pattern():
    b = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.f16_decode(b)
    ref = b.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_every_value_round_trips():
    assert np.array_equal(oracle.f16_round(oracle.f16_decode(FINITE)), FINITE)
    inf = np.array([0x7C00, 0xFC00], dtype=np.uint16)
    assert np.array_equal(oracle.f16_round(oracle.f16_decode(inf)), inf)


def test_midpoints_tie_to_even_and_neighbours_round_to_nearer():
    pos = np.arange(0, 0x7BFF, dtype=np.uint16)          # 0 .. the value below 65504
    a, b = oracle.f16_decode(pos), oracle.f16_decode(pos + 1)
    mid = (a + b) / 2                                       # exact in binary64
    even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
    assert np.array_equal(oracle.f16_round(mid), even)
    assert np.array_equal(oracle.f16_round(np.nextafter(mid, np.inf)), pos + 1)
    assert np.array_equal(oracle.f16_round(np.nextafter(mid, -np.inf)), pos)
    assert np.array_equal(oracle.f16_round(-mid), even | 0x8000)


def test_overflow_and_special_values():
    r = lambda v: int(oracle.f16_round(np.array([v]))[0])
    assert r(65504.0) == 0x7BFF and r(np.nextafter(65520.0, 0)) == 0x7BFF
    assert r(65520.0) == 0x7C00 and r(1e6) == 0x7C00 and r(-65520.0) == 0xFC00
    assert r(np.inf) == 0x7C00 and r(-np.inf) == 0xFC00
    assert r(np.nan) == 0x7E00 and r(-np.nan) == 0xFE00
    assert r(0.0) == 0x0000 and r(-0.0) == 0x8000
    assert r(2.0 ** -24) == 0x0001 and r(2.0 ** -25) == 0x0000          # tie to even (zero)
    assert r(2.0 ** -25 * (1 + 2.0 ** -30)) == 0x0001 and r(-(2.0 ** -26)) == 0x8000
    assert r(3 * 2.0 ** -25) == 0x0002                                  # tie between 1 and 2
    assert r(2.0 ** -14) == 0x0400 and r(2.0 ** -14 - 2.0 ** -25) == 0x0400
    assert r(1.0) == 0x3C00 and r(1.0 + 2.0 ** -11) == 0x3C00 and r(1.0 + 3 * 2.0 ** -11) == 0x3C02


def test_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(400000) * 10.0 ** rng.uniform(-10, 6, 400000)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_round(v), ref)


def test_matches_torch_float32_conversion():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = [0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x7FFF, 0x8000, 0xFFFF]
    f = np.concatenate([hi | np.uint32(lo) for lo in lows]).view(np.float32)
    f = f[~np.isnan(f)]
    ours = oracle.f16_round(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_float16_forwards_compose_the_definitions():
    """residual_out = binary16(binary32(x) + binary32(r)), composed with
    numpy; y = RMSNorm(residual_out) * w in binary64 (torch's rms_norm on the
    CPU), rounded once to binary16; float32 rstd."""
    inp = synth.add_rmsnorm_fwd_inputs(37, 1000, torch.float16, seed=3, r_std=0.5)
    x, r, w = inp["x"], inp["r"], inp["w"]
    y, res, rstd = oracle.add_rmsnorm_fwd(x, r, w, 1e-6)
    want_res = (x.numpy().astype(np.float32) + r.numpy().astype(np.float32)).astype(np.float16)
    assert np.array_equal(res.numpy().view(np.uint16), want_res.view(np.uint16))
    h = res.double()
    y64 = torch.nn.functional.rms_norm(h, (1000,), w.double(), eps=float(np.float32(1e-6)))
    assert np.array_equal(y.numpy().view(np.uint16), oracle.f16_round(y64.numpy()))
    rs = 1.0 / torch.sqrt((h * h).mean(-1) + float(np.float32(1e-6)))
    np.testing.assert_allclose(rstd.numpy(), rs.numpy(), rtol=2.0 ** -23, atol=0)
    # the plain forward and the backward take float16 tensors too
    y2, _ = oracle.rmsnorm_fwd(res, w, 1e-6)
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    dy = synth.store(synth.normal(4, "dy", (37, 1000)), torch.float16)
    dx, dw, _ = oracle.rmsnorm_bwd(dy, res, w, rstd)
    assert dx.dtype == torch.float16 and dw.dtype == torch.float32
    g = dy.double() * w.double()
    xh = res.double() * rstd.double()[:, None]
    c = (g * xh).mean(-1, keepdim=True)
    dx64 = rstd.double()[:, None] * (g - xh * c)
    assert np.array_equal(dx.numpy().view(np.uint16), oracle.f16_round(dx64.numpy()))
