"""Pins of the oracle's MXFP4 output (CPU only).

MXFP4 is named, not defined, on the pages (the "Machete" README lists MXFP4
decode kernels in "Built-In Areas"). The definition used is OCP Microscaling
Formats v1.0:
- FP4 E2M1 elements, nearest rounding with ties to the even code, saturating
  at +-6;
- one E8M0 power-of-two scale 2^E per block of 32 values, with
  E = floor(log2(max |y|)) - 2.

The oracle is checked against:
- a brute-force nearest search over the E2M1 grid in exact rational
  arithmetic;
- the round trip of every code;
- the defining property of E, 4 <= amax / 2^E < 8 (or the clamp);
- hand-derived rows;
- the error bound of every element;
- special blocks: zero, NaN, ragged;
- the fused form."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def brute_e2m1(v: float) -> int:
    """Nearest grid magnitude to |v| (exact), ties to the even code; > 6 -> 6."""
    a = abs(Fraction(v))
    sign = 0x8 if np.signbit(v) else 0
    if a >= 6:
        return sign | 7
    best = min(range(8), key=lambda k: (abs(GRID[k] - a), k % 2))
    return sign | best


def test_encoder_matches_brute_force():
    vals = []
    for k in range(8):
        g = float(GRID[k])
        vals += [g, -g, np.nextafter(g, 0), np.nextafter(g, 10)]
        if k < 7:
            mid = float((GRID[k] + GRID[k + 1]) / 2)
            vals += [mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, 10)]
    vals += [6.0001, 7.999, 8.0, 1e30, -1e30, 1e-30, -1e-30, 0.0, -0.0]
    vals += list(synth.normal(5, "fp4", (2000,), std=4.0))
    got = oracle.fp4e2m1_encode(vals)
    want = np.array([brute_e2m1(v) for v in vals], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(vals[i], got[i], want[i]) for i in bad[:5]]


def test_every_code_round_trips():
    for c in range(16):
        v = oracle.fp4e2m1_decode(np.array([c], dtype=np.uint8))[0]
        assert oracle.fp4e2m1_encode([v])[0] == c
    assert list(oracle.fp4e2m1_decode(np.arange(8, dtype=np.uint8))) == [float(g) for g in GRID]


def _split(q, scale, N):
    codes = oracle.unpack_fp4(q)
    s = scale.numpy().astype(np.int64)
    return codes, s


def test_hand_derived_rows():
    # x = [2]*32 + [-2]*32, w = 1, eps = 0: rstd = 1/2, y = +-1; amax 1 ->
    # E = -2 (scale code 125), y / 2^-2 = +-4: codes 6 and 14 (0x66, 0xEE)
    x = torch.tensor([[2.0] * 32 + [-2.0] * 32], dtype=torch.float64)
    w = torch.ones(64, dtype=torch.float64)
    q, s, rstd = oracle.rmsnorm_fwd_mxfp4(x, w, 0.0, eps_exact=True)
    assert rstd.item() == 0.5
    assert s.tolist() == [[125, 125]]
    assert torch.all(q[0, :16] == 0x66) and torch.all(q[0, 16:] == 0xEE)
    # x = [16, 0 x 63]: rstd = 1/2, y0 = 8 -> E = 3 - 2 = 1 (code 128), 8 / 2 = 4
    # (code 6); the second block is all zero -> E = -127 (code 0), codes 0
    x = torch.zeros(1, 64, dtype=torch.float64)
    x[0, 0] = 16.0
    q, s, _ = oracle.rmsnorm_fwd_mxfp4(x, w, 0.0, eps_exact=True)
    assert s.tolist() == [[128, 0]]
    assert q[0, 0].item() == 0x06 and torch.all(q[0, 1:] == 0)
    # saturation: x = [14] + [2]*15 + [0]*48, sum x^2 = 196 + 60 = 256 = 4 * 64,
    # so rstd = 1/2 and y = [7] + [1]*15 + [0]*48.  Block 0: amax 7 -> E = 0
    # (code 127); 7 saturates to 6 (code 7), 1 is code 2.  Block 1 is zero.
    x = torch.tensor([[14.0] + [2.0] * 15 + [0.0] * 48], dtype=torch.float64)
    q, s, rstd = oracle.rmsnorm_fwd_mxfp4(x, w, 0.0, eps_exact=True)
    assert rstd.item() == 0.5 and s.tolist() == [[127, 0]]
    assert q[0, 0].item() == 0x27 and torch.all(q[0, 1:8] == 0x22) and torch.all(q[0, 8:] == 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N", [32, 48, 1024, 7168])
def test_scale_rule_and_error_bound(dtype, N):
    M = 20
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, seed=N + 3)
    x, w = inp["x"], inp["w"]
    x[3] *= 1e-30 if dtype == torch.float32 else 1.0      # a row of tiny values
    q, s, _ = oracle.rmsnorm_fwd_mxfp4(x, w, 1e-6)
    y64, _ = oracle.rmsnorm_fwd(x, w, 1e-6, y_dtype=torch.float64)
    yf = y64.numpy().astype(np.float32).astype(np.float64)
    codes, sc = _split(q, s, N)
    nb = (N + 31) // 32
    assert sc.shape == (M, nb) and codes.shape == (M, N)
    E = sc - 127
    for b in range(nb):
        blk = slice(32 * b, min(N, 32 * (b + 1)))
        amax = np.abs(yf[:, blk]).max(axis=1)
        ratio = amax * np.exp2(-E[:, b].astype(np.float64))
        # the defining property of E: the block maximum lands in [4, 8), unless
        # E is clamped at -127 (tiny or zero blocks)
        clamped = E[:, b] == -127
        assert np.all(clamped | ((ratio >= 4) & (ratio < 8))), (b, ratio[~clamped])
        assert np.all(~clamped | (ratio < 8))
        X = np.exp2(E[:, b].astype(np.float64))[:, None]
        v = yf[:, blk] / X
        deq = oracle.fp4e2m1_decode(codes[:, blk])
        # nearest on the grid: within half the local spacing, or saturated at 6
        spacing = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
        sat = np.abs(v) > 6
        assert np.all(sat | (np.abs(deq - v) <= spacing / 2))
        assert np.all(~sat | (deq == np.sign(v) * 6))


def test_special_blocks():
    N = 96
    w = torch.ones(N, dtype=torch.float32)
    x = torch.zeros(3, N, dtype=torch.float32)
    x[1] = synth.store(synth.normal(9, "x", (N,)), torch.float32)
    x[1, 40] = float("nan")                  # NaN: the whole row is NaN
    x[2] = synth.store(synth.normal(10, "x", (N,)), torch.float32)
    q, s, _ = oracle.rmsnorm_fwd_mxfp4(x, w, 1e-6)
    assert s[0].tolist() == [0, 0, 0] and torch.all(q[0] == 0)    # zero row: E = -127
    assert s[1].tolist() == [255, 255, 255] and torch.all(q[1] == 0)
    assert torch.all(s[2] != 255) and torch.all(s[2] > 100)


def test_fused_form():
    M, N = 16, 256
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=13)
    q, s, res, _ = oracle.rmsnorm_fwd_mxfp4(inp["x"], inp["w"], 1e-6, residual=inp["r"])
    _, res_ref, _ = oracle.add_rmsnorm_fwd(inp["x"], inp["r"], inp["w"], 1e-6)
    assert torch.equal(res.view(torch.int16), res_ref.view(torch.int16))
    q2, s2, _ = oracle.rmsnorm_fwd_mxfp4(res, inp["w"], 1e-6)
    assert torch.equal(q, q2) and torch.equal(s, s2)
