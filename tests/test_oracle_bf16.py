"""Pins for the oracle's bfloat16 rounding (CPU only).

The oracle's converter is checked against two things other than itself:
torch's own float32 -> bfloat16 conversion (round-to-nearest-even), over every
bfloat16 upper half combined with every rounding-relevant lower half; and a
brute-force nearest-value search over the table of all finite bfloat16 values
with exact rational arithmetic, for binary64 inputs (the single rounding the
oracle applies to its binary64 results)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _f32_from_bits(bits: np.ndarray) -> np.ndarray:
    return bits.astype(np.uint32).view(np.float32)


def test_f32_to_bf16_matches_torch_structured_sweep():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    rng = np.random.default_rng(1234)
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF] + list(
        rng.integers(0, 1 << 16, size=6))
    bits = np.concatenate([hi | np.uint32(lo) for lo in lows])
    f = _f32_from_bits(bits)
    with np.errstate(invalid="ignore"):
        ours = oracle.bf16_round(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    # NaN: both must be NaN (payloads are not part of the contract), sign kept by ours.
    ours_nan = ((ours & 0x7F80) == 0x7F80) & ((ours & 0x007F) != 0)
    assert np.array_equal(ours_nan, nan)
    assert np.array_equal(ours[nan] >> 15, (bits[nan] >> 31).astype(np.uint16))
    mism = np.nonzero(ours[~nan] != ref[~nan])[0]
    assert mism.size == 0, f"{mism.size} mismatches, first bits {bits[~nan][mism[:5]]}"


def _bf16_table():
    pos = np.arange(0x0000, 0x7F80, dtype=np.uint32) << 16  # all finite non-negative
    return pos.view(np.float32).astype(np.float64)


def _brute_bf16(v: float, table: np.ndarray) -> int:
    """Nearest bfloat16 to v, ties to even significand, by exact comparison."""
    if np.isnan(v):
        return -1
    sign = 0x8000 if np.signbit(v) else 0
    a = abs(v)
    bf16_max = Fraction(table[-1])
    half_ulp_top = Fraction(2) ** 119
    if np.isinf(a) or Fraction(a) >= bf16_max + half_ulp_top:
        return sign | 0x7F80
    k = int(np.searchsorted(table, a, side="right")) - 1  # table[k] <= a
    if table[k] == a or k == table.size - 1:
        return sign | k
    lo, hi = Fraction(table[k]), Fraction(table[k + 1])
    A = Fraction(a)
    if A - lo < hi - A:
        return sign | k
    if hi - A < A - lo:
        return sign | (k + 1)
    return sign | (k if k % 2 == 0 else k + 1)


def test_f64_to_bf16_single_rounding_brute_force():
    table = _bf16_table()
    rng = np.random.default_rng(99)
    vals = []
    # random magnitudes over the whole range, subnormals included
    e = rng.uniform(-140, 129, size=3000)
    vals += list(np.sign(rng.standard_normal(3000)) * np.exp2(e) * rng.uniform(1, 2, 3000))
    # exact midpoints between neighbours and their binary64 neighbours
    idx = rng.integers(0, table.size - 1, size=1500)
    mids = (table[idx] + table[idx + 1]) / 2
    vals += list(mids) + list(np.nextafter(mids, 0)) + list(np.nextafter(mids, np.inf))
    # values that double rounding through binary32 would get wrong: just above a
    # bfloat16 midpoint by less than half a binary32 ulp
    vals += list(mids * (1 + 2.0 ** -30))
    vals += [0.0, -0.0, 1.0, -1.0, float(table[-1]), 2.0 ** 128 - 2.0 ** 119,
             np.nextafter(2.0 ** 128 - 2.0 ** 119, 0), 1e300, -1e300, 5e-324, 2.0 ** -133,
             2.0 ** -134, 3 * 2.0 ** -135, np.inf, -np.inf]
    vals = np.array(vals, dtype=np.float64)
    ours = oracle.bf16_round(vals)
    for v, o in zip(vals, ours):
        want = _brute_bf16(float(v), table)
        assert int(o) == want, f"v={v!r}: got {int(o):#06x} want {want:#06x}"


def test_f64_nan_is_quiet_nan():
    out = oracle.bf16_round(np.array([np.nan, -np.nan]))
    assert all(((o & 0x7F80) == 0x7F80) and (o & 0x0040) for o in out)


def test_residual_rounding_worked_examples():
    """Hand-derived residual sums (golden file) through the oracle's fused op."""
    cases = json.load(open(GOLDEN))["residual_rounding_bf16"]
    for c in cases:
        x = torch.tensor([int(c["x_bits"], 16)], dtype=torch.int32).to(torch.int16).view(
            torch.bfloat16).reshape(1, 1)
        r = torch.tensor([int(c["r_bits"], 16)], dtype=torch.int32).to(torch.int16).view(
            torch.bfloat16).reshape(1, 1)
        w = torch.ones(1, dtype=torch.bfloat16)
        _, res, _ = oracle.add_rmsnorm_fwd(x, r, w, 1e-6)
        got = int(res.view(torch.int16).item()) & 0xFFFF
        assert got == int(c["res_bits"], 16), c["name"]
