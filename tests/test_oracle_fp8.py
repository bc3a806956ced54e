"""Pins for the oracle's E4M3 encoding and the FP8-output RMSNorm (CPU only).

The encoder is checked against torch's float32 -> float8_e4m3fn conversion
(round-to-nearest-even) wherever torch does not overflow (|v| < 464), against
a brute-force nearest-value search over the table of all finite E4M3 values
in exact rational arithmetic (ties, subnormals, saturation), and by the
round trip of every code.  The row quantisation is checked against the
binary64 RMSNorm (torch-pinned elsewhere): the largest element encodes as
+-448, every value is recovered within half an E4M3 step times the scale, and
the special rows (zero, NaN) follow the stated rules."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _table():
    """All non-negative finite E4M3 values, indexed by code 0x00..0x7E."""
    return np.array([oracle.fp8e4m3_decode([c])[0] for c in range(0x7F)])


def _brute(v: float, table: np.ndarray) -> int:
    if np.isnan(v):
        return -1
    sign = 0x80 if np.signbit(v) else 0
    a = abs(v)
    if a >= 448:
        return sign | 0x7E
    k = int(np.searchsorted(table, a, side="right")) - 1
    if table[k] == a:
        return sign | k
    lo, hi, A = Fraction(table[k]), Fraction(table[k + 1]), Fraction(a)
    if A - lo < hi - A:
        return sign | k
    if hi - A < A - lo:
        return sign | (k + 1)
    return sign | (k if k % 2 == 0 else k + 1)


def test_table_is_monotone_and_spans_the_format():
    t = _table()
    assert t[0] == 0 and t[1] == 2.0 ** -9 and t[8] == 2.0 ** -6 and t[-1] == 448.0
    assert np.all(np.diff(t) > 0)


def test_matches_torch_float8_e4m3fn_where_torch_is_in_range():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xABCD]
    f = np.concatenate([hi | np.uint32(lo) for lo in lows]).view(np.float32)
    with np.errstate(invalid="ignore"):
        keep = np.isnan(f) | (np.abs(f) < 464.0)
    f = f[keep]
    with np.errstate(invalid="ignore"):  # signalling NaN patterns raise the flag when widened
        ours = oracle.fp8e4m3_encode(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = np.isnan(f)
    assert np.all((ours[nan] & 0x7F) == 0x7F)
    bad = np.nonzero(ours[~nan] != ref[~nan])[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {f[~nan][bad[:5]]}"


def test_brute_force_grid_search():
    t = _table()
    rng = np.random.default_rng(123)
    vals = list(np.sign(rng.standard_normal(4000)) * np.exp2(rng.uniform(-12, 10, 4000)))
    k = rng.integers(0, t.size - 1, 500)
    mids = (t[k] + t[k + 1]) / 2
    vals += list(mids) + list(np.nextafter(mids, 0)) + list(np.nextafter(mids, np.inf))
    vals += [0.0, -0.0, 448.0, 447.9, 464.0, 500.0, 1e30, -np.inf, np.inf, 2.0 ** -10,
             2.0 ** -11, 3 * 2.0 ** -11, 2.0 ** -6, np.nextafter(2.0 ** -6, 0)]
    vals = np.array(vals)
    ours = oracle.fp8e4m3_encode(vals)
    for v, o in zip(vals, ours):
        assert int(o) == _brute(float(v), t), f"v={v!r}: got {int(o):#04x}"


def test_round_trip_of_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.fp8e4m3_decode(codes)
    back = oracle.fp8e4m3_encode(vals)
    assert np.array_equal(back, codes)
    assert all(np.isnan(oracle.fp8e4m3_decode([0x7F, 0xFF])))


@pytest.mark.parametrize("fused", [False, True])
def test_row_quantisation(fused):
    M, N = 64, 1000
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=201)
    x, r, w = inp["x"], inp["r"], inp["w"]
    if fused:
        q, scale, res, rstd = oracle.rmsnorm_fwd_fp8(x, w, 1e-6, residual=r)
        _, res_ref, _ = oracle.add_rmsnorm_fwd(x, r, w, 1e-6)
        assert torch.equal(res.view(torch.int16), res_ref.view(torch.int16))
        y64, _ = oracle.rmsnorm_fwd(res, w, 1e-6, y_dtype=torch.float64)
    else:
        q, scale, rstd = oracle.rmsnorm_fwd_fp8(x, w, 1e-6)
        y64, _ = oracle.rmsnorm_fwd(x, w, 1e-6, y_dtype=torch.float64)
    y = y64.numpy()
    qn = q.numpy()
    s = scale.numpy().astype(np.float64)
    amax = np.abs(y).max(axis=1)
    np.testing.assert_allclose(s * 448.0, amax, rtol=1e-6)
    arg = np.abs(y).argmax(axis=1)
    assert np.all((qn[np.arange(M), arg] & 0x7F) == 0x7E)
    deq = oracle.fp8e4m3_decode(qn) * s[:, None]
    # half an E4M3 step at the value's magnitude (3 mantissa bits), or half the
    # subnormal step, times the scale, plus float32 slack
    mag = np.abs(y) / s[:, None]
    step = np.where(mag < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-30))) - 3))
    assert np.all(np.abs(deq - y) <= (0.5 * step * (1 + 1e-6) + 1e-6 * mag) * s[:, None])


def test_special_rows():
    N = 32
    w = torch.ones(N, dtype=torch.bfloat16)
    x = torch.zeros(3, N, dtype=torch.bfloat16)
    x[1, 5] = float("nan")
    x[2] = 1.0
    q, scale, _ = oracle.rmsnorm_fwd_fp8(x, w, 1e-6)
    assert scale[0].item() == 1.0 and torch.all(q[0] == 0)
    assert scale[1].item() == 1.0 and torch.all((q[1] & 0x7F) == 0x7F)   # NaN row
    assert torch.all(q[2] == 0x7E)                                       # constant row: all amax


# ---- one scale per group of columns -----------------------------------------

def test_group_of_the_whole_row_is_the_per_row_scale():
    M, N = 16, 300
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=301)
    q0, s0, _ = oracle.rmsnorm_fwd_fp8(inp["x"], inp["w"], 1e-6)
    for g in (N, N + 5):
        q1, s1, _ = oracle.rmsnorm_fwd_fp8(inp["x"], inp["w"], 1e-6, group=g)
        assert torch.equal(q0, q1) and torch.equal(s0, s1.reshape(M))


def test_constant_groups_have_closed_form_scales():
    # one row: 128 columns of a, 128 of b, a ragged last group of 44 columns of c
    a, b, c = 3.0, -0.25, 40.0
    x = torch.tensor([[a] * 128 + [b] * 128 + [c] * 44], dtype=torch.float64)
    w = torch.ones(300, dtype=torch.float64)
    q, s, rstd = oracle.rmsnorm_fwd_fp8(x, w, 0.0, group=128, eps_exact=True)
    assert s.shape == (1, 3)
    rs = 1.0 / np.sqrt((128 * a * a + 128 * b * b + 44 * c * c) / 300)
    for k, v in enumerate((a, b, c)):
        assert s[0, k].item() == np.float32(np.abs(v * rs) / 448.0)
    # every value is its group's maximum: the codes are +-448
    qn = q.numpy()[0]
    assert np.all(qn[:128] == 0x7E) and np.all(qn[128:256] == 0xFE) and np.all(qn[256:] == 0x7E)


def test_groups_of_one_column():
    M, N = 3, 64
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.float32, seed=303)
    x = inp["x"].clone()
    x[1, 7] = 0.0
    q, s, _ = oracle.rmsnorm_fwd_fp8(x, inp["w"], 1e-6, group=1)
    y, _ = oracle.rmsnorm_fwd(x, inp["w"], 1e-6, y_dtype=torch.float64)
    y = y.numpy()
    np.testing.assert_array_equal(s.numpy(), np.where(y == 0, np.float32(1),
                                                      (np.abs(y) / 448.0).astype(np.float32)))
    qn = q.numpy()
    assert qn[1, 7] == 0
    nz = y != 0
    assert np.all((qn[nz] & 0x7F) == 0x7E) and np.all((qn[nz] >> 7) == (y[nz] < 0))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("N,group", [(1000, 128), (7168, 128), (300, 32)])
def test_grouped_quantisation(fused, N, group):
    M = 24
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=N + group)
    x, r, w = inp["x"], inp["r"], inp["w"]
    if fused:
        q, scale, res, _ = oracle.rmsnorm_fwd_fp8(x, w, 1e-6, residual=r, group=group)
        _, res_ref, _ = oracle.add_rmsnorm_fwd(x, r, w, 1e-6)
        assert torch.equal(res.view(torch.int16), res_ref.view(torch.int16))
        y64, _ = oracle.rmsnorm_fwd(res, w, 1e-6, y_dtype=torch.float64)
    else:
        q, scale, _ = oracle.rmsnorm_fwd_fp8(x, w, 1e-6, group=group)
        y64, _ = oracle.rmsnorm_fwd(x, w, 1e-6, y_dtype=torch.float64)
    ng = (N + group - 1) // group
    assert scale.shape == (M, ng)
    y = y64.numpy()
    s = scale.numpy().astype(np.float64)
    cols = np.arange(N) // group
    sg = s[:, cols]                                   # each element's own scale
    qn = q.numpy()
    for g in range(ng):
        blk = slice(g * group, min(N, (g + 1) * group))
        amax = np.abs(y[:, blk]).max(axis=1)
        np.testing.assert_allclose(s[:, g] * 448.0, amax, rtol=1e-6)
        # the group's largest value encodes as +-448
        assert np.all((qn[:, blk] & 0x7F).max(axis=1) == 0x7E)
    deq = oracle.fp8e4m3_decode(qn) * sg
    mag = np.abs(y) / sg
    step = np.where(mag < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-30))) - 3))
    assert np.all(np.abs(deq - y) <= (0.5 * step * (1 + 1e-6) + 1e-6 * mag) * sg)
