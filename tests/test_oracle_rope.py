"""Pins of the oracle's per-head RMSNorm + RoPE (CPU only).

The composition is RMSNorm over each head's D values, then the rotary
position embedding of the normalised pairs (RoFormer, Su et al. 2021). The
"Machete" README lists RMSNorm and RoPE side by side in "Built-In Areas". The
oracle is checked against things other than itself:
- hand-derived rational cases (tests/golden/closed_form_cases.json);
- torch's float64 rms_norm followed by numpy complex multiplication (a pair
  (a, b) is the complex number a + ib, rotated by e^{i*angle});
- the rotation's invariants: pair norms are kept, and the dot product of a
  rotated query and key depends only on the difference of their positions;
- views of a packed projection buffer, which give the same bits as contiguous
  copies;
- positions outside the table, which give NaN heads."""
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


rope_table = synth.rope_table


def complex_reference(x, w, cos, sin, pos, eps, interleaved):
    """torch float64 rms_norm, then each pair times e^{i*angle} in numpy complex128."""
    D = x.shape[-1]
    n = F.rms_norm(x.double(), (D,), w.double(), oracle.eps_as_float32(eps)).numpy()
    rot = (cos.double().numpy() + 1j * sin.double().numpy())[pos.numpy()][:, None, :]
    if interleaved:
        z = (n[..., 0::2] + 1j * n[..., 1::2]) * rot
        out = np.empty_like(n)
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    else:
        z = (n[..., :D // 2] + 1j * n[..., D // 2:]) * rot
        out = np.concatenate([z.real, z.imag], axis=-1)
    return out


def heads(T, H, D, dtype, seed):
    return synth.store(synth.normal(seed, "x", (T, H, D)), dtype)


def test_golden_cases():
    for c in json.load(open(GOLDEN))["rmsnorm_rope"]:
        D = len(c["x"])
        fr = lambda v: float(Fraction(str(v)))
        x = torch.tensor([[[fr(v) for v in c["x"]]]], dtype=torch.float64)
        w = torch.tensor([fr(v) for v in c["w"]], dtype=torch.float64)
        cos = torch.tensor([[fr(v) for v in row] for row in c["cos"]], dtype=torch.float32)
        sin = torch.tensor([[fr(v) for v in row] for row in c["sin"]], dtype=torch.float32)
        assert cos.shape == (2, D // 2)
        y = oracle.rmsnorm_rope(x, w, cos, sin, torch.tensor([c["pos"]]), fr(c["eps"]),
                                interleaved=c["interleaved"], eps_exact=True)
        want = [float(Fraction(v)) for v in c["y"]]
        assert y[0, 0].tolist() == pytest.approx(want, rel=1e-15, abs=1e-16), c["name"]


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float64, 64), (torch.float32, 6)])
def test_matches_complex_rotation_of_torch_rms_norm(interleaved, dtype, D):
    T, H, P = 9, 3, 4096
    x = heads(T, H, D, dtype, 11)
    w = synth.weight(11, D, dtype)
    cos, sin = rope_table(P, D)
    pos = synth.positions(11, T, P)
    y = oracle.rmsnorm_rope(x, w, cos, sin, pos, 1e-6, interleaved=interleaved,
                            y_dtype=torch.float64)
    ref = complex_reference(x, w, cos, sin, pos, 1e-6, interleaved)
    np.testing.assert_allclose(y.numpy(), ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_keeps_pair_norms(interleaved):
    T, H, D, P = 16, 2, 32, 1000
    x = heads(T, H, D, torch.float64, 13)
    w = synth.weight(13, D, torch.float64)
    cos, sin = rope_table(P, D)
    pos = torch.arange(0, 16 * 61, 61)
    y = oracle.rmsnorm_rope(x, w, cos, sin, pos, 1e-6, interleaved=interleaved).numpy()
    n = F.rms_norm(x, (D,), w, oracle.eps_as_float32(1e-6)).numpy()
    pair = (lambda v: v[..., 0::2] ** 2 + v[..., 1::2] ** 2) if interleaved else \
        (lambda v: v[..., :D // 2] ** 2 + v[..., D // 2:] ** 2)
    unit = (cos.double() ** 2 + sin.double() ** 2).numpy()[pos.numpy()][:, None, :]
    np.testing.assert_allclose(pair(y), pair(n) * unit, rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("interleaved", [False, True])
def test_dot_product_depends_on_position_difference_only(interleaved):
    D, P = 64, 8192
    cos, sin = rope_table(P, D)
    q = heads(1, 1, D, torch.float64, 17)
    k = heads(1, 1, D, torch.float64, 18)
    wq, wk = synth.weight(17, D, torch.float64), synth.weight(18, D, torch.float64)

    def rot(v, w, p):
        return oracle.rmsnorm_rope(v.expand(len(p), 1, D).contiguous(), w, cos, sin,
                                   torch.tensor(p), 1e-6, interleaved=interleaved)[:, 0].numpy()

    for m, n in [(5, 2), (100, 37), (4000, 3999), (17, 900)]:
        shifts = [0, 1, 250, 3000]
        dots = [float(rot(q, wq, [m + s])[0] @ rot(k, wk, [n + s])[0]) for s in shifts]
        scale = float(np.linalg.norm(rot(q, wq, [0])) * np.linalg.norm(rot(k, wk, [0])))
        # float32 tables: each entry is within 2^-24 relative of the true cos/sin
        assert max(dots) - min(dots) <= 1e-6 * scale, (m, n, dots)
    # the same position: the rotation cancels, leaving the normalised dot product
    same = float(rot(q, wq, [1234])[0] @ rot(k, wk, [1234])[0])
    plain = float(rot(q, wq, [0])[0] @ rot(k, wk, [0])[0])
    assert abs(same - plain) <= 1e-6 * scale


def test_views_of_a_packed_projection_buffer():
    T, Hq, Hk, D = 7, 4, 2, 64
    qkv = synth.store(synth.normal(19, "x", (T, (Hq + 2 * Hk) * D)), torch.bfloat16)
    q = qkv[:, :Hq * D].view(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D)
    assert q.stride(0) == (Hq + 2 * Hk) * D
    cos, sin = rope_table(512, D)
    pos = torch.tensor([0, 3, 3, 100, 511, 7, 8])
    w = synth.weight(19, D, torch.bfloat16)
    for v in (q, k):
        a = oracle.rmsnorm_rope(v, w, cos, sin, pos, 1e-6)
        b = oracle.rmsnorm_rope(v.contiguous(), w, cos, sin, pos, 1e-6)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_position_zero_is_the_plain_norm_and_rounding_is_single():
    T, H, D = 5, 3, 128
    x = heads(T, H, D, torch.bfloat16, 23)
    w = synth.weight(23, D, torch.bfloat16)
    cos, sin = rope_table(16, D)
    y = oracle.rmsnorm_rope(x, w, cos, sin, torch.zeros(T, dtype=torch.int64), 1e-6)
    yn, _ = oracle.rmsnorm_fwd(x.reshape(T * H, D), w, 1e-6)
    assert torch.equal(y.reshape(T * H, D).view(torch.int16), yn.view(torch.int16))
    # at other positions the bf16 output is the binary64 result rounded once
    pos = torch.tensor([1, 2, 3, 9, 15])
    y = oracle.rmsnorm_rope(x, w, cos, sin, pos, 1e-6)
    y64 = oracle.rmsnorm_rope(x, w, cos, sin, pos, 1e-6, y_dtype=torch.float64)
    assert torch.equal(y.view(torch.int16), y64.to(torch.bfloat16).view(torch.int16))


def test_positions_outside_the_table_give_nan_heads():
    T, H, D, P = 4, 2, 16, 10
    x = heads(T, H, D, torch.float32, 29)
    w = synth.weight(29, D, torch.float32)
    cos, sin = rope_table(P, D)
    y = oracle.rmsnorm_rope(x, w, cos, sin, torch.tensor([-1, P, 0, P - 1]), 1e-6)
    assert torch.all(torch.isnan(y[:2])) and not torch.any(torch.isnan(y[2:]))
    ref = oracle.rmsnorm_rope(x[2:], w, cos, sin, torch.tensor([0, P - 1]), 1e-6)
    assert torch.equal(y[2:], ref)


def test_two_dimensional_heads_pair_the_same_way_in_both_layouts():
    x = heads(6, 2, 2, torch.float64, 31)
    w = synth.weight(31, 2, torch.float64)
    cos, sin = rope_table(64, 2)
    pos = torch.tensor([0, 1, 5, 20, 33, 63])
    a = oracle.rmsnorm_rope(x, w, cos, sin, pos, 1e-6, interleaved=False)
    b = oracle.rmsnorm_rope(x, w, cos, sin, pos, 1e-6, interleaved=True)
    assert torch.equal(a, b)
