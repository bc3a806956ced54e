"""Pins for the oracle's LayerNorm (CPU only): torch float64 layer_norm and
its autograd (library routines), hand-derived rational worked examples
(tests/golden), central finite differences, closed forms (constant rows give
the bias; zero mean and unit variance for w = 1, b = 0), the exact
power-of-two scale identity, the residual add, and the backward's identities
sum_j dx_j = 0 and sum_j xh_j dx_j = N eps rstd^3 mean_j(g_j xh_j)."""
import json
import os
from fractions import Fraction

import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")
Q = lambda v: float(Fraction(str(v)))


def _case(M, N, seed, bias=True):
    x = synth.store(synth.normal(seed, "x", (M, N), mean=0.5), torch.float64)
    dy = synth.store(synth.normal(seed, "dy", (M, N)), torch.float64)
    w = synth.weight(seed, N, torch.float64)
    b = synth.store(synth.normal(seed, "r", (N,), std=0.1), torch.float64) if bias else None
    return x, dy, w, b


@pytest.mark.parametrize("M,N", [(1, 1), (3, 2), (5, 17), (4, 300)])
@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("eps", [1e-5, 0.2])
def test_forward_matches_torch_float64(M, N, bias, eps):
    x, _, w, b = _case(M, N, 81, bias)
    y, mean, rstd = oracle.layernorm_fwd(x, w, b, eps, eps_exact=True, stat_dtype=torch.float64)
    torch.testing.assert_close(y, F.layer_norm(x, (N,), w, b, eps), rtol=1e-12, atol=1e-13)
    torch.testing.assert_close(mean, x.mean(-1), rtol=1e-14, atol=1e-15)
    torch.testing.assert_close(rstd, torch.rsqrt(x.var(-1, unbiased=False) + eps), rtol=1e-12,
                               atol=0)


@pytest.mark.parametrize("M,N", [(1, 2), (3, 17), (6, 128)])
@pytest.mark.parametrize("eps", [1e-5, 0.2])
def test_backward_matches_torch_autograd_float64(M, N, eps):
    x, dy, w, b = _case(M, N, 83)
    _, mean, rstd = oracle.layernorm_fwd(x, w, b, eps, eps_exact=True, stat_dtype=torch.float64)
    dx, dw, db, _, _ = oracle.layernorm_bwd(dy, x, w, mean, rstd, dwb_dtype=torch.float64)
    xr, wr, br = (t.clone().requires_grad_(True) for t in (x, w, b))
    F.layer_norm(xr, (N,), wr, br, eps).backward(dy)
    torch.testing.assert_close(dx, xr.grad, rtol=1e-10, atol=1e-12)
    torch.testing.assert_close(dw, wr.grad, rtol=1e-11, atol=1e-12)
    torch.testing.assert_close(db, br.grad, rtol=1e-12, atol=1e-13)


def test_golden_cases():
    g = json.load(open(GOLDEN))
    for c in g["layernorm_forward"]:
        x = torch.tensor([[Q(v) for v in c["x"]]], dtype=torch.float64)
        w = torch.tensor([Q(v) for v in c["w"]], dtype=torch.float64)
        b = torch.tensor([Q(v) for v in c["b"]], dtype=torch.float64)
        y, mean, rstd = oracle.layernorm_fwd(x, w, b, Q(c["eps"]), eps_exact=True,
                                             stat_dtype=torch.float64)
        assert mean.item() == Q(c["mean"]) and rstd.item() == Q(c["rstd"]), c["name"]
        assert y[0].tolist() == pytest.approx([Q(v) for v in c["y"]], rel=1e-15, abs=1e-16)
    for c in g["layernorm_backward"]:
        x = torch.tensor([[Q(v) for v in c["x"]]], dtype=torch.float64)
        w = torch.tensor([Q(v) for v in c["w"]], dtype=torch.float64)
        dy = torch.tensor([[Q(v) for v in c["dy"]]], dtype=torch.float64)
        _, mean, rstd = oracle.layernorm_fwd(x, w, None, Q(c["eps"]), eps_exact=True,
                                             stat_dtype=torch.float64)
        dx, dw, db, _, _ = oracle.layernorm_bwd(dy, x, w, mean, rstd, dwb_dtype=torch.float64)
        assert dx[0].tolist() == pytest.approx([Q(v) for v in c["dx"]], rel=1e-15, abs=1e-16)
        assert dw.tolist() == pytest.approx([Q(v) for v in c["dw"]], rel=1e-15, abs=1e-16)
        assert db.tolist() == pytest.approx([Q(v) for v in c["db"]], rel=1e-15, abs=1e-16)


@pytest.mark.parametrize("M,N", [(1, 2), (2, 3), (1, 9)])
def test_finite_differences(M, N):
    eps, h = 1e-3, 1e-6
    x, dy, w, b = _case(M, N, 87)

    def loss(xx, ww, bb):
        y, _, _ = oracle.layernorm_fwd(xx, ww, bb, eps, eps_exact=True)
        return float((y * dy).sum())

    _, mean, rstd = oracle.layernorm_fwd(x, w, b, eps, eps_exact=True, stat_dtype=torch.float64)
    dx, dw, db, _, _ = oracle.layernorm_bwd(dy, x, w, mean, rstd, dwb_dtype=torch.float64)
    for name, t, g in (("x", x, dx), ("w", w, dw), ("b", b, db)):
        fd = torch.empty_like(t)
        flat, fdf = t.view(-1), fd.view(-1)
        for k in range(flat.numel()):
            p, m = t.clone(), t.clone()
            p.view(-1)[k] += h
            m.view(-1)[k] -= h
            args_p = {"x": (p, w, b), "w": (x, p, b), "b": (x, w, p)}[name]
            args_m = {"x": (m, w, b), "w": (x, m, b), "b": (x, w, m)}[name]
            fdf[k] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert float((fd - g).abs().max()) < 1e-7 * max(1.0, float(g.abs().max())), name


@pytest.mark.parametrize("dtype", [torch.float64, torch.float32, torch.bfloat16])
def test_power_of_two_scale_identity_is_exact(dtype):
    x = synth.store(synth.normal(89, "x", (4, 80), mean=1.0), dtype)
    w = synth.weight(89, 80, dtype)
    b = synth.store(synth.normal(89, "r", (80,), std=0.1), dtype)
    y1, _, _ = oracle.layernorm_fwd((x.double() * 4).to(dtype), w, b, 1e-5, eps_exact=True)
    y2, _, _ = oracle.layernorm_fwd(x, w, b, 1e-5 / 16, eps_exact=True)
    assert torch.equal(y1.double(), y2.double())


def test_constant_rows_give_bias_and_unit_moments():
    N = 50
    w = synth.weight(91, N, torch.float64)
    b = synth.store(synth.normal(91, "r", (N,)), torch.float64)
    y, _, _ = oracle.layernorm_fwd(torch.full((3, N), -2.5, dtype=torch.float64), w, b, 1e-5,
                                   eps_exact=True)
    assert torch.equal(y, b.expand(3, N))
    x = synth.store(synth.normal(92, "x", (6, 333), mean=3.0, std=0.1), torch.float64)
    y, _, _ = oracle.layernorm_fwd(x, torch.ones(333, dtype=torch.float64), None, 1e-3,
                                   eps_exact=True)
    var = x.var(-1, unbiased=False)
    torch.testing.assert_close(y.mean(-1), torch.zeros(6, dtype=torch.float64), atol=1e-13, rtol=0)
    torch.testing.assert_close(y.pow(2).mean(-1), var / (var + 1e-3), rtol=1e-12, atol=0)


@pytest.mark.parametrize("eps", [0.0, 1e-3])
def test_backward_identities(eps):
    M, N = 5, 64
    x, dy, w, b = _case(M, N, 93)
    _, mean, rstd = oracle.layernorm_fwd(x, w, b, eps, eps_exact=True, stat_dtype=torch.float64)
    dx, _, _, _, _ = oracle.layernorm_bwd(dy, x, w, mean, rstd, dwb_dtype=torch.float64)
    torch.testing.assert_close(dx.sum(-1), torch.zeros(M, dtype=torch.float64), atol=1e-12, rtol=0)
    xh = (x - mean[:, None]) * rstd[:, None]
    mgx = (dy * w * xh).mean(-1)
    torch.testing.assert_close((xh * dx).sum(-1), N * eps * rstd ** 3 * mgx, atol=1e-11, rtol=1e-9)


def test_fused_residual():
    M, N = 32, 300
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=95)
    b = synth.store(synth.normal(95, "r", (N,), std=0.1), torch.bfloat16)
    y, res, mean, rstd = oracle.add_layernorm_fwd(inp["x"], inp["r"], inp["w"], b, 1e-5)
    want = (inp["x"].float() + inp["r"].float()).to(torch.bfloat16)
    assert torch.equal(res.view(torch.int16), want.view(torch.int16))
    y2, mean2, rstd2 = oracle.layernorm_fwd(res, inp["w"], b, 1e-5)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(mean, mean2) and torch.equal(rstd, rstd2)
    ref = F.layer_norm(want.double(), (N,), inp["w"].double(), b.double(),
                       oracle.eps_as_float32(1e-5))
    y64, _, _, _ = oracle.add_layernorm_fwd(inp["x"], inp["r"], inp["w"], b, 1e-5,
                                            y_dtype=torch.float64)
    torch.testing.assert_close(y64, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("M,N", [(1, 3), (4, 33), (3, 256)])
def test_fused_backward_matches_torch_autograd_float64(M, N):
    eps = 1e-4
    x, dy, w, b = _case(M, N, 97)
    r = synth.store(synth.normal(97, "r", (M, N)), torch.float64)
    dres = synth.store(synth.normal(98, "dy", (M, N)), torch.float64)
    _, res, mean, rstd = oracle.add_layernorm_fwd(x, r, w, b, eps, eps_exact=True,
                                                  stat_dtype=torch.float64)
    dh, dw, db, _, _ = oracle.add_layernorm_bwd(dy, dres, res, w, mean, rstd,
                                                dwb_dtype=torch.float64)
    xr, rr, wr, br = (t.clone().requires_grad_(True) for t in (x, r, w, b))
    s = xr + rr
    ((F.layer_norm(s, (N,), wr, br, eps) * dy).sum() + (s * dres).sum()).backward()
    torch.testing.assert_close(dh, xr.grad, rtol=1e-10, atol=1e-12)
    torch.testing.assert_close(dh, rr.grad, rtol=1e-10, atol=1e-12)
    torch.testing.assert_close(dw, wr.grad, rtol=1e-11, atol=1e-12)
    torch.testing.assert_close(db, br.grad, rtol=1e-12, atol=1e-13)
    # no residual gradient: the plain backward, bit for bit
    dh0, dw0, db0, _, _ = oracle.add_layernorm_bwd(dy, None, res, w, mean, rstd,
                                                   dwb_dtype=torch.float64)
    dx, dwp, dbp, _, _ = oracle.layernorm_bwd(dy, res, w, mean, rstd, dwb_dtype=torch.float64)
    assert torch.equal(dh0, dx) and torch.equal(dw0, dwp) and torch.equal(db0, dbp)
    # no gradient of y: dh is the residual gradient exactly, dw = db = 0
    dh1, dw1, db1, _, _ = oracle.add_layernorm_bwd(torch.zeros_like(dy), dres, res, w, mean, rstd,
                                                   dwb_dtype=torch.float64)
    assert torch.equal(dh1, dres) and torch.all(dw1 == 0) and torch.all(db1 == 0)
