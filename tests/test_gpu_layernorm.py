"""GPU parity of the LayerNorm variants (HIP library through the C ABI)
against the CPU oracle on seeded inputs: forward with and without bias and
residual, the saved statistics, backward dx/dw/db, every kernel variant,
ragged shapes, in-place buffers and the empty batch."""
import sys

import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_bits_equal, assert_close, assert_dw_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 1e-5


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def inputs(M, N, dtype, wdtype=None, seed=0, bias=True):
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=seed, r_std=0.5)
    # activations with a non-zero mean, so the centring matters
    inp["x"] = synth.store(synth.normal(seed, "x", (M, N), mean=0.75), dtype)
    inp["b"] = synth.store(synth.normal(seed, "b", (N,), std=0.1), wdtype or dtype) if bias else None
    return inp


def check_fwd(inp, fused, what=""):
    x, w, b = inp["x"], inp["w"], inp["b"]
    g = lambda t: None if t is None else t.to(DEV)
    if fused:
        y, res, mean, rstd = ar.add_layernorm_fwd(g(x), g(inp["r"]), g(w), g(b), EPS,
                                                  return_stats=True)
        ry, rres, rmean, rrstd = by_rows(oracle.add_layernorm_fwd, x, inp["r"], w, b, EPS)
        assert_bits_equal(res.cpu(), rres, f"residual_out {what}")
    else:
        y, mean, rstd = ar.layernorm_fwd(g(x), g(w), g(b), EPS, return_stats=True)
        ry, rmean, rrstd = by_rows(oracle.layernorm_fwd, x, w, b, EPS)
    torch.cuda.synchronize()
    assert_close(y.cpu(), ry, f"y {what}")
    assert_close(mean.cpu(), rmean, f"mean {what}", atol=1e-6, rtol=1e-5)
    assert_close(rstd.cpu(), rrstd, f"rstd {what}", atol=0, rtol=1e-5)


def check_bwd(inp, what="", with_db=True):
    x, w = inp["x"], inp["w"]
    M, N = x.shape
    dy = synth.store(synth.normal(7, "dy", (M, N)), x.dtype)
    _, mean, rstd = by_rows(oracle.layernorm_fwd, x, w, inp["b"], EPS)
    dx, dw, db = ar.layernorm_bwd(dy.to(DEV), x.to(DEV), w.to(DEV), mean.to(DEV), rstd.to(DEV),
                                  with_db=with_db)
    torch.cuda.synchronize()
    rdx, rdw, rdb, mw, mb = oracle.layernorm_bwd(dy, x, w, mean, rstd)
    assert_close(dx.cpu(), rdx, f"dx {what}")
    assert_dw_close(dw.cpu(), rdw, mw, f"dw {what}")
    if with_db:
        assert_dw_close(db.cpu(), rdb, mb, f"db {what}")
    else:
        assert db is None


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("M,N", [(16384, 7168), (4096, 4096), (3, 8192)])
def test_forward_bf16(fused, bias, M, N):
    check_fwd(inputs(M, N, torch.bfloat16, seed=M + N, bias=bias), fused, f"{M}x{N}")


@pytest.mark.parametrize("dtype,wdtype", [(torch.float32, torch.float32),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.bfloat16)])
def test_forward_dtypes(dtype, wdtype):
    inp = inputs(513, 2048, dtype, wdtype, seed=3)
    check_fwd(inp, False, str(dtype))
    check_fwd(inp, True, str(dtype))


@pytest.mark.parametrize("wpr", [1, 2, 4, 8, 16])
def test_forward_forced_waves_per_row(knobs, wpr):
    knobs.setenv("ADDRMS_FWD_WPR", str(wpr))
    for M, N in [(37, 4096), (5, 1032)]:
        inp = inputs(M, N, torch.bfloat16, seed=M, bias=True)
        check_fwd(inp, True, f"wpr={wpr} {M}x{N}")
        check_fwd(inp, False, f"wpr={wpr} {M}x{N}")


@pytest.mark.parametrize("N", [1, 7, 64, 65, 4095, 8193, 65536])
def test_forward_edge_shapes(N):
    M = max(1, min(300, (1 << 22) // N))
    inp = inputs(M, N, torch.bfloat16, seed=N)
    check_fwd(inp, True, f"N={N}")
    check_fwd(inp, False, f"N={N}")


@pytest.mark.parametrize("M,N", [(4, 4096), (64, 1000)])
def test_forward_elementwise(knobs, M, N):
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    inp = inputs(M, N, torch.bfloat16, seed=11)
    check_fwd(inp, True, "elem")
    check_fwd(inp, False, "elem")


def test_forward_in_place_and_empty():
    inp = inputs(200, 4096, torch.bfloat16, seed=13)
    ry, rres, _, _ = by_rows(oracle.add_layernorm_fwd, inp["x"], inp["r"], inp["w"], inp["b"], EPS)
    x, r = inp["x"].to(DEV), inp["r"].to(DEV)
    ar.add_layernorm_fwd(x, r, inp["w"].to(DEV), inp["b"].to(DEV), EPS, y=x, residual_out=r)
    torch.cuda.synchronize()
    assert_bits_equal(r.cpu(), rres, "residual in r")
    assert_close(x.cpu(), ry, "y in x")
    e = torch.empty(0, 4096, dtype=torch.bfloat16, device=DEV)
    y = ar.layernorm_fwd(e, inp["w"].to(DEV), None, EPS)
    assert y.shape == (0, 4096)


# 16384 x 7168 and 600 x 6152 (769 vectors, the last one ragged) take 8 waves
# per row by default
@pytest.mark.parametrize("M,N", [(32768, 4096), (16384, 7168), (600, 6152), (3001, 1032), (7, 8192)])
def test_backward_bf16(M, N):
    check_bwd(inputs(M, N, torch.bfloat16, seed=M), f"{M}x{N}")


@pytest.mark.parametrize("wpr", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.float32, torch.float32),
                                          (torch.bfloat16, torch.float32)])
def test_backward_variants(knobs, wpr, dtype, wdtype):
    knobs.setenv("ADDRMS_BWD_WPR", str(wpr))
    check_bwd(inputs(1000, 2048, dtype, wdtype, seed=wpr), f"wpr={wpr}")


# The wide variant (1024-thread blocks, 2 waves per row; dw and db share its
# LDS tree) where it is built for LayerNorm: up to 3 vectors a lane
@pytest.mark.parametrize("dtype,M,N", [(torch.bfloat16, 3001, 3072), (torch.bfloat16, 9000, 1040),
                                       (torch.float32, 1000, 1536)])
def test_backward_wide_variant(knobs, dtype, M, N):
    knobs.setenv("ADDRMS_BWD_WPR", "2")
    knobs.setenv("ADDRMS_BWD_WIDE", "1")
    check_bwd(inputs(M, N, dtype, seed=M), f"wide {M}x{N}")


# The next-row prefetch variant (2 waves per row): forced at 1 to 4 vectors a
# lane and ragged rows, and on its default shapes (4 vectors a lane)
@pytest.mark.parametrize("dtype,M,N", [(torch.bfloat16, 3001, 4096), (torch.bfloat16, 777, 2056),
                                       (torch.bfloat16, 2049, 520), (torch.float32, 1001, 2048),
                                       (torch.float32, 9, 772)])
def test_backward_prefetch_forced(knobs, dtype, M, N):
    knobs.setenv("ADDRMS_BWD_WPR", "2")
    knobs.setenv("ADDRMS_BWD_WIDE", "2")
    knobs.setenv("ADDRMS_BWD_PREFETCH", "1")
    check_bwd(inputs(M, N, dtype, seed=M + N), f"prefetch {M}x{N}")


@pytest.mark.parametrize("M,N", [(8192, 4096), (32768, 3584)])
def test_backward_prefetch_default_shapes(M, N):
    check_bwd(inputs(M, N, torch.bfloat16, seed=M), f"{M}x{N}")


@pytest.mark.parametrize("N", [1, 5, 65, 4100, 16392])
def test_backward_edge_shapes(N):
    check_bwd(inputs(max(1, min(500, (1 << 22) // N)), N, torch.bfloat16, seed=N), f"N={N}")


@pytest.mark.parametrize("M,N", [(9, 4096), (130, 1000)])
def test_backward_elementwise_and_no_db(knobs, M, N):
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    check_bwd(inputs(M, N, torch.bfloat16, seed=17), "elem")
    check_bwd(inputs(M, N, torch.float32, seed=18), "elem f32", with_db=False)


@pytest.mark.parametrize("prefetch", ["0", "1"])
def test_backward_in_place_and_empty(knobs, prefetch):
    """dx over dy; with prefetch = 1 through the next-row prefetch kernel,
    whose loads of the next row go out before the current row's dx stores."""
    if prefetch == "1":
        knobs.setenv("ADDRMS_BWD_WPR", "2")
        knobs.setenv("ADDRMS_BWD_WIDE", "2")
        knobs.setenv("ADDRMS_BWD_PREFETCH", "1")
        # 16 partial rows cap the grid at 16 blocks, so each block walks many
        # row steps: the next row's loads are in flight while this row's dx is
        # stored over its input
        knobs.setenv("ADDRMS_MAX_PARTIALS", "16")
    inp = inputs(300, 4096, torch.bfloat16, seed=19)
    x, w = inp["x"], inp["w"]
    dy = synth.store(synth.normal(19, "dy", (300, 4096)), torch.bfloat16)
    _, mean, rstd = by_rows(oracle.layernorm_fwd, x, w, None, EPS)
    rdx, rdw, rdb, mw, mb = oracle.layernorm_bwd(dy, x, w, mean, rstd)
    d = dy.to(DEV)
    dx, dw, db = ar.layernorm_bwd(d, x.to(DEV), w.to(DEV), mean.to(DEV), rstd.to(DEV), dx=d)
    torch.cuda.synchronize()
    assert_close(d.cpu(), rdx, "dx over dy")
    assert_dw_close(dw.cpu(), rdw, mw)
    assert_dw_close(db.cpu(), rdb, mb, "db")
    e = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    z = torch.empty(0, dtype=torch.float32, device=DEV)
    dw0 = torch.full((64,), 3.0, device=DEV)
    db0 = torch.full((64,), 3.0, device=DEV)
    ar.layernorm_bwd(e, e, w[:64].to(DEV), z, z, dw=dw0, db=db0)
    torch.cuda.synchronize()
    assert torch.all(dw0 == 0) and torch.all(db0 == 0)


# ---- fused backward and autograd ------------------------------------------------

@pytest.mark.parametrize("M,N,dtype", [(4096, 4096, torch.bfloat16), (333, 1000, torch.bfloat16),
                                       (500, 2048, torch.float32),
                                       # 8 waves per row by default (769 and 1792 vectors)
                                       (1000, 6152, torch.bfloat16), (600, 7168, torch.float32),
                                       # 12 vectors per lane; rows too long for the
                                       # register-resident variants (element-wise path)
                                       (24, 24576, torch.bfloat16), (24, 30720, torch.bfloat16),
                                       (20, 16384, torch.float32)])
def test_fused_backward(M, N, dtype):
    _fused_backward_case(M, N, dtype)


# the fused LayerNorm backward in the wide variant (1024-thread blocks, 2
# waves per row), built up to 2 vectors a lane: forced, with a ragged row
@pytest.mark.parametrize("M,N,dtype", [(3001, 2048, torch.bfloat16), (777, 1032, torch.bfloat16),
                                       (500, 1024, torch.float32)])
def test_fused_backward_wide_variant(knobs, M, N, dtype):
    knobs.setenv("ADDRMS_BWD_WPR", "2")
    knobs.setenv("ADDRMS_BWD_WIDE", "1")
    _fused_backward_case(M, N, dtype)


# the fused LayerNorm backward through the next-row prefetch kernel: forced
# at 2 and 4 vectors a lane, and on a default shape (4 vectors a lane)
# (forced cases also with the grid capped at 16 blocks, so that every block
# walks many row steps with the next row's loads in flight; float32 rows,
# and bf16 rows with float32 weights)
@pytest.mark.parametrize("M,N,dtype,wdtype,force", [
    (1001, 4096, torch.bfloat16, None, True), (777, 2056, torch.bfloat16, None, True),
    (500, 2048, torch.float32, None, True), (1001, 4096, torch.bfloat16, torch.float32, True),
    (700, 2048, torch.float32, torch.bfloat16, True), (16384, 4096, torch.bfloat16, None, False)])
def test_fused_backward_prefetch(knobs, M, N, dtype, wdtype, force):
    if force:
        knobs.setenv("ADDRMS_BWD_WPR", "2")
        knobs.setenv("ADDRMS_BWD_WIDE", "2")
        knobs.setenv("ADDRMS_BWD_PREFETCH", "1")
    _fused_backward_case(M, N, dtype, wdtype)
    if force:
        knobs.setenv("ADDRMS_MAX_PARTIALS", "16")
        _fused_backward_case(M, N, dtype, wdtype)


def _fused_backward_case(M, N, dtype, wdtype=None):
    inp = inputs(M, N, dtype, wdtype, seed=29)
    _, h, mean, rstd = by_rows(oracle.add_layernorm_fwd, inp["x"], inp["r"], inp["w"], inp["b"], EPS)
    dy = synth.store(synth.normal(29, "dy", (M, N)), dtype)
    dres = synth.store(synth.normal(30, "dy", (M, N)), dtype)
    g = lambda t: t.to(DEV)
    dh, dw, db = ar.add_layernorm_bwd(g(dy), g(dres), g(h), g(inp["w"]), g(mean), g(rstd))
    torch.cuda.synchronize()
    rdh, rdw, rdb, mw, mb = oracle.add_layernorm_bwd(dy, dres, h, inp["w"], mean, rstd)
    assert_close(dh.cpu(), rdh, "dh")
    assert_dw_close(dw.cpu(), rdw, mw, "dw")
    assert_dw_close(db.cpu(), rdb, mb, "db")


def test_layer_norm_autograd():
    import add_rmsnorm_amd.autograd as ag
    M, N = 256, 2048
    inp = inputs(M, N, torch.float32, seed=31)
    gy = synth.store(synth.normal(31, "dy", (M, N)), torch.float32)
    gres = synth.store(synth.normal(32, "dy", (M, N)), torch.float32)
    x, r, w, b = (inp[k].to(DEV).requires_grad_(True) for k in ("x", "r", "w", "b"))
    y, res = ag.add_layer_norm(x, r, w, b, EPS)
    torch.autograd.backward([y, res], [gy.to(DEV), gres.to(DEV)])
    torch.cuda.synchronize()
    ry, rres, rmean, rrstd = by_rows(oracle.add_layernorm_fwd, inp["x"], inp["r"], inp["w"], inp["b"], EPS)
    assert_close(y.detach().cpu(), ry, "y")
    rdh, rdw, rdb, mw, mb = oracle.add_layernorm_bwd(gy, gres, rres, inp["w"], rmean, rrstd)
    assert_close(x.grad.cpu(), rdh, "x.grad")
    assert_close(r.grad.cpu(), rdh, "r.grad")
    assert_dw_close(w.grad.cpu(), rdw, mw, "w.grad")
    assert_dw_close(b.grad.cpu(), rdb, mb, "b.grad")
    # plain layer_norm and the modules
    x2 = inp["x"].to(DEV).requires_grad_(True)
    y2 = ag.layer_norm(x2, w.detach(), None, EPS)
    y2.backward(gy.to(DEV))
    _, m2, s2 = by_rows(oracle.layernorm_fwd, inp["x"], inp["w"], None, EPS)
    rdx, _, _, _, _ = oracle.layernorm_bwd(gy, inp["x"], inp["w"], m2, s2)
    assert_close(x2.grad.cpu(), rdx, "x2.grad")
    mod = ag.AddLayerNorm(N, dtype=torch.bfloat16, device=DEV)
    xb = inp["x"].to(DEV, torch.bfloat16).requires_grad_(True)
    yb, rb = mod(xb, torch.zeros_like(xb))
    (yb.float().sum() + rb.float().sum()).backward()
    assert mod.weight.grad is not None and mod.bias.grad is not None
    torch.library.opcheck(torch.ops.addrms.add_layer_norm_fwd,
                          (x.detach(), r.detach(), w.detach(), b.detach(), EPS))
    torch.library.opcheck(torch.ops.addrms.layer_norm_fwd, (x.detach(), w.detach(), None, EPS))


def test_rounded_once_full_size():
    """LayerNorm y (fused, 16384 x 7168, with bias) and dx (32768 x 4096)
    within half a bf16 ulp of the binary64 values plus float32 noise scaled
    by the terms each is computed from."""
    from parity import assert_correctly_rounded
    inp = inputs(16384, 7168, torch.bfloat16, seed=51)
    x, r, w, b = inp["x"], inp["r"], inp["w"], inp["b"]
    g = lambda t: t.to(DEV)
    y, res = ar.add_layernorm_fwd(g(x), g(r), g(w), g(b), EPS)
    torch.cuda.synchronize()
    y64, h, mean, rstd = by_rows(oracle.add_layernorm_fwd, x, r, w, b, EPS, y_dtype=torch.float64,
                                                  stat_dtype=torch.float64)
    hd, mu, rs = h.double(), mean.double()[:, None], rstd.double()[:, None]
    mag = rs * w.double().abs() * ((hd - mu).abs() + mu.abs()) + b.double().abs()
    assert_correctly_rounded(y, y64, mag, "LayerNorm y")
    del y, res, y64, h, hd, mag
    inp = inputs(32768, 4096, torch.bfloat16, seed=52)
    x, w = inp["x"], inp["w"]
    M, N = x.shape
    dy = synth.store(synth.normal(53, "dy", (M, N)), x.dtype)
    _, mean, rstd = by_rows(oracle.layernorm_fwd, x, w, inp["b"], EPS)
    dx, _, _ = ar.layernorm_bwd(g(dy), g(x), g(w), g(mean), g(rstd))
    torch.cuda.synchronize()
    dx64 = oracle.layernorm_bwd(dy, x, w, mean, rstd, dx_dtype=torch.float64)[0]
    gg = dy.double() * w.double()
    xh = (x.double() - mean.double()[:, None]) * rstd.double()[:, None]
    c1 = gg.mean(dim=1, keepdim=True)
    c2 = (gg * xh).mean(dim=1, keepdim=True)
    # c1 and c2 are float32 sums over the row: their error scales with the
    # mean magnitude of their terms
    c1_terms = gg.abs().mean(dim=1, keepdim=True)
    c2_terms = (gg * xh).abs().mean(dim=1, keepdim=True)
    mag = rstd.double()[:, None] * (gg.abs() + c1.abs() + c1_terms +
                                    xh.abs() * (c2.abs() + c2_terms))
    assert_correctly_rounded(dx, dx64, mag, "LayerNorm dx")
