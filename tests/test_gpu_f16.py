"""GPU parity of every operation with IEEE binary16 (float16) storage, through
the C ABI, against the CPU oracle: float16 rows with float16, float32 or
bfloat16 weights, and float16 weights with the other row types.

Tolerances: float16 y and dx within 1e-4 + 2e-3 |ref| (about two float16
ulps), the residual bit for bit, and at full size every y and dx within half
a float16 ulp of the binary64 value plus float32 noise (one rounding).
Coverage: the full headline shape (forward) and the full backward shapes;
smaller batches of the same widths for LayerNorm and the quantised outputs,
whose full shapes run in bfloat16 elsewhere; every forward launch shape (waves per
row) and the element-wise path; ragged widths; every x pattern of the
residual add against a grid of r patterns (subnormals, infinities, NaN and
the largest values included); outputs past float16's range; the backwards
(plain, fused, LayerNorm); the E4M3 and MXFP4 outputs; RMSNorm + RoPE; the
autograd ops."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import add_rmsnorm_amd.autograd as ag
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_bits_equal, assert_close, assert_correctly_rounded, assert_dw_close
from test_gpu_fwd import check_fused, check_plain, gpu_fused, gpu_plain

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H = torch.float16


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


# ---- forward ---------------------------------------------------------------------

def test_fused_16384x7168_rounded_once():
    inp = synth.add_rmsnorm_fwd_inputs(16384, 7168, H, seed=61, r_std=0.5)
    y, res, _ = check_fused(inp["x"], inp["r"], inp["w"], 1e-6, "float16 16384x7168")
    y64 = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6, y_dtype=torch.float64)[0]
    assert_correctly_rounded(y, y64, None, "float16 y")
    yp, _ = gpu_plain(inp["x"], inp["w"], 1e-6)
    yp64 = by_rows(oracle.rmsnorm_fwd, inp["x"], inp["w"], 1e-6, y_dtype=torch.float64)[0]
    assert_correctly_rounded(yp, yp64, None, "float16 plain y")
    # fused = plain on the residual, bit for bit (the two take different
    # launch shapes at this size)
    y2, _ = gpu_plain(res, inp["w"], 1e-6)
    assert_bits_equal(y2, y, "plain(residual_out) vs fused y")


PAIRS = [(H, H), (H, torch.float32), (H, torch.bfloat16), (torch.bfloat16, H), (torch.float32, H)]


@pytest.mark.parametrize("wpr", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("dtype,wdtype", PAIRS)
def test_forced_waves_per_row(knobs, wpr, dtype, wdtype):
    knobs.setenv("ADDRMS_FWD_WPR", str(wpr))
    for M, N in [(37, 4096), (5, 1032), (300, 512), (9, 7168)]:
        inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=M + N, r_std=0.5)
        check_fused(inp["x"], inp["r"], inp["w"], 1e-6, f"wpr={wpr} {M}x{N}")
        check_plain(inp["x"], inp["w"], 1e-6, f"wpr={wpr} {M}x{N}")


@pytest.mark.parametrize("dtype,wdtype", [(H, H), (H, torch.float32)])
@pytest.mark.parametrize("M,N", [(3, 4096), (64, 7168), (2, 8), (5, 1001)])
def test_elementwise_path(knobs, dtype, wdtype, M, N):
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=7)
    check_fused(inp["x"], inp["r"], inp["w"], 1e-6, "elem")
    check_plain(inp["x"], inp["w"], 1e-6, "elem")


@pytest.mark.parametrize("N", [1, 7, 8, 63, 64, 65, 520, 4095, 4096, 7168, 8193, 16384, 65536])
@pytest.mark.parametrize("M", [1, 1023])
def test_edge_shapes(M, N):
    if M * N > 1 << 24:
        M = max(1, (1 << 24) // N)
    inp = synth.add_rmsnorm_fwd_inputs(M, N, H, seed=N)
    check_fused(inp["x"], inp["r"], inp["w"], 1e-6, f"{M}x{N}")


def test_residual_add_exhaustive_sweep():
    """Every float16 pattern of x against a strided grid of r patterns (zeros,
    subnormals, the smallest normal, the largest finite, infinities, NaN):
    residual_out bit for bit, the float32 add rounded once to float16."""
    xs = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    rs = np.unique(np.concatenate([
        np.arange(0, 1 << 16, 1031, dtype=np.uint32),
        np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF,
                  0xFBFF, 0x7C00, 0xFC00, 0x7E00, 0x3BFF, 0x3C01], dtype=np.uint32)]).astype(np.uint16))
    N = 4096
    x = torch.from_numpy(np.tile(xs, rs.size).view(np.int16)).view(H).view(-1, N)
    r = torch.from_numpy(np.repeat(rs, xs.size).view(np.int16)).view(H).view(-1, N)
    w = torch.ones(N, dtype=H)
    _, res, _ = gpu_fused(x, r, w, 1e-6)
    _, rres, _ = by_rows(oracle.add_rmsnorm_fwd, x, r, w, 1e-6)
    assert_bits_equal(res, rres, "float16 residual sweep")


def test_outputs_beyond_float16_range():
    """y past 65504 stores as infinity (and the residual of two large values
    too), exactly where the oracle's one rounding puts it."""
    inp = synth.add_rmsnorm_fwd_inputs(64, 1024, H, seed=9)
    w = torch.full((1024,), 30000.0, dtype=H)
    x = inp["x"].clone()
    x[3, :] = 60000.0
    r = inp["r"].clone()
    r[3, :] = 30000.0                     # residual 90000 -> inf
    check_fused(x, r, w, 1e-6, "beyond range")
    check_plain(inp["x"], w, 1e-6, "beyond range")


# ---- backwards -----------------------------------------------------------------

@pytest.mark.parametrize("dtype,wdtype", [(H, H), (H, torch.float32), (torch.bfloat16, H)])
@pytest.mark.parametrize("M,N", [(32768, 4096), (333, 1000), (1500, 2048), (64, 7168)])
def test_rms_backward(dtype, wdtype, M, N):
    if M * N > 1 << 26 and (dtype, wdtype) != (H, H):
        M = 4096
    inp = synth.rmsnorm_bwd_inputs(M, N, dtype, wdtype, seed=M + N)
    rstd = by_rows(oracle.rmsnorm_fwd, inp["x"], inp["w"], 1e-6)[1]
    dx, dw = ar.rmsnorm_bwd(inp["dy"].to(DEV), inp["x"].to(DEV), inp["w"].to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    rdx, rdw, mag = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], rstd)
    assert_close(dx.cpu(), rdx, f"dx {M}x{N}")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw {M}x{N}")
    if dtype == H and M == 32768:
        dx64 = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], rstd, dx_dtype=torch.float64)[0]
        from test_gpu_bwd import _dx_terms
        terms = _dx_terms(inp["dy"], inp["x"], inp["w"], rstd)
        assert_correctly_rounded(dx.cpu(), dx64, terms, "float16 dx")


@pytest.mark.parametrize("wpr", [1, 2, 4, 8])
def test_rms_backward_forced_waves_per_row(knobs, wpr):
    knobs.setenv("ADDRMS_BWD_WPR", str(wpr))
    inp = synth.rmsnorm_bwd_inputs(777, 4096, H, seed=wpr)
    rstd = by_rows(oracle.rmsnorm_fwd, inp["x"], inp["w"], 1e-6)[1]
    dx, dw = ar.rmsnorm_bwd(inp["dy"].to(DEV), inp["x"].to(DEV), inp["w"].to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    rdx, rdw, mag = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], rstd)
    assert_close(dx.cpu(), rdx, f"dx wpr={wpr}")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw wpr={wpr}")


@pytest.mark.parametrize("M,N", [(16384, 7168), (4096, 4096), (600, 6152), (301, 1000)])
def test_fused_backward(M, N):
    inp = synth.add_rmsnorm_fwd_inputs(M, N, H, seed=M, r_std=0.5)
    _, h, rstd = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)
    dy = synth.store(synth.normal(M, "dy", (M, N)), H)
    dres = synth.store(synth.normal(M + 1, "dy", (M, N)), H)
    dh, dw = ar.add_rmsnorm_bwd(dy.to(DEV), dres.to(DEV), h.to(DEV), inp["w"].to(DEV),
                                rstd.to(DEV))
    torch.cuda.synchronize()
    rdh, rdw, mag = oracle.add_rmsnorm_bwd(dy, dres, h, inp["w"], rstd)
    assert_close(dh.cpu(), rdh, f"dh {M}x{N}")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw {M}x{N}")


@pytest.mark.parametrize("M,N", [(4096, 7168), (8192, 4096), (333, 1000)])
def test_layernorm(M, N):
    inp = synth.add_rmsnorm_fwd_inputs(M, N, H, seed=M + 3, r_std=0.5)
    x, r, w = inp["x"], inp["r"], inp["w"]
    b = synth.store(synth.normal(5, "b", (N,), std=0.1), H)
    g = lambda t: t.to(DEV)
    y, res, mean, rstd = ar.add_layernorm_fwd(g(x), g(r), g(w), g(b), 1e-5, return_stats=True)
    torch.cuda.synchronize()
    ry, rres, rmean, rrstd = by_rows(oracle.add_layernorm_fwd, x, r, w, b, 1e-5)
    assert_bits_equal(res.cpu(), rres, "LayerNorm residual_out")
    assert_close(y.cpu(), ry, "LayerNorm y")
    assert_close(mean.cpu(), rmean, "mean", atol=1e-6, rtol=1e-5)
    assert_close(rstd.cpu(), rrstd, "rstd", atol=0, rtol=1e-5)
    dy = synth.store(synth.normal(6, "dy", (M, N)), H)
    _, lmean, lrstd = by_rows(oracle.layernorm_fwd, x, w, b, 1e-5)
    dx, dw, db = ar.layernorm_bwd(g(dy), g(x), g(w), g(lmean), g(lrstd))
    torch.cuda.synchronize()
    rdx, rdw, rdb, mw, mb = oracle.layernorm_bwd(dy, x, w, lmean, lrstd)
    assert_close(dx.cpu(), rdx, "LayerNorm dx")
    assert_dw_close(dw.cpu(), rdw, mw, "LayerNorm dw")
    assert_dw_close(db.cpu(), rdb, mb, "LayerNorm db")


# ---- quantised outputs, RoPE, autograd -----------------------------------------

@pytest.mark.parametrize("group", [None, 128])
@pytest.mark.parametrize("M,N", [(2048, 7168), (33, 1032)])
def test_fp8_output(M, N, group):
    from test_gpu_fp8 import run
    inp = synth.add_rmsnorm_fwd_inputs(M, N, H, seed=M + N, r_std=0.5)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"float16 {M}x{N}", group=group)
    run(inp["x"], None, inp["w"], 1e-6, f"float16 plain {M}x{N}", group=group)


@pytest.mark.parametrize("M,N", [(4096, 7168), (40, 1000)])
def test_mxfp4_output(M, N):
    from test_gpu_mxfp4 import run
    inp = synth.add_rmsnorm_fwd_inputs(M, N, H, seed=M + N, r_std=0.5)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"float16 {M}x{N}")


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("wdtype", [H, torch.float32])
def test_rope(interleaved, wdtype):
    from test_gpu_rope import run_packed
    run_packed(2051, 32, 8, 128, H, wdtype, interleaved, seed=3)
    run_packed(37, 4, 2, 64, H, wdtype, interleaved, seed=4)


def test_autograd():
    M, N = 256, 4096
    inp = synth.add_rmsnorm_fwd_inputs(M, N, H, seed=17, r_std=0.5)
    gy = synth.store(synth.normal(17, "dy", (M, N)), H)
    gres = synth.store(synth.normal(18, "dy", (M, N)), H)
    x, r, w = (inp[k].to(DEV).requires_grad_(True) for k in ("x", "r", "w"))
    y, res = ag.add_rms_norm(x, r, w, 1e-6)
    torch.autograd.backward([y, res], [gy.to(DEV), gres.to(DEV)])
    torch.cuda.synchronize()
    ry, rres, rrstd = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)
    assert_close(y.detach().cpu(), ry, "y")
    rdh, rdw, mag = oracle.add_rmsnorm_bwd(gy, gres, rres, inp["w"], rrstd)
    assert_close(x.grad.cpu(), rdh, "x.grad")
    assert_close(r.grad.cpu(), rdh, "r.grad")
    assert w.grad.dtype == H
    # dw is computed in float32 and returned in w's dtype (float16)
    assert_close(w.grad.cpu().float(), rdw.to(H).float(), "w.grad", atol=1e-2, rtol=2e-3)
