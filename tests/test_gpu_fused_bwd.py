"""GPU parity of the fused op's backward (add_rmsnorm_bwd through the C ABI)
and of the autograd custom ops, against the CPU oracle on seeded inputs."""
import sys

import pytest
import torch

import add_rmsnorm_amd as ar
import add_rmsnorm_amd.autograd as ag
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_close, assert_dw_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def fused_case(M, N, dtype, wdtype=None, seed=0):
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=seed, r_std=0.5)
    _, h, rstd = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)
    dy = synth.store(synth.normal(seed, "dy", (M, N)), dtype)
    dres = synth.store(synth.normal(seed + 1, "dy", (M, N)), dtype)
    return dy, dres, h, inp["w"], rstd


def check(dy, dres, h, w, rstd, what=""):
    dh, dw = ar.add_rmsnorm_bwd(dy.to(DEV), None if dres is None else dres.to(DEV), h.to(DEV),
                                w.to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    rdh, rdw, mag = oracle.add_rmsnorm_bwd(dy, dres, h, w, rstd)
    assert_close(dh.cpu(), rdh, f"dh {what}")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw {what}")


# default choices: 16384 x 7168 and 600 x 6152 (769 vectors, ragged) take 8
# waves per row; 4096 x 4096 the next-row prefetch kernel (2 waves per row,
# 4 vectors a lane)
@pytest.mark.parametrize("M,N", [(16384, 7168), (600, 6152), (4096, 4096), (300, 1032)])
def test_fused_bwd_bf16(M, N):
    check(*fused_case(M, N, torch.bfloat16), f"{M}x{N}")


# float32 rows on the same default paths: 1024 vectors (8 waves per row) and
# 512 vectors with enough rows for one wave per row
@pytest.mark.parametrize("M,N", [(500, 4096), (1500, 2048)])
def test_fused_bwd_f32_default_paths(M, N):
    check(*fused_case(M, N, torch.float32, seed=M), f"f32 {M}x{N}")


@pytest.mark.parametrize("dtype,wdtype", [(torch.float32, torch.float32),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.bfloat16)])
def test_fused_bwd_dtypes(dtype, wdtype):
    check(*fused_case(777, 2048, dtype, wdtype, seed=5), str(dtype))


@pytest.mark.parametrize("wpr", [1, 2, 4, 8])
def test_fused_bwd_forced_waves_per_row(knobs, wpr):
    knobs.setenv("ADDRMS_BWD_WPR", str(wpr))
    check(*fused_case(1000, 4096, torch.bfloat16, seed=7), f"wpr={wpr}")


# The wide variant (1024-thread blocks, 2 waves per row) where it is built
# for the fused backward: up to 3 vectors a lane
@pytest.mark.parametrize("dtype,M,N", [(torch.bfloat16, 3001, 3072), (torch.bfloat16, 9000, 1040),
                                       (torch.float32, 1000, 1536)])
def test_fused_bwd_wide_variant(knobs, dtype, M, N):
    knobs.setenv("ADDRMS_BWD_WPR", "2")
    knobs.setenv("ADDRMS_BWD_WIDE", "1")
    check(*fused_case(M, N, dtype, seed=M), f"wide {M}x{N}")


# The next-row prefetch kernel (2 waves per row): forced at 1 to 4 vectors a
# lane on every dtype pair, and on its default shapes (4 vectors a lane)
@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16)])
def test_fused_bwd_prefetch_forced(knobs, dtype, wdtype):
    knobs.setenv("ADDRMS_BWD_WPR", "2")
    knobs.setenv("ADDRMS_BWD_WIDE", "2")
    knobs.setenv("ADDRMS_BWD_PREFETCH", "1")
    cases = [(1001, 4096), (777, 2056), (9, 520)] if dtype == torch.bfloat16 \
        else [(1001, 2048), (777, 1028), (9, 260)]
    for M, N in cases:
        check(*fused_case(M, N, dtype, wdtype, seed=M + N), f"prefetch {M}x{N}")
    # the grid capped at 16 blocks: every block walks many row steps
    knobs.setenv("ADDRMS_MAX_PARTIALS", "16")
    for M, N in cases:
        check(*fused_case(M, N, dtype, wdtype, seed=M + N), f"prefetch, 16 blocks, {M}x{N}")


@pytest.mark.parametrize("M,N", [(24576, 3584), (16384, 4096)])
def test_fused_bwd_prefetch_default_shapes(M, N):
    check(*fused_case(M, N, torch.bfloat16, seed=M), f"{M}x{N}")


@pytest.mark.parametrize("M,N", [(5, 4096), (129, 7), (64, 1000)])
def test_fused_bwd_elementwise(knobs, M, N):
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    check(*fused_case(M, N, torch.bfloat16, seed=9), f"elem {M}x{N}")


@pytest.mark.parametrize("N", [1, 8, 65, 8193, 16384, 30720])
def test_fused_bwd_edge_shapes(N):
    check(*fused_case(33, N, torch.bfloat16, seed=N), f"N={N}")


def test_fused_bwd_without_residual_gradient_is_plain_bwd():
    dy, _, h, w, rstd = fused_case(512, 4096, torch.bfloat16, seed=11)
    check(dy, None, h, w, rstd, "dres=None")
    args = [dy.to(DEV), h.to(DEV), w.to(DEV), rstd.to(DEV)]
    a = ar.add_rmsnorm_bwd(args[0], None, *args[1:])
    b = ar.rmsnorm_bwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


@pytest.mark.parametrize("prefetch", [False, True])
@pytest.mark.parametrize("target", ["dy", "dres", "h"])
def test_fused_bwd_in_place(knobs, target, prefetch):
    """dh over each of its inputs; with prefetch, through the next-row
    prefetch kernel on a grid of 16 blocks, so the next row's loads of dy,
    dres and h are in flight while this row's dh is stored over one of them."""
    if prefetch:
        knobs.setenv("ADDRMS_BWD_WPR", "2")
        knobs.setenv("ADDRMS_BWD_WIDE", "2")
        knobs.setenv("ADDRMS_BWD_PREFETCH", "1")
        knobs.setenv("ADDRMS_MAX_PARTIALS", "16")
    dy, dres, h, w, rstd = fused_case(300, 4096, torch.bfloat16, seed=13)
    rdh, rdw, mag = oracle.add_rmsnorm_bwd(dy, dres, h, w, rstd)
    t = {"dy": dy.to(DEV), "dres": dres.to(DEV), "h": h.to(DEV)}
    dh, dw = ar.add_rmsnorm_bwd(t["dy"], t["dres"], t["h"], w.to(DEV), rstd.to(DEV), dh=t[target])
    assert dh.data_ptr() == t[target].data_ptr()
    assert_close(t[target].cpu(), rdh, f"dh over {target}")
    assert_dw_close(dw.cpu(), rdw, mag)


# ---- autograd custom ops -------------------------------------------------------

@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32)])
def test_add_rms_norm_autograd(dtype, wdtype):
    M, N = 256, 4096
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=17, r_std=0.5)
    gy = synth.store(synth.normal(17, "dy", (M, N)), dtype)
    gres = synth.store(synth.normal(18, "dy", (M, N)), dtype)
    x, r, w = (inp[k].to(DEV).requires_grad_(True) for k in ("x", "r", "w"))
    y, res = ag.add_rms_norm(x, r, w, 1e-6)
    torch.autograd.backward([y, res], [gy.to(DEV), gres.to(DEV)])
    torch.cuda.synchronize()
    ry, rres, rrstd = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)
    assert_close(y.detach().cpu(), ry, "y")
    rdh, rdw, mag = oracle.add_rmsnorm_bwd(gy, gres, rres, inp["w"], rrstd)
    assert_close(x.grad.cpu(), rdh, "x.grad")
    assert_close(r.grad.cpu(), rdh, "r.grad")
    assert w.grad.dtype == wdtype
    assert_dw_close(w.grad.cpu(), rdw, mag, "w.grad")


def test_rms_norm_autograd_and_modules():
    M, N = 128, 2048
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.float32, seed=19)
    x = inp["x"].to(DEV).requires_grad_(True)
    w = inp["w"].to(DEV).requires_grad_(True)
    y = ag.rms_norm(x, w, 1e-6)
    y.backward(inp["dy"].to(DEV))
    torch.cuda.synchronize()
    ry, rrstd = by_rows(oracle.rmsnorm_fwd, inp["x"], inp["w"], 1e-6)
    rdx, rdw, mag = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], rrstd)
    assert_close(y.detach().cpu(), ry, "y")
    assert_close(x.grad.cpu(), rdx, "x.grad")
    assert_dw_close(w.grad.cpu(), rdw, mag, "w.grad")
    # the module forms run and produce gradients for their weights
    m = ag.AddRMSNorm(N, dtype=torch.bfloat16, device=DEV)
    xb = inp["x"].to(DEV, torch.bfloat16).requires_grad_(True)
    yb, resb = m(xb, torch.zeros_like(xb))
    (yb.float().sum() + resb.float().sum()).backward()
    assert m.weight.grad is not None and m.weight.grad.dtype == torch.bfloat16
    assert xb.grad is not None and torch.isfinite(xb.grad.float()).all()
    n = ag.RMSNorm(N, dtype=torch.bfloat16, device=DEV)
    n(xb.detach()).float().sum().backward()
    assert n.weight.grad is not None


def test_custom_op_registration_checks():
    """torch.library.opcheck: schema, fake implementation, autograd
    registration of each op on real GPU tensors."""
    M, N = 8, 512
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, torch.float32, seed=23)
    x, r, w = (inp[k].to(DEV) for k in ("x", "r", "w"))
    torch.library.opcheck(torch.ops.addrms.add_rms_norm_fwd, (x, r, w, 1e-6))
    torch.library.opcheck(torch.ops.addrms.rms_norm_fwd, (x, w, 1e-6))
    _, h, rstd = torch.ops.addrms.add_rms_norm_fwd(x, r, w, 1e-6)
    torch.library.opcheck(torch.ops.addrms.add_rms_norm_bwd, (x, r, h, w, rstd))
    torch.library.opcheck(torch.ops.addrms.rms_norm_bwd, (x, h, w, rstd))


def test_autograd_non_contiguous_inputs():
    """Transposed and column-sliced activations: forward and backward run on
    contiguous copies and give the same bits as contiguous inputs; every
    output is contiguous (as the fake implementations declare), and opcheck
    accepts the strided samples."""
    M, N = 384, 1024
    inp = synth.add_rmsnorm_fwd_inputs(N, M, torch.bfloat16, seed=29, r_std=0.5)
    xt = inp["x"].to(DEV).t()                       # [M, N], transposed view
    wide = synth.store(synth.normal(29, "x", (M, 2 * N)), torch.bfloat16).to(DEV)
    xs = wide[:, ::2]                               # [M, N], column stride 2
    r = synth.store(synth.normal(29, "r", (M, N)), torch.bfloat16).to(DEV)
    w = synth.weight(29, N, torch.bfloat16).to(DEV)
    b = synth.store(synth.normal(29, "b", (N,), std=0.1), torch.bfloat16).to(DEV)
    dy = synth.store(synth.normal(29, "dy", (M, N)), torch.bfloat16).to(DEV)
    dres = synth.store(synth.normal(30, "dy", (M, N)), torch.bfloat16).to(DEV)

    def grads(fn, xv, *rest):
        leaves = [xv.detach().clone() if xv.is_contiguous() else xv.detach(), *rest]
        leaves = [t.requires_grad_(True) if t is not None else None for t in leaves]
        out = fn(*leaves)
        outs = out if isinstance(out, tuple) else (out,)
        for o in outs:
            assert o.is_contiguous()
        torch.autograd.backward(list(outs), [dy, dres][:len(outs)])
        torch.cuda.synchronize()
        return [o.detach() for o in outs], [t.grad for t in leaves if t is not None]

    cases = [
        ("rms_norm", lambda x, w_: ag.rms_norm(x, w_, 1e-6), (w,)),
        ("add_rms_norm", lambda x, r_, w_: ag.add_rms_norm(x, r_, w_, 1e-6), (r, w)),
        ("layer_norm", lambda x, w_, b_: ag.layer_norm(x, w_, b_, 1e-5), (w, b)),
        ("add_layer_norm", lambda x, r_, w_, b_: ag.add_layer_norm(x, r_, w_, b_, 1e-5),
         (r, w, b)),
    ]
    for name, fn, rest in cases:
        for xv in (xt, xs):
            assert not xv.is_contiguous()
            rest_a = [t.detach().clone() for t in rest]
            rest_b = [t.detach().clone() for t in rest]
            out_nc, g_nc = grads(fn, xv, *rest_a)
            out_c, g_c = grads(fn, xv.contiguous(), *rest_b)
            for a, c in zip(out_nc + g_nc, out_c + g_c):
                assert torch.equal(a.contiguous().view(torch.uint8),
                                   c.contiguous().view(torch.uint8)), name
    torch.library.opcheck(torch.ops.addrms.rms_norm_fwd, (xt, w, 1e-6))
    torch.library.opcheck(torch.ops.addrms.add_rms_norm_fwd, (xs, r, w, 1e-6))
    torch.library.opcheck(torch.ops.addrms.layer_norm_fwd, (xt, w, b, 1e-5))
    _, h, rstd = torch.ops.addrms.add_rms_norm_fwd(xs, r, w, 1e-6)
    torch.library.opcheck(torch.ops.addrms.rms_norm_bwd, (dy.t().contiguous().t(), xt, w, rstd))


def test_dh_is_rounded_once_16384x7168():
    """dh within half a bf16 ulp of the binary64 value plus float32 noise
    scaled by its terms: one rounding of rstd * (g - hh * c) + dres."""
    from test_gpu_bwd import _dx_terms
    from parity import assert_correctly_rounded
    M, N = 16384, 7168
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=41, r_std=0.5)
    h = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)[1]
    w = inp["w"]
    rstd = by_rows(oracle.rmsnorm_fwd, h, w, 1e-6)[1]
    dy = synth.store(synth.normal(41, "dy", (M, N)), torch.bfloat16)
    dres = synth.store(synth.normal(42, "dy", (M, N)), torch.bfloat16)
    dh, _ = ar.add_rmsnorm_bwd(dy.to(DEV), dres.to(DEV), h.to(DEV), w.to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    dh64 = oracle.add_rmsnorm_bwd(dy, dres, h, w, rstd, dh_dtype=torch.float64)[0]
    assert_correctly_rounded(dh, dh64, _dx_terms(dy, h, w, rstd, dres), "dh")
