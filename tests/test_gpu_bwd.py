"""GPU parity of the backward (HIP library through the C ABI) against the CPU
oracle on seeded inputs: dx element by element, dw per column, with the same
saved float32 rstd (from the oracle's forward) fed to both sides; the named
workload at full size, every kernel variant, ragged shapes, aliasing, an
empty batch, determinism, and forward->backward chained on the GPU."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_close, assert_correctly_rounded, assert_dw_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def oracle_rstd(x, w, eps):
    return by_rows(oracle.rmsnorm_fwd, x, w, eps)[1]


def check_bwd(dy, x, w, eps, what="", rstd=None):
    rstd = oracle_rstd(x, w, eps) if rstd is None else rstd
    dx, dw = ar.rmsnorm_bwd(dy.to(DEV), x.to(DEV), w.to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    rdx, rdw, mag = oracle.rmsnorm_bwd(dy, x, w, rstd)
    assert_close(dx.cpu(), rdx, f"dx {what}")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw {what}")
    return dx.cpu(), dw.cpu()


def test_rmsnorm_bwd_bf16_32768x4096():
    inp = synth.workload_inputs("rmsnorm_bwd_bf16_32768x4096")
    check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6)


@pytest.mark.parametrize("wpr", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16)])
def test_forced_waves_per_row(knobs, wpr, dtype, wdtype):
    knobs.setenv("ADDRMS_BWD_WPR", str(wpr))
    for M, N in [(1000, 4096), (7, 1032), (3001, 256)]:
        inp = synth.rmsnorm_bwd_inputs(M, N, dtype, wdtype, seed=M + N)
        check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, f"wpr={wpr} {M}x{N}")


# The wide variant (1024-thread blocks, 8 rows of 2 waves per step) forced
# on every dtype pair: 1 to 4 vectors a lane, ragged last vectors, fewer rows
# than one step of the grid, and more rows than 8 per CU (several steps).
@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16)])
def test_wide_variant_forced(knobs, dtype, wdtype):
    knobs.setenv("ADDRMS_BWD_WPR", "2")
    knobs.setenv("ADDRMS_BWD_WIDE", "1")
    cases = [(1000, 4096), (3001, 3072), (7, 1032), (2049, 520), (9000, 1536)] if dtype == torch.bfloat16 \
        else [(1000, 2048), (3001, 1536), (7, 516), (2049, 260), (9000, 768)]
    for M, N in cases:
        inp = synth.rmsnorm_bwd_inputs(M, N, dtype, wdtype, seed=M + 3 * N)
        check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, f"wide {M}x{N}")


# The next-row prefetch variant (2 waves per row) forced on every dtype pair,
# 1 to 4 vectors a lane, ragged rows, a batch that ends mid-step, and with
# ADDRMS_BWD_PREFETCH=2 the plain kernel at 4 vectors a lane (the prefetch's
# default): dx bit-identical between the two.
@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16)])
def test_prefetch_variant_forced(knobs, dtype, wdtype):
    knobs.setenv("ADDRMS_BWD_WPR", "2")
    knobs.setenv("ADDRMS_BWD_WIDE", "2")
    knobs.setenv("ADDRMS_BWD_PREFETCH", "1")
    cases = [(1001, 4096), (3001, 3072), (7, 1032), (2049, 520), (9001, 1536)] if dtype == torch.bfloat16 \
        else [(1001, 2048), (3001, 1536), (7, 516), (2049, 260), (9001, 768)]
    for M, N in cases:
        inp = synth.rmsnorm_bwd_inputs(M, N, dtype, wdtype, seed=M + 5 * N)
        dx, _ = check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, f"prefetch {M}x{N}")
        if N in (4096, 2048):
            knobs.setenv("ADDRMS_BWD_PREFETCH", "2")
            dx2, _ = check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, f"no prefetch {M}x{N}")
            knobs.setenv("ADDRMS_BWD_PREFETCH", "1")
            assert torch.equal(dx.view(torch.int16) if dtype == torch.bfloat16 else dx,
                               dx2.view(torch.int16) if dtype == torch.bfloat16 else dx2)


# default choices of the wide variant: 3 vectors a lane at any batch, 4 up to
# 32 rows per CU; the 32768 x 4096 workload stays on 256-thread blocks (with
# the next-row prefetch), as do 12288 x 4096 and 32768 x 3584
@pytest.mark.parametrize("M,N", [(2048, 3072), (32768, 3072), (4096, 4096), (8192, 4096),
                                 (12288, 4096), (32768, 3584)])
def test_wide_variant_default_shapes(M, N):
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.bfloat16, seed=M + N)
    check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, f"{M}x{N}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N", [(5, 4096), (2000, 7168), (3, 8), (1025, 1000)])
def test_elementwise_path(knobs, dtype, M, N):
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    inp = synth.rmsnorm_bwd_inputs(M, N, dtype, seed=5)
    check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, "elem")


BWD_N = [1, 7, 8, 64, 65, 520, 4095, 4096, 7168, 8192, 8200, 16384, 16392, 65536]


@pytest.mark.parametrize("N", BWD_N)
@pytest.mark.parametrize("M", [1, 3, 2049])
def test_edge_shapes_bf16(M, N):
    if M * N > 1 << 24:
        M = max(1, (1 << 24) // N)
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.bfloat16, seed=N)
    check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, f"{M}x{N}")


@pytest.mark.parametrize("N", [1, 5, 4096, 4100, 8192])
@pytest.mark.parametrize("M", [2, 700])
def test_edge_shapes_f32(M, N):
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.float32, seed=N)
    check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, f"{M}x{N}")


def test_many_rows_exceed_partial_rows():
    """More blocks' worth of rows than partial rows (1024): the grid is capped
    and each block accumulates many rows."""
    inp = synth.rmsnorm_bwd_inputs(70000, 256, torch.bfloat16, seed=23)
    check_bwd(inp["dy"], inp["x"], inp["w"], 1e-6, "70000x256")


@pytest.mark.parametrize("force_elem", ["0", "1", "prefetch"])
def test_dx_in_place(knobs, force_elem):
    """dx over dy or x; "prefetch": the next-row prefetch kernel, whose loads
    of the next row go out before the current row's dx stores."""
    if force_elem == "prefetch":
        knobs.setenv("ADDRMS_BWD_WPR", "2")
        knobs.setenv("ADDRMS_BWD_WIDE", "2")
        knobs.setenv("ADDRMS_BWD_PREFETCH", "1")
        # 16 partial rows cap the grid at 16 blocks, so each block walks many
        # row steps: the next row's loads are in flight while this row's dx is
        # stored over its input
        knobs.setenv("ADDRMS_MAX_PARTIALS", "16")
    else:
        knobs.setenv("ADDRMS_FORCE_ELEM", force_elem)
    M, N = 300, 4096
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.bfloat16, seed=29)
    rstd = oracle_rstd(inp["x"], inp["w"], 1e-6)
    rdx, rdw, mag = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], rstd)
    for target in ("dy", "x"):
        dy, x = inp["dy"].to(DEV), inp["x"].to(DEV)
        out = dy if target == "dy" else x
        dx, dw = ar.rmsnorm_bwd(dy, x, inp["w"].to(DEV), rstd.to(DEV), dx=out)
        assert dx.data_ptr() == out.data_ptr()
        assert_close(out.cpu(), rdx, f"dx over {target}")
        assert_dw_close(dw.cpu(), rdw, mag, f"dw (dx over {target})")


def test_empty_batch_zeroes_dw():
    N = 4096
    w = torch.ones(N, dtype=torch.bfloat16, device=DEV)
    x = torch.empty(0, N, dtype=torch.bfloat16, device=DEV)
    rstd = torch.empty(0, dtype=torch.float32, device=DEV)
    dw = torch.full((N,), 7.0, device=DEV)
    ar.rmsnorm_bwd(x, x, w, rstd, dw=dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_deterministic():
    inp = synth.rmsnorm_bwd_inputs(4096, 4096, torch.bfloat16, seed=31)
    rstd = oracle_rstd(inp["x"], inp["w"], 1e-6).to(DEV)
    args = [inp["dy"].to(DEV), inp["x"].to(DEV), inp["w"].to(DEV), rstd]
    a = ar.rmsnorm_bwd(*args)
    b = ar.rmsnorm_bwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


def test_forward_then_backward_on_gpu():
    """GPU forward's rstd feeding the GPU backward, against the oracle chain."""
    M, N = 2048, 4096
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.bfloat16, seed=37)
    x, w, dy = inp["x"].to(DEV), inp["w"].to(DEV), inp["dy"].to(DEV)
    _, rstd = ar.rmsnorm_fwd(x, w, 1e-6, return_rstd=True)
    dx, dw = ar.rmsnorm_bwd(dy, x, w, rstd)
    torch.cuda.synchronize()
    rrstd = oracle_rstd(inp["x"], inp["w"], 1e-6)
    assert_close(rstd.cpu(), rrstd, "rstd", atol=0, rtol=1e-5)
    rdx, rdw, mag = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], rrstd)
    assert_close(dx.cpu(), rdx, "dx")
    assert_dw_close(dw.cpu(), rdw, mag)


def test_workspace_too_small_is_an_error():
    M, N = 64, 512
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.bfloat16, seed=41)
    rstd = oracle_rstd(inp["x"], inp["w"], 1e-6).to(DEV)
    ws = torch.empty(ar.rmsnorm_bwd_workspace_bytes(M, N) - 4, dtype=torch.uint8, device=DEV)
    with pytest.raises(ar.AddRmsError, match="workspace"):
        ar.rmsnorm_bwd(inp["dy"].to(DEV), inp["x"].to(DEV), inp["w"].to(DEV), rstd, workspace=ws)


def _dx_terms(dy, x, w, rstd, dres=None):
    """Per element, the magnitude of the terms dx = rstd (g - xh c) (+ dres)
    is computed from, binary64: the scale of float32 error in dx.  c is a
    float32 sum over the row, so its own error scales with the mean of |g xh|
    (its terms), not with |c|, which cancellation can make far smaller."""
    g = dy.double() * w.double()
    xh = x.double() * rstd.double()[:, None]
    t = g * xh
    c = t.mean(dim=1, keepdim=True)
    c_terms = t.abs().mean(dim=1, keepdim=True)
    mag = rstd.double()[:, None] * (g.abs() + xh.abs() * (c.abs() + c_terms))
    return mag if dres is None else mag + dres.double().abs()


def test_dx_is_rounded_once_32768x4096():
    """dx within half a bf16 ulp of the binary64 value plus float32 noise
    scaled by its terms: one rounding of rstd * (g - xh * c)."""
    inp = synth.workload_inputs("rmsnorm_bwd_bf16_32768x4096")
    dy, x, w = inp["dy"], inp["x"], inp["w"]
    rstd = oracle_rstd(x, w, 1e-6)
    dx, _ = ar.rmsnorm_bwd(dy.to(DEV), x.to(DEV), w.to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    dx64 = oracle.rmsnorm_bwd(dy, x, w, rstd, dx_dtype=torch.float64)[0]
    assert_correctly_rounded(dx, dx64, _dx_terms(dy, x, w, rstd), "dx")
