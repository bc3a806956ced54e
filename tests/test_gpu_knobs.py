"""GPU parity under the dispatcher's remaining tuning knobs, each of which
selects a launch shape no default choice takes:
- BLOCKS_PER_CU: the forward on a persistent grid of one or two blocks per CU,
  with many more rows than blocks, so every block walks many rows and reuses
  its LDS reduction slots row after row (RMS, LayerNorm, the E4M3 and MXFP4
  epilogues, for several waves per row);
- FWD_VPL: the forward's target vectors per lane, which moves the choice of
  waves per row;
- MAX_PARTIALS: the backwards with very few dw partial rows, so every block
  accumulates many rows before its merge;
- ROPE_BLOCKS_PER_CU: RMSNorm + RoPE on a capped grid, each block looping
  over several steps.
All through the C ABI, against the CPU oracle."""
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


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _fused_rms(inp, eps, what):
    g = lambda t: t.to(DEV)
    y, res, rstd = ar.add_rmsnorm_fwd(g(inp["x"]), g(inp["r"]), g(inp["w"]), eps, return_rstd=True)
    torch.cuda.synchronize()
    ry, rres, rrstd = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], eps)
    assert_bits_equal(res.cpu(), rres, f"residual_out {what}")
    assert_close(y.cpu(), ry, f"y {what}")
    assert_close(rstd.cpu(), rrstd, f"rstd {what}", atol=0, rtol=1e-5)


def _fused_ln(inp, eps, what):
    g = lambda t: t.to(DEV)
    b = synth.store(synth.normal(3, "b", (inp["x"].shape[1],), std=0.1), inp["w"].dtype)
    y, res, mean, rstd = ar.add_layernorm_fwd(g(inp["x"]), g(inp["r"]), g(inp["w"]), g(b), eps,
                                              return_stats=True)
    torch.cuda.synchronize()
    ry, rres, rmean, rrstd = by_rows(oracle.add_layernorm_fwd, inp["x"], inp["r"], inp["w"], b, eps)
    assert_bits_equal(res.cpu(), rres, f"residual_out {what}")
    assert_close(y.cpu(), ry, f"y {what}")
    assert_close(mean.cpu(), rmean, f"mean {what}", atol=1e-6, rtol=1e-5)
    assert_close(rstd.cpu(), rrstd, f"rstd {what}", atol=0, rtol=1e-5)


def _fp8_rows(inp, eps, what, group=None):
    # the E4M3 epilogue's own checker: robust codes exact, every code within
    # half a step, scales to rtol 1e-5
    from test_gpu_fp8 import run
    run(inp["x"], inp["r"], inp["w"], eps, what, group=group)


def _mxfp4_rows(inp, eps, what):
    from test_gpu_mxfp4 import run as run_mx
    run_mx(inp["x"], inp["r"], inp["w"], eps, what)


# ---- persistent forward grid: many rows per block -----------------------------

@pytest.mark.parametrize("per_cu", [1, 2])
@pytest.mark.parametrize("wpr", [1, 2, 8, 16])
def test_forward_persistent_grid_many_rows_per_block(knobs, per_cu, wpr):
    knobs.setenv("ADDRMS_BLOCKS_PER_CU", per_cu)
    knobs.setenv("ADDRMS_FWD_WPR", wpr)
    # 2087 rows on 256 or 512 blocks: 4 to 9 rows per block (4 per step with
    # one wave per row), and a last sweep that leaves some blocks idle
    M, N = 2087, 4096
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=wpr + 10 * per_cu, r_std=0.5)
    what = f"blocks/CU={per_cu} wpr={wpr}"
    _fused_rms(inp, 1e-6, what)
    _fused_ln(inp, 1e-5, what)
    _fp8_rows(inp, 1e-6, what)
    _fp8_rows(inp, 1e-6, what + " group 128", group=128)
    _mxfp4_rows(inp, 1e-6, what)


@pytest.mark.parametrize("dtype,wdtype", [(torch.float32, torch.float32),
                                          (torch.bfloat16, torch.float32)])
def test_forward_persistent_grid_other_dtypes(knobs, dtype, wdtype):
    knobs.setenv("ADDRMS_BLOCKS_PER_CU", 1)
    inp = synth.add_rmsnorm_fwd_inputs(3001, 2048, dtype, wdtype, seed=21)
    _fused_rms(inp, 1e-6, f"{dtype} w {wdtype}")


# ---- target vectors per lane ---------------------------------------------------

@pytest.mark.parametrize("vpl", [1, 3, 4, 8])
@pytest.mark.parametrize("N", [4096, 7168, 16384])
def test_forward_vectors_per_lane(knobs, vpl, N):
    knobs.setenv("ADDRMS_FWD_VPL", vpl)
    inp = synth.add_rmsnorm_fwd_inputs(129, N, torch.bfloat16, seed=vpl * N, r_std=0.5)
    _fused_rms(inp, 1e-6, f"vpl={vpl} N={N}")
    _fp8_rows(inp, 1e-6, f"vpl={vpl} N={N}")


# ---- few dw partial rows ---------------------------------------------------------

@pytest.mark.parametrize("cap", [1, 3, 100])
@pytest.mark.parametrize("M,N", [(2000, 4096), (333, 1000)])
def test_backward_few_partial_rows(knobs, cap, M, N):
    knobs.setenv("ADDRMS_MAX_PARTIALS", cap)
    inp = synth.rmsnorm_bwd_inputs(M, N, torch.bfloat16, seed=cap + N)
    dy, x, w = inp["dy"], inp["x"], inp["w"]
    rstd = by_rows(oracle.rmsnorm_fwd, x, w, 1e-6)[1]
    what = f"cap={cap} {M}x{N}"
    # RMS backward
    dx, dw = ar.rmsnorm_bwd(dy.to(DEV), x.to(DEV), w.to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    rdx, rdw, mag = oracle.rmsnorm_bwd(dy, x, w, rstd)
    assert_close(dx.cpu(), rdx, f"dx {what}")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw {what}")
    # fused backward (dres added)
    dres = synth.store(synth.normal(cap, "dres", (M, N)), torch.bfloat16)
    dh, dw = ar.add_rmsnorm_bwd(dy.to(DEV), dres.to(DEV), x.to(DEV), w.to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    rdh, rdw, mag = oracle.add_rmsnorm_bwd(dy, dres, x, w, rstd)
    assert_close(dh.cpu(), rdh, f"dh {what}")
    assert_dw_close(dw.cpu(), rdw, mag, f"fused dw {what}")
    # LayerNorm backward (dw and db partials side by side in the workspace)
    _, mean, lrstd = by_rows(oracle.layernorm_fwd, x, w, None, 1e-5)
    dx, dw, db = ar.layernorm_bwd(dy.to(DEV), x.to(DEV), w.to(DEV), mean.to(DEV), lrstd.to(DEV))
    torch.cuda.synchronize()
    rdx, rdw, rdb, mw, mb = oracle.layernorm_bwd(dy, x, w, mean, lrstd)
    assert_close(dx.cpu(), rdx, f"ln dx {what}")
    assert_dw_close(dw.cpu(), rdw, mw, f"ln dw {what}")
    assert_dw_close(db.cpu(), rdb, mb, f"ln db {what}")


# ---- RMSNorm + RoPE on a capped grid ----------------------------------------------

@pytest.mark.parametrize("per_cu", [1, 2])
@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_capped_grid(knobs, per_cu, interleaved):
    from test_gpu_rope import run_packed
    knobs.setenv("ADDRMS_ROPE_BLOCKS_PER_CU", per_cu)
    # 2051 tokens x 40 heads of 128: 641 steps of 128 heads on 256 or 512
    # blocks, so blocks loop two or three times
    run_packed(2051, 32, 8, 128, torch.bfloat16, torch.bfloat16, interleaved, seed=per_cu)
