"""GPU parity of the backward launch shapes the dispatcher takes from its
measured table (at least 32 rows per CU, 2 blocks per CU): the
RMS, fused RMS, LayerNorm and fused LayerNorm backwards at widths in each of
the table's ranges (257-384, 385-448 and 449-512 vectors a row, and for the
RMS backward 641-768 and 961-1024), against the CPU oracle through the C ABI.
dx (dh) to the bf16, float16 or float32 tolerance, dw and db to the dw
tolerance.  8192 rows fill 32 rows per CU on a 256-CU device, the table's
threshold; the float16 cases take the same shapes, and float32 rows their
own entries (193-384, 449-512 and 961-1024 vectors)."""
import sys

import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_close, assert_dw_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
M = 8192


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _inputs(N, dtype, seed):
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, seed=seed, r_std=0.5)
    dy = synth.store(synth.normal(seed, "dy", (M, N)), dtype)
    dres = synth.store(synth.normal(seed + 1, "dy", (M, N)), dtype)
    return inp["x"], inp["w"], dy, dres


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("N", [2560, 3584, 4096, 6144, 8192])
def test_rms(dtype, N):
    x, w, dy, _ = _inputs(N, dtype, N)
    rstd = by_rows(oracle.rmsnorm_fwd, x, w, 1e-6)[1]
    dx, dw = ar.rmsnorm_bwd(dy.to(DEV), x.to(DEV), w.to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    rdx, rdw, mag = oracle.rmsnorm_bwd(dy, x, w, rstd)
    assert_close(dx.cpu(), rdx, f"dx {M}x{N}")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw {M}x{N}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("N", [3072, 3584, 4096])
def test_fused_rms(dtype, N):
    x, w, dy, dres = _inputs(N, dtype, N + 1)
    rstd = by_rows(oracle.rmsnorm_fwd, x, w, 1e-6)[1]
    dh, dw = ar.add_rmsnorm_bwd(dy.to(DEV), dres.to(DEV), x.to(DEV), w.to(DEV), rstd.to(DEV))
    torch.cuda.synchronize()
    rdh, rdw, mag = oracle.add_rmsnorm_bwd(dy, dres, x, w, rstd)
    assert_close(dh.cpu(), rdh, f"dh {M}x{N}")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw {M}x{N}")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("N", [1024, 1536, 2048, 4096])
def test_float32_rows(fused, N):
    # float32 rows: 2 waves with the prefetch at 257 to 384 vectors (and for
    # the fused forms at 193 to 256), 8 waves at 449 to 512 and (the RMS
    # backwards) 961 to 1024
    x, w, dy, dres = _inputs(N, torch.float32, N + 3)
    rstd = by_rows(oracle.rmsnorm_fwd, x, w, 1e-6)[1]
    g = lambda t: t.to(DEV)
    if fused:
        dx, dw = ar.add_rmsnorm_bwd(g(dy), g(dres), g(x), g(w), g(rstd))
        rdx, rdw, mag = oracle.add_rmsnorm_bwd(dy, dres, x, w, rstd)
    else:
        dx, dw = ar.rmsnorm_bwd(g(dy), g(x), g(w), g(rstd))
        rdx, rdw, mag = oracle.rmsnorm_bwd(dy, x, w, rstd)
    torch.cuda.synchronize()
    assert_close(dx.cpu(), rdx, f"dx {M}x{N} float32")
    assert_dw_close(dw.cpu(), rdw, mag, f"dw {M}x{N} float32")
    _, mean, lrstd = by_rows(oracle.layernorm_fwd, x, w, None, 1e-5)
    if fused:
        dx, dw, db = ar.add_layernorm_bwd(g(dy), g(dres), g(x), g(w), g(mean), g(lrstd))
        rdx, rdw, rdb, mw, mb = oracle.add_layernorm_bwd(dy, dres, x, w, mean, lrstd)
    else:
        dx, dw, db = ar.layernorm_bwd(g(dy), g(x), g(w), g(mean), g(lrstd))
        rdx, rdw, rdb, mw, mb = oracle.layernorm_bwd(dy, x, w, mean, lrstd)
    torch.cuda.synchronize()
    assert_close(dx.cpu(), rdx, f"LayerNorm dx {M}x{N} float32")
    assert_dw_close(dw.cpu(), rdw, mw, f"LayerNorm dw {M}x{N} float32")
    assert_dw_close(db.cpu(), rdb, mb, f"LayerNorm db {M}x{N} float32")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("N", [2560, 3584, 4096])
def test_layernorm(fused, N):
    x, w, dy, dres = _inputs(N, torch.bfloat16, N + 2)
    _, mean, rstd = by_rows(oracle.layernorm_fwd, x, w, None, 1e-5)
    g = lambda t: t.to(DEV)
    if fused:
        dx, dw, db = ar.add_layernorm_bwd(g(dy), g(dres), g(x), g(w), g(mean), g(rstd))
        rdx, rdw, rdb, mw, mb = oracle.add_layernorm_bwd(dy, dres, x, w, mean, rstd)
    else:
        dx, dw, db = ar.layernorm_bwd(g(dy), g(x), g(w), g(mean), g(rstd))
        rdx, rdw, rdb, mw, mb = oracle.layernorm_bwd(dy, x, w, mean, rstd)
    torch.cuda.synchronize()
    assert_close(dx.cpu(), rdx, f"dx {M}x{N}")
    assert_dw_close(dw.cpu(), rdw, mw, f"dw {M}x{N}")
    assert_dw_close(db.cpu(), rdb, mb, f"db {M}x{N}")
