"""The no-allocation backward (rmsnorm_bwd_noalloc, dw partials in the
library's own device scratch) against rmsnorm_bwd with a caller's workspace,
through the C ABI: dx bit for bit, dw bit for bit where both use the same
partial rows and within the dw tolerance where the scratch holds fewer.
Several calls in a row with shrinking inputs, so each call runs over the
scratch contents the previous one left."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import synth
from parity import assert_bits_equal, assert_dw_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCRATCH = 16 << 20


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _case(M, N, dtype, wdtype, seed):
    inp = synth.rmsnorm_bwd_inputs(M, N, dtype, wdtype, seed=seed)
    dy, x, w = (inp[k].to(DEV) for k in ("dy", "x", "w"))
    _, rstd = ar.rmsnorm_fwd(x, w, 1e-6, return_rstd=True)
    return dy, x, w, rstd


def _mag(dy, x, rstd):
    """sum_i |dy_ij * x_ij * rstd_i| per column, binary64 on the host."""
    t = dy.cpu().double() * x.cpu().double() * rstd.cpu().double()[:, None]
    return t.abs().sum(0)


def _compare(M, N, dtype, wdtype, seed, same_partials):
    dy, x, w, rstd = _case(M, N, dtype, wdtype, seed)
    # reference: the workspace entry point, with its own workspace
    dx_ref, dw_ref = ar.rmsnorm_bwd(dy, x, w, rstd)
    # outputs preallocated and poisoned, so the call under test allocates nothing
    dx = torch.full_like(x, float("nan"))
    dw = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    ar.rmsnorm_bwd_noalloc(dy, x, w, rstd, dx=dx, dw=dw)
    torch.cuda.synchronize()
    assert_bits_equal(dx, dx_ref, f"dx {M}x{N}")
    if same_partials:
        assert_bits_equal(dw, dw_ref, f"dw {M}x{N}")
    else:
        assert_dw_close(dw.cpu(), dw_ref.cpu(), _mag(dy, x, rstd), f"dw {M}x{N}")
    assert np.isfinite(dw.cpu().numpy()).all()


def test_noalloc_matches_workspace_entry_point():
    # 1. the backward workload (1024 partial rows of 4096 fit: same grid and
    #    the same partial rows as the workspace path)
    _compare(32768, 4096, torch.bfloat16, torch.bfloat16, 1, same_partials=True)
    # 2. smaller, wider rows: 585 rows of 7168 fit in the scratch
    _compare(8192, 7168, torch.bfloat16, torch.bfloat16, 2, same_partials=False)
    # 3. smaller still, rows too wide for the workspace path's grid to fit
    #    the scratch (256 partial rows of 16384)
    _compare(2048, 16384, torch.bfloat16, torch.float32, 3, same_partials=False)
    # 4. the element-wise path (N not a whole number of 16-byte vectors):
    #    row chunks of 2 instead of 1
    _compare(700, 7170, torch.bfloat16, torch.bfloat16, 4, same_partials=False)
    # 5. float32 rows, small
    _compare(300, 2048, torch.float32, torch.float32, 5, same_partials=True)


def test_noalloc_twice_in_a_row_shrinking():
    # the second call is smaller and must not see the first one's partial rows
    _compare(4096, 4096, torch.bfloat16, torch.bfloat16, 6, same_partials=True)
    _compare(33, 4096, torch.bfloat16, torch.bfloat16, 7, same_partials=True)


def test_noalloc_empty_batch_writes_zero_dw():
    N = 4096
    w = torch.ones(N, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(0, N, dtype=torch.bfloat16, device=DEV)
    dw = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    ar.rmsnorm_bwd_noalloc(e, e, w, torch.empty(0, device=DEV), dx=torch.empty_like(e), dw=dw)
    torch.cuda.synchronize()
    assert torch.equal(dw.cpu(), torch.zeros(N))
