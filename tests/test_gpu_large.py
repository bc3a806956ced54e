"""Past 2^31 elements: the forwards (plain output, E4M3, MXFP4, LayerNorm),
the backward and RMSNorm + RoPE on tensors of more than 2^31 elements (4.3
GB each in bf16), so that offsets beyond the 32-bit range are exercised,
through the C ABI.

The inputs tile seeded blocks of a prime number of rows (x: 1031 rows, r:
1033, dy: 1039), so row i of x is block row i mod 1031; a row read from
the wrong place (an offset wrapped at 32 bits, 2^19 rows of 4096 back) lands
on a different block row and fails.  Sampled rows (the first, those around
the 2^31-element boundary, the last, and seeded random ones) are compared
with the oracle row by row; dw, a sum over every row, is compared with its
definition, the column sums of dy * x * rstd taken in binary64 on the GPU in
chunks of rows."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_bits_equal, assert_close, assert_dw_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N = 4096
M = (1 << 31) // N + 1000          # 525288 rows: 2,151,579,648 elements per tensor
BX, BR, BD = 1031, 1033, 1039      # block rows (primes)


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sample_rows():
    edge = (1 << 31) // N
    rng = np.random.default_rng(7)
    rows = {0, 1, 2, edge - 1, edge, edge + 1, M - 2, M - 1}
    rows.update(int(v) for v in rng.integers(0, M, 12))
    return sorted(rows)


def _tile(block: torch.Tensor) -> torch.Tensor:
    """[M, N] on the GPU: row i is block row i mod len(block)."""
    b = block.to(DEV)
    reps = -(-M // b.shape[0])
    return b.repeat(reps, 1)[:M].contiguous()


def _blocks(dtype):
    inp = synth.add_rmsnorm_fwd_inputs(BX, N, dtype, seed=31, r_std=0.5)
    r = synth.store(synth.normal(32, "r", (BR, N), std=0.5), dtype)
    return inp["x"], r, inp["w"]


def test_fused_forward_past_2_31_elements():
    assert M * N > (1 << 31)
    bx, br, w = _blocks(torch.bfloat16)
    x, r = _tile(bx), _tile(br)
    y, res, rstd = ar.add_rmsnorm_fwd(x, r, w.to(DEV), 1e-6, return_rstd=True)
    torch.cuda.synchronize()
    rows = _sample_rows()
    idx = torch.tensor(rows, device=DEV)
    xs = torch.stack([bx[i % BX] for i in rows])
    rs_ = torch.stack([br[i % BR] for i in rows])
    ry, rres, rrstd = by_rows(oracle.add_rmsnorm_fwd, xs, rs_, w, 1e-6)
    assert_bits_equal(res[idx].cpu(), rres, "residual_out, sampled rows")
    assert_close(y[idx].cpu(), ry, "y, sampled rows")
    assert_close(rstd[idx].cpu(), rrstd, "rstd, sampled rows", atol=0, rtol=1e-5)
    # the element-wise path on the same matrices: its own row addressing
    del y, res, rstd
    with ar.tuning(FORCE_ELEM=1):
        y, res = ar.add_rmsnorm_fwd(x, r, w.to(DEV), 1e-6)
    torch.cuda.synchronize()
    assert_bits_equal(res[idx].cpu(), rres, "residual_out, element-wise path, sampled rows")
    assert_close(y[idx].cpu(), ry, "y, element-wise path, sampled rows")


def test_fused_layernorm_forward_past_2_31_elements():
    bx, br, w = _blocks(torch.bfloat16)
    b = synth.store(synth.normal(33, "b", (N,), std=0.1), torch.bfloat16)
    x, r = _tile(bx), _tile(br)
    y, res, mean, rstd = ar.add_layernorm_fwd(x, r, w.to(DEV), b.to(DEV), 1e-5, return_stats=True)
    torch.cuda.synchronize()
    rows = _sample_rows()
    idx = torch.tensor(rows, device=DEV)
    xs = torch.stack([bx[i % BX] for i in rows])
    rs_ = torch.stack([br[i % BR] for i in rows])
    ry, rres, rmean, rrstd = by_rows(oracle.add_layernorm_fwd, xs, rs_, w, b, 1e-5)
    assert_bits_equal(res[idx].cpu(), rres, "residual_out, sampled rows")
    assert_close(y[idx].cpu(), ry, "y, sampled rows")
    assert_close(mean[idx].cpu(), rmean, "mean, sampled rows", atol=1e-6, rtol=1e-5)
    assert_close(rstd[idx].cpu(), rrstd, "rstd, sampled rows", atol=0, rtol=1e-5)


def test_backward_past_2_31_elements():
    bx, _, w = _blocks(torch.bfloat16)
    bdy = synth.store(synth.normal(34, "dy", (BD, N)), torch.bfloat16)
    brstd = by_rows(oracle.rmsnorm_fwd, bx, w, 1e-6)[1]           # rstd of each x block row
    x, dy = _tile(bx), _tile(bdy)
    rstd = _tile(brstd.view(BX, 1)).view(M)
    dx, dw = ar.rmsnorm_bwd(dy, x, w.to(DEV), rstd)
    torch.cuda.synchronize()
    rows = _sample_rows()
    idx = torch.tensor(rows, device=DEV)
    rdx, _, _ = oracle.rmsnorm_bwd(torch.stack([bdy[i % BD] for i in rows]),
                                   torch.stack([bx[i % BX] for i in rows]), w,
                                   torch.stack([brstd[i % BX] for i in rows]))
    assert_close(dx[idx].cpu(), rdx, "dx, sampled rows")
    # dw_j = sum_i dy_ij * x_ij * rstd_i, and its magnitude sum_i |...|, in
    # binary64 over chunks of rows
    ref = torch.zeros(N, dtype=torch.float64, device=DEV)
    mag = torch.zeros(N, dtype=torch.float64, device=DEV)
    for r0 in range(0, M, 32768):
        r1 = min(M, r0 + 32768)
        t = dy[r0:r1].double() * x[r0:r1].double() * rstd[r0:r1].double()[:, None]
        ref += t.sum(0)
        mag += t.abs().sum(0)
        del t
    assert_dw_close(dw.cpu(), ref.cpu(), mag.cpu(), "dw over all rows")


@pytest.mark.parametrize("group", [None, 128])
def test_fp8_output_past_2_31_elements(group):
    from test_gpu_fp8 import check_codes
    bx, br, w = _blocks(torch.bfloat16)
    x, r = _tile(bx), _tile(br)
    q, s, res = ar.add_rmsnorm_fwd_fp8(x, r, w.to(DEV), 1e-6, group=group)
    torch.cuda.synchronize()
    del x, r
    rows = _sample_rows()
    idx = torch.tensor(rows, device=DEV)
    xs = torch.stack([bx[i % BX] for i in rows])
    rs_ = torch.stack([br[i % BR] for i in rows])
    qr, sr, rres, _ = by_rows(oracle.rmsnorm_fwd_fp8, xs, w, 1e-6, residual=rs_, group=group or 0)
    assert_bits_equal(res[idx].cpu(), rres, "residual_out, sampled rows")
    y64, _ = by_rows(oracle.rmsnorm_fwd, rres, w, 1e-6, y_dtype=torch.float64)
    # index the codes as bytes (float8 tensors need not support indexing)
    check_codes(q.view(torch.uint8)[idx], s[idx], qr, sr, y64, f"E4M3 group {group}, sampled rows",
                group)


def test_mxfp4_output_past_2_31_elements():
    from test_gpu_mxfp4 import check_mx
    bx, br, w = _blocks(torch.bfloat16)
    x, r = _tile(bx), _tile(br)
    q, s, res = ar.add_rmsnorm_fwd_mxfp4(x, r, w.to(DEV), 1e-6)
    torch.cuda.synchronize()
    del x, r
    rows = _sample_rows()
    idx = torch.tensor(rows, device=DEV)
    xs = torch.stack([bx[i % BX] for i in rows])
    rs_ = torch.stack([br[i % BR] for i in rows])
    qr, sr, rres, _ = by_rows(oracle.rmsnorm_fwd_mxfp4, xs, w, 1e-6, residual=rs_)
    assert_bits_equal(res[idx].cpu(), rres, "residual_out, sampled rows")
    y64, _ = by_rows(oracle.rmsnorm_fwd, rres, w, 1e-6, y_dtype=torch.float64)
    qs = q.view(torch.uint8)[idx].view(q.dtype)
    ss = s.view(torch.uint8)[idx].view(s.dtype)
    check_mx(qs, ss, qr, sr, y64, "MXFP4, sampled rows")


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_in_place_past_2_31_elements(interleaved):
    """RMSNorm + RoPE in place on a packed [T, (32 + 2*8) * 128] buffer of
    more than 2^31 elements; sampled tokens against the oracle, and the value
    heads of those tokens untouched."""
    from test_gpu_rope import references
    Hq, Hk, D = 32, 8, 128
    W = (Hq + 2 * Hk) * D
    T = (1 << 31) // W + 1000
    assert T * W > (1 << 31)
    blk = synth.rmsnorm_rope_inputs(BX, Hq, Hk, D, torch.bfloat16, seed=35, P=4096)
    pos = synth.positions(36, T, 4096)
    qkv = torch.empty(T, W, dtype=torch.bfloat16, device=DEV)
    b = blk["qkv"].to(DEV)
    for t0 in range(0, T, BX):
        n = min(BX, T - t0)
        qkv[t0:t0 + n] = b[:n]
    del b
    q = qkv[:, :Hq * D].view(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D)
    ar.rmsnorm_rope_qk(q, k, blk["wq"].to(DEV), blk["wk"].to(DEV), blk["cos"].to(DEV),
                       blk["sin"].to(DEV), pos.to(DEV), 1e-6, interleaved=interleaved,
                       q_out=q, k_out=k)
    torch.cuda.synchronize()
    edge = (1 << 31) // W
    rng = np.random.default_rng(8)
    toks = sorted({0, 1, edge - 1, edge, edge + 1, T - 2, T - 1} |
                  {int(v) for v in rng.integers(0, T, 12)})
    idx = torch.tensor(toks, device=DEV)
    got = qkv[idx].cpu()
    src = torch.stack([blk["qkv"][t % BX] for t in toks])
    sub = {"cos": blk["cos"], "sin": blk["sin"], "pos": pos[toks]}
    n = len(toks)
    rq, q64 = references(src[:, :Hq * D].reshape(n, Hq, D), blk["wq"], sub, interleaved,
                         torch.bfloat16)
    rk, k64 = references(src[:, Hq * D:(Hq + Hk) * D].reshape(n, Hk, D), blk["wk"], sub,
                         interleaved, torch.bfloat16)
    from test_gpu_rope import check
    check(got[:, :Hq * D].reshape(n, Hq, D), rq, "q, sampled tokens", q64)
    check(got[:, Hq * D:(Hq + Hk) * D].reshape(n, Hk, D), rk, "k, sampled tokens", k64)
    assert torch.equal(got[:, (Hq + Hk) * D:].view(torch.uint8),
                       src[:, (Hq + Hk) * D:].contiguous().view(torch.uint8)), "value heads changed"
