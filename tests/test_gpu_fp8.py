"""GPU parity of the FP8-output RMSNorm (rmsnorm_fwd_fp8 / add_rmsnorm_fwd_fp8
through the C ABI) against the CPU oracle on seeded inputs.

The residual is compared bit for bit and the per-row scale to rtol 1e-5.  The
E4M3 codes are quantised values of float32 y, which the GPU and the oracle
compute with different rounding (float32 vs binary64 then one rounding), so
they can differ only where the oracle's scaled value v = y * inv lies within
2^-15 (relative) of an E4M3 rounding boundary: every code whose value is not
that close must match exactly, and every code, close or not, must decode to
within half an E4M3 step (times the scale) of the binary64 y."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
import synth
from parity import assert_bits_equal, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def check_codes(q_gpu, s_gpu, q_ref, s_ref, y64, what):
    q = q_gpu.view(torch.uint8).cpu().numpy().astype(np.uint8)
    qr = q_ref.numpy()
    sg = s_gpu.cpu().numpy().astype(np.float64)
    sr = s_ref.numpy().astype(np.float64)
    np.testing.assert_allclose(sg, sr, rtol=1e-5, err_msg=f"scale {what}")
    y = y64.numpy()
    nan = np.isnan(y)
    assert np.array_equal((q & 0x7F) == 0x7F, nan), f"NaN codes {what}"
    # the oracle's scaled values, and whether a tiny relative change of them
    # changes the code (a rounding boundary within reach)
    v = (y.astype(np.float32).astype(np.float64) * (448.0 / np.maximum(np.abs(y).max(1), 1e-300))[:, None])
    v = np.where(np.isfinite(v), v, 0.0)
    lo = oracle.fp8e4m3_encode(v * (1 - 2.0 ** -15))
    hi = oracle.fp8e4m3_encode(v * (1 + 2.0 ** -15))
    robust = (lo == hi) & ~nan
    bad = np.nonzero(robust & (q != qr))
    assert bad[0].size == 0, (f"codes {what}: {bad[0].size} robust codes differ, first at "
                              f"{bad[0][0], bad[1][0]}: gpu {q[bad][0]:#04x} ref {qr[bad][0]:#04x}")
    ok = ~nan
    deq = oracle.fp8e4m3_decode(q[ok]) * np.broadcast_to(sg[:, None], q.shape)[ok]
    mag = np.abs(y[ok]) / np.broadcast_to(sg[:, None], q.shape)[ok]
    step = np.where(mag < 2.0 ** -6, 2.0 ** -9,
                    2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-30))) - 3))
    lim = (0.5 * step * (1 + 1e-5) + 1e-5 * mag) * np.broadcast_to(sg[:, None], q.shape)[ok]
    err = np.abs(deq - y[ok])
    assert np.all(err <= lim), f"dequantised {what}: max excess {(err - lim).max()}"


def run(x, r, w, eps, what):
    g = lambda t: t.to(DEV)
    if r is None:
        q, s = ar.rmsnorm_fwd_fp8(g(x), g(w), eps)
        qr, sr, _ = oracle.rmsnorm_fwd_fp8(x, w, eps)
        y64, _ = oracle.rmsnorm_fwd(x, w, eps, y_dtype=torch.float64)
    else:
        q, s, res = ar.add_rmsnorm_fwd_fp8(g(x), g(r), g(w), eps)
        qr, sr, rres, _ = oracle.rmsnorm_fwd_fp8(x, w, eps, residual=r)
        torch.cuda.synchronize()
        assert_bits_equal(res.cpu(), rres, f"residual_out {what}")
        y64, _ = oracle.rmsnorm_fwd(rres, w, eps, y_dtype=torch.float64)
    torch.cuda.synchronize()
    assert q.dtype == torch.float8_e4m3fn
    check_codes(q, s, qr, sr, y64, what)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("M,N", [(16384, 7168), (4096, 4096), (33, 1032)])
def test_fp8_bf16(fused, M, N):
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=M + N, r_std=0.5)
    run(inp["x"], inp["r"] if fused else None, inp["w"], 1e-6, f"{M}x{N}")


@pytest.mark.parametrize("M", [1, 32, 512])
def test_fp8_decode_with_outliers(M):
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_decode_n8192", M=M)
    run(inp["x"], inp["r"], inp["w"], 1e-5, f"decode M={M}")


@pytest.mark.parametrize("dtype,wdtype", [(torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16)])
def test_fp8_float32_rows(dtype, wdtype):
    inp = synth.add_rmsnorm_fwd_inputs(300, 2048, dtype, wdtype, seed=5)
    run(inp["x"], inp["r"], inp["w"], 1e-6, str(dtype))
    run(inp["x"], None, inp["w"], 1e-6, str(dtype))


@pytest.mark.parametrize("wpr", [1, 2, 4, 8, 16])
def test_fp8_forced_waves_per_row(monkeypatch, wpr):
    monkeypatch.setenv("ADDRMS_FWD_WPR", str(wpr))
    inp = synth.add_rmsnorm_fwd_inputs(37, 4096, torch.bfloat16, seed=wpr)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"wpr={wpr}")


@pytest.mark.parametrize("N", [1, 7, 65, 8193])
def test_fp8_edge_and_elementwise(monkeypatch, N):
    inp = synth.add_rmsnorm_fwd_inputs(17, N, torch.bfloat16, seed=N)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"N={N}")
    monkeypatch.setenv("ADDRMS_FORCE_ELEM", "1")
    inp = synth.add_rmsnorm_fwd_inputs(9, 4096, torch.bfloat16, seed=N + 1)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"elem N={N}")


def test_fp8_special_rows():
    N = 4096
    inp = synth.add_rmsnorm_fwd_inputs(4, N, torch.bfloat16, seed=3)
    x = inp["x"].clone()
    x[0] = 0
    x[1, 10] = float("nan")
    x[2] = 2.0
    q, s = ar.rmsnorm_fwd_fp8(x.to(DEV), inp["w"].to(DEV), 1e-6)
    torch.cuda.synchronize()
    qb = q.view(torch.uint8).cpu()
    assert s[0].item() == 1.0 and torch.all(qb[0] == 0)
    assert s[1].item() == 1.0 and torch.all((qb[1] & 0x7F) == 0x7F)
    amax = int(torch.argmax((inp["w"].float()).abs()))
    assert (int(qb[2, amax]) & 0x7F) == 0x7E
    # dequantisation in torch agrees with the scale convention
    deq = q.float().cpu()[3] * s[3].cpu()
    y, _ = oracle.rmsnorm_fwd(x[3:4], inp["w"], 1e-6, y_dtype=torch.float32)
    assert_close(deq, y[0], "dequantised row", atol=float(s[3]) * 2.0 ** -9, rtol=0.07)
