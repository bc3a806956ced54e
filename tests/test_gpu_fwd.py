"""GPU parity of the forward ops (HIP library through the C ABI) against the
CPU oracle, element by element, on seeded synthetic inputs: the five named
workloads at full size, every kernel variant, ragged and degenerate shapes,
unaligned and in-place buffers, non-finite rows, and an exhaustive sweep of
the bfloat16 residual add."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_bits_equal, assert_close, assert_correctly_rounded

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def gpu_fused(x, r, w, eps):
    y, res, rstd = ar.add_rmsnorm_fwd(x.to(DEV), r.to(DEV), w.to(DEV), eps, return_rstd=True)
    torch.cuda.synchronize()
    return y.cpu(), res.cpu(), rstd.cpu()


def gpu_plain(x, w, eps):
    y, rstd = ar.rmsnorm_fwd(x.to(DEV), w.to(DEV), eps, return_rstd=True)
    torch.cuda.synchronize()
    return y.cpu(), rstd.cpu()


def check_fused(x, r, w, eps, what=""):
    y, res, rstd = gpu_fused(x, r, w, eps)
    ry, rres, rrstd = by_rows(oracle.add_rmsnorm_fwd, x, r, w, eps)
    assert_bits_equal(res, rres, f"residual_out {what}")
    assert_close(y, ry, f"y {what}")
    assert_close(rstd, rrstd, f"rstd {what}", atol=0, rtol=1e-5)
    return y, res, rstd


def check_plain(x, w, eps, what=""):
    y, rstd = gpu_plain(x, w, eps)
    ry, rrstd = by_rows(oracle.rmsnorm_fwd, x, w, eps)
    assert_close(y, ry, f"y {what}")
    assert_close(rstd, rrstd, f"rstd {what}", atol=0, rtol=1e-5)
    return y, rstd


# ---- the named workloads, full size ----------------------------------------

def test_rmsnorm_f32_256x4096():
    inp = synth.workload_inputs("rmsnorm_fwd_f32_256x4096")
    check_plain(inp["x"], inp["w"], 1e-6)


def test_add_rmsnorm_bf16_4096x4096():
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_4096x4096")
    check_fused(inp["x"], inp["r"], inp["w"], 1e-6)


def test_add_rmsnorm_bf16_16384x7168():
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_16384x7168")
    check_fused(inp["x"], inp["r"], inp["w"], 1e-6)


@pytest.mark.parametrize("M", [1, 8, 32, 128, 512])
def test_decode_bf16_fp32_weight_n8192(M):
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_decode_n8192", M=M)
    assert inp["w"].dtype == torch.float32
    check_fused(inp["x"], inp["r"], inp["w"], 1e-5, f"M={M}")


# ---- every kernel variant ----------------------------------------------------

@pytest.mark.parametrize("wpr", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16)])
def test_forced_waves_per_row(knobs, wpr, dtype, wdtype):
    knobs.setenv("ADDRMS_FWD_WPR", str(wpr))
    for M, N in [(37, 4096), (5, 1032), (300, 512)]:
        inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=M + N)
        check_fused(inp["x"], inp["r"], inp["w"], 1e-6, f"wpr={wpr} {M}x{N}")
        check_plain(inp["x"], inp["w"], 1e-6, f"wpr={wpr} {M}x{N}")


@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.float32, torch.float32),
                                          (torch.bfloat16, torch.float32)])
@pytest.mark.parametrize("M,N", [(3, 4096), (64, 7168), (2, 8)])
def test_elementwise_path(knobs, dtype, wdtype, M, N):
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=7)
    check_fused(inp["x"], inp["r"], inp["w"], 1e-6, "elem")
    check_plain(inp["x"], inp["w"], 1e-6, "elem")


# ---- ragged and degenerate shapes ---------------------------------------------

EDGE_N = [1, 7, 8, 63, 64, 65, 520, 4095, 4096, 7168, 8192, 8193, 16384, 65536, 131080]


@pytest.mark.parametrize("N", EDGE_N)
@pytest.mark.parametrize("M", [1, 2, 1023])
def test_edge_shapes_bf16(M, N):
    if M * N > 1 << 24:
        M = max(1, (1 << 24) // N)
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=N)
    check_fused(inp["x"], inp["r"], inp["w"], 1e-6, f"{M}x{N}")


@pytest.mark.parametrize("N", [1, 3, 4, 5, 1028, 4096, 4100, 16384, 65536])
@pytest.mark.parametrize("M", [1, 513])
def test_edge_shapes_f32(M, N):
    if M * N > 1 << 23:
        M = max(1, (1 << 23) // N)
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.float32, seed=N)
    check_fused(inp["x"], inp["r"], inp["w"], 1e-6, f"{M}x{N}")
    check_plain(inp["x"], inp["w"], 1e-6, f"{M}x{N}")


def test_empty_batch():
    x = torch.empty(0, 4096, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    y, res = ar.add_rmsnorm_fwd(x, x, w)
    assert y.shape == (0, 4096) and res.shape == (0, 4096)


def test_three_dim_input_and_no_rstd():
    inp = synth.add_rmsnorm_fwd_inputs(6 * 5, 1024, torch.bfloat16, seed=3)
    x, r = inp["x"].view(6, 5, 1024), inp["r"].view(6, 5, 1024)
    y, res = ar.add_rmsnorm_fwd(x.to(DEV), r.to(DEV), inp["w"].to(DEV), 1e-6)
    ry, rres, _ = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)
    assert_bits_equal(res.cpu().view(30, 1024), rres, "residual_out")
    assert_close(y.cpu().view(30, 1024), ry, "y")


# ---- buffers: alignment and aliasing -------------------------------------------

@pytest.mark.parametrize("offset", [1, 2, 3, 5])
def test_unaligned_views_take_elementwise_path(offset):
    M, N = 33, 2048
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=offset)
    big = torch.zeros(3, M * N + 16, dtype=torch.bfloat16, device=DEV)
    x = big[0, offset:offset + M * N].view(M, N)
    r = big[1, offset:offset + M * N].view(M, N)
    x.copy_(inp["x"].to(DEV))
    r.copy_(inp["r"].to(DEV))
    out = big[2, offset:offset + M * N].view(M, N)
    y, res = ar.add_rmsnorm_fwd(x, r, inp["w"].to(DEV), 1e-6, residual_out=out)
    ry, rres, _ = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)
    assert_bits_equal(res.cpu(), rres, "residual_out")
    assert_close(y.cpu(), ry, "y")


@pytest.mark.parametrize("force_elem", ["0", "1"])
def test_in_place(knobs, force_elem):
    knobs.setenv("ADDRMS_FORCE_ELEM", force_elem)
    M, N = 257, 4096
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=11)
    ry, rres, _ = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)
    # residual_out written over r, y over x (the usual in-place residual update)
    x, r, w = inp["x"].to(DEV), inp["r"].to(DEV), inp["w"].to(DEV)
    y, res = ar.add_rmsnorm_fwd(x, r, w, 1e-6, y=x, residual_out=r)
    assert y.data_ptr() == x.data_ptr() and res.data_ptr() == r.data_ptr()
    assert_bits_equal(r.cpu(), rres, "residual_out in r")
    assert_close(x.cpu(), ry, "y in x")
    # residual over x, y over r
    x, r = inp["x"].to(DEV), inp["r"].to(DEV)
    ar.add_rmsnorm_fwd(x, r, w, 1e-6, y=r, residual_out=x)
    assert_bits_equal(x.cpu(), rres, "residual_out in x")
    assert_close(r.cpu(), ry, "y in r")
    # plain op in place
    py, _ = by_rows(oracle.rmsnorm_fwd, inp["x"], inp["w"], 1e-6)
    x = inp["x"].to(DEV)
    ar.rmsnorm_fwd(x, w, 1e-6, y=x)
    assert_close(x.cpu(), py, "rmsnorm in place")


# ---- properties the GPU path must keep ----------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N", [(512, 4096), (512, 7168), (512, 1000), (4096, 7168),
                                 (16384, 7168), (2048, 5632), (4096, 8192), (3000, 6000),
                                 (8192, 3072), (16384, 4096), (4096, 2560)])
def test_fused_equals_plain_on_residual_bit_exact(M, N, dtype):
    """The fused y is the plain forward of the stored residual, bit for bit,
    also where the two take different launch shapes (with 8 or more rows per
    CU the fused forward runs one vector a lane, in 16 waves at 601 to 1024
    vectors a row, and in 8 waves at 257 to 448 from 16 rows per CU and at
    449 to 512 from 64; the plain one two vectors a lane)."""
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, seed=13)
    y, res, rstd = gpu_fused(inp["x"], inp["r"], inp["w"], 1e-6)
    y2, rstd2 = gpu_plain(res, inp["w"], 1e-6)
    assert_bits_equal(y, y2, "y fused vs plain")
    assert torch.equal(rstd, rstd2)


def test_power_of_two_scale_identity_bit_exact():
    """y(4x; eps) == y(x; eps/16) bit for bit on the GPU too."""
    inp = synth.rmsnorm_fwd_inputs(128, 4096, torch.bfloat16, seed=17)
    x, w = inp["x"], inp["w"]
    y1, _ = gpu_plain((x.float() * 4).to(torch.bfloat16), w, 1e-6)
    y2, _ = gpu_plain(x, w, float(np.float32(1e-6)) / 16)
    assert_bits_equal(y1, y2, "scaled")


def test_deterministic():
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_4096x4096")
    a = gpu_fused(inp["x"], inp["r"], inp["w"], 1e-6)
    b = gpu_fused(inp["x"], inp["r"], inp["w"], 1e-6)
    for u, v in zip(a, b):
        assert torch.equal(u.view(-1).view(torch.uint8), v.view(-1).view(torch.uint8))


def test_nonfinite_and_zero_rows():
    M, N = 8, 4096
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=19)
    x, r = inp["x"].clone(), inp["r"].clone()
    x[1, 5] = float("nan")
    x[2, 7] = float("inf")
    r[3, 9] = float("-inf")
    x[4], r[4] = 0, 0  # zero row: y = 0
    x[5, 11], r[5, 11] = float("inf"), float("-inf")  # inf - inf = nan
    x[6] = 1e-30  # tiny row: the squares underflow float32, eps dominates
    check_fused(x, r, inp["w"], 1e-6, "nonfinite")
    check_plain(x, inp["w"], 1e-6, "nonfinite")


def test_residual_add_exhaustive_sweep():
    """Every bfloat16 pattern of x against a strided grid of r patterns
    (special values included): residual_out bit-exact to the oracle."""
    xs = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    rs = np.unique(np.concatenate([
        np.arange(0, 1 << 16, 1031, dtype=np.uint32),
        np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F,
                  0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x3B80, 0x3B7F], dtype=np.uint32)]).astype(np.uint16))
    N = 4096
    x = torch.from_numpy(np.tile(xs, rs.size).view(np.int16)).view(torch.bfloat16).view(-1, N)
    r = torch.from_numpy(np.repeat(rs, xs.size).view(np.int16)).view(torch.bfloat16).view(-1, N)
    w = torch.ones(N, dtype=torch.bfloat16)
    _, res, _ = gpu_fused(x, r, w, 1e-6)
    _, rres, _ = by_rows(oracle.add_rmsnorm_fwd, x, r, w, 1e-6)
    assert_bits_equal(res, rres, "residual sweep")


# ---- one rounding (reading R5) ---------------------------------------------------

@pytest.mark.parametrize("name,M", [("add_rmsnorm_fwd_bf16_16384x7168", None),
                                    ("add_rmsnorm_fwd_bf16_4096x4096", None),
                                    ("add_rmsnorm_fwd_bf16_decode_n8192", 512)])
def test_fused_y_is_rounded_once(name, M):
    """y within half a bf16 ulp of the binary64 value (plus float32 noise):
    h * rstd * w is rounded once, with no bf16 step in between."""
    inp = synth.workload_inputs(name, M=M)
    eps = synth.WORKLOADS[name]["eps"]
    y, _, _ = gpu_fused(inp["x"], inp["r"], inp["w"], eps)
    y64 = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], eps, y_dtype=torch.float64)[0]
    assert_correctly_rounded(y, y64, None, f"y {name}")
    yp, _ = gpu_plain(inp["x"], inp["w"], eps)
    yp64 = by_rows(oracle.rmsnorm_fwd, inp["x"], inp["w"], eps, y_dtype=torch.float64)[0]
    assert_correctly_rounded(yp, yp64, None, f"plain y {name}")
