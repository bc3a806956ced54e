"""GPU parity of the FP8-output RMSNorm (rmsnorm_fwd_fp8 / add_rmsnorm_fwd_fp8
through the C ABI) against the CPU oracle on seeded inputs.

The residual is compared bit for bit and the per-row scale to rtol 1e-5.  The
oracle's codes are E4M3(y / scale) of the binary64 y and its stored scale;
the GPU's are E4M3(y * (448 / amax)) in float32.  Both values agree to about
1e-6 relative, so the codes can differ only where the oracle's scaled value
v = y / scale lies within 2^-15 (relative) of an E4M3 rounding boundary:
every code whose value is not that close must match exactly, and every code,
close or not, must decode to within half an E4M3 step (times the scale) of
the binary64 y.

At 16384x7168 the GPU runs the whole matrix, in the launch the library takes
for that shape, and 2048 of its rows (the first and last 64, the rest seeded
random) are checked against the oracle; smaller shapes are checked whole."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
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


def check_codes(q_gpu, s_gpu, q_ref, s_ref, y64, what, group=None):
    q = q_gpu.view(torch.uint8).cpu().numpy().astype(np.uint8)
    qr = q_ref.numpy()
    sg = s_gpu.cpu().numpy().astype(np.float64)
    sr = s_ref.numpy().astype(np.float64)
    assert sg.shape == sr.shape, (sg.shape, sr.shape)
    np.testing.assert_allclose(sg, sr, rtol=1e-5, err_msg=f"scale {what}")
    y = y64.numpy()
    M, N = y.shape
    # each element's group: the whole row, or `group` consecutive columns
    cols = np.arange(N) // group if group else np.zeros(N, dtype=np.int64)
    se = (sg if sg.ndim == 2 else sg[:, None])[:, cols]
    nan = np.isnan(y)
    assert np.array_equal((q & 0x7F) == 0x7F, nan), f"NaN codes {what}"
    # the oracle's scaled values, and whether a tiny relative change of them
    # changes the code (a rounding boundary within reach)
    sre = (sr if sr.ndim == 2 else sr[:, None])[:, cols]
    v = np.where(nan, 0.0, y) / sre
    lo = oracle.fp8e4m3_encode(v * (1 - 2.0 ** -15))
    hi = oracle.fp8e4m3_encode(v * (1 + 2.0 ** -15))
    robust = (lo == hi) & ~nan
    bad = np.nonzero(robust & (q != qr))
    assert bad[0].size == 0, (f"codes {what}: {bad[0].size} robust codes differ, first at "
                              f"{bad[0][0], bad[1][0]}: gpu {q[bad][0]:#04x} ref {qr[bad][0]:#04x}")
    ok = ~nan
    deq = oracle.fp8e4m3_decode(q[ok]) * se[ok]
    mag = np.abs(y[ok]) / se[ok]
    step = np.where(mag < 2.0 ** -6, 2.0 ** -9,
                    2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-30))) - 3))
    lim = (0.5 * step * (1 + 1e-5) + 1e-5 * mag) * se[ok]
    err = np.abs(deq - y[ok])
    assert np.all(err <= lim), f"dequantised {what}: max excess {(err - lim).max()}"


def sample_rows(M, k=2048, seed=0):
    """Row indices for the full-shape cases: the first and last 64 rows and
    seeded random ones, k in all (every row is computed on its own, so a
    sample of rows checks the full launch)."""
    rng = np.random.default_rng(seed)
    rows = set(range(64)) | set(range(M - 64, M))
    while len(rows) < k:
        rows.add(int(rng.integers(0, M)))
    return torch.tensor(sorted(rows))


def run(x, r, w, eps, what, group=None, rows=None):
    """The GPU over all of x (and r); the oracle over all rows, or over the
    rows `rows` only, compared with the same rows of the GPU's outputs."""
    g = lambda t: t.to(DEV)
    pick = (lambda t: t) if rows is None else (lambda t: t[rows.to(t.device)])
    xs, rs_ = pick(x), None if r is None else pick(r)
    if r is None:
        q, s = ar.rmsnorm_fwd_fp8(g(x), g(w), eps, group=group)
        qr, sr, _ = by_rows(oracle.rmsnorm_fwd_fp8, xs, w, eps, group=group or 0)
        y64, _ = by_rows(oracle.rmsnorm_fwd, xs, w, eps, y_dtype=torch.float64)
    else:
        q, s, res = ar.add_rmsnorm_fwd_fp8(g(x), g(r), g(w), eps, group=group)
        qr, sr, rres, _ = by_rows(oracle.rmsnorm_fwd_fp8, xs, w, eps, residual=rs_, group=group or 0)
        torch.cuda.synchronize()
        assert_bits_equal(pick(res).cpu(), rres, f"residual_out {what}")
        y64, _ = by_rows(oracle.rmsnorm_fwd, rres, w, eps, y_dtype=torch.float64)
    torch.cuda.synchronize()
    # index the codes as bytes (float8 tensors need not support indexing)
    q, s = pick(q.view(torch.uint8)).view(q.dtype), pick(s)
    assert q.dtype == torch.float8_e4m3fn
    N = x.shape[-1]
    check_codes(q, s, qr, sr, y64, what, group if group and group < N else None)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("M,N", [(16384, 7168), (4096, 4096), (33, 1032)])
def test_fp8_bf16(fused, M, N):
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=M + N, r_std=0.5)
    rows = sample_rows(M) if M * N > (1 << 25) else None
    run(inp["x"], inp["r"] if fused else None, inp["w"], 1e-6, f"{M}x{N}", rows=rows)


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
def test_fp8_forced_waves_per_row(knobs, wpr):
    knobs.setenv("ADDRMS_FWD_WPR", str(wpr))
    inp = synth.add_rmsnorm_fwd_inputs(37, 4096, torch.bfloat16, seed=wpr)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"wpr={wpr}")


@pytest.mark.parametrize("N", [1, 7, 65, 8193])
def test_fp8_edge_and_elementwise(knobs, N):
    inp = synth.add_rmsnorm_fwd_inputs(17, N, torch.bfloat16, seed=N)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"N={N}")
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
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
    y, _ = by_rows(oracle.rmsnorm_fwd, x[3:4], inp["w"], 1e-6, y_dtype=torch.float32)
    assert_close(deq, y[0], "dequantised row", atol=float(s[3]) * 2.0 ** -9, rtol=0.07)


@pytest.mark.parametrize("fused", [False, True])
def test_fp8_infinite_rows(fused):
    """A row holding +-Inf: rstd is 0, so y is NaN there and a zero of either
    sign elsewhere; the row's scale stays 1 (no finite nonzero y), as in the
    oracle."""
    N = 4096
    inp = synth.add_rmsnorm_fwd_inputs(2, N, torch.bfloat16, seed=5)
    x = inp["x"].clone()
    x[0, 7] = float("inf")
    x[1, 9] = float("-inf")
    if fused:
        r = torch.zeros_like(x)
        q, s, _ = ar.add_rmsnorm_fwd_fp8(x.to(DEV), r.to(DEV), inp["w"].to(DEV), 1e-6)
    else:
        q, s = ar.rmsnorm_fwd_fp8(x.to(DEV), inp["w"].to(DEV), 1e-6)
    torch.cuda.synchronize()
    qr, sr = by_rows(oracle.rmsnorm_fwd_fp8, x, inp["w"], 1e-6)[:2]
    assert torch.equal(s.cpu(), sr) and torch.all(sr == 1.0)
    qb = q.view(torch.uint8).cpu().numpy() & 0x7F
    rb = qr.view(torch.uint8).numpy() & 0x7F
    assert np.array_equal(qb, rb)
    assert qb[0, 7] == 0x7F and qb[1, 9] == 0x7F and int((qb != 0).sum()) == 2


# ---- one scale per group of columns -----------------------------------------

@pytest.mark.parametrize("fused", [True, False])
def test_grouped_128_full_shape(fused):
    inp = synth.add_rmsnorm_fwd_inputs(16384, 7168, torch.bfloat16, seed=71, r_std=0.5)
    run(inp["x"], inp["r"] if fused else None, inp["w"], 1e-6, "16384x7168 g128", group=128,
        rows=sample_rows(16384, seed=71))


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("M,N", [(2048, 5120), (2048, 6144), (2048, 4608)])
def test_four_waves_of_three(fused, M, N):
    # 513 to 768 vectors a row (to 640 per row) with 8 or more rows per CU:
    # the E4M3 forwards take 4 waves of 3 vectors a lane (a group of 128
    # columns then spans lanes of one wave in a different pattern than with
    # 2 vectors)
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=M + N + 7, r_std=0.5)
    r = inp["r"] if fused else None
    run(inp["x"], r, inp["w"], 1e-6, f"{M}x{N} g128", group=128)
    if N <= 5120:
        run(inp["x"], r, inp["w"], 1e-6, f"{M}x{N} per row")


@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.float32, torch.float32),
                                          (torch.bfloat16, torch.float32)])
@pytest.mark.parametrize("group", [4, 8, 16, 32, 128, 256, 512, 100, 1, 7168, 9000])
def test_grouped_sizes(dtype, wdtype, group):
    # vector path where the group is a power of two of whole vectors (up to a
    # wave), the element-wise path otherwise; the group spanning the row is the
    # per-row scale
    inp = synth.add_rmsnorm_fwd_inputs(40, 7168, dtype, wdtype, seed=group)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"{dtype} g{group}", group=group)


@pytest.mark.parametrize("M", [1, 32, 512])
def test_grouped_decode_with_outliers(M):
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_decode_n8192", M=M)
    run(inp["x"], inp["r"], inp["w"], 1e-5, f"decode M={M} g128", group=128)


@pytest.mark.parametrize("N", [136, 1000, 4104, 24576, 65536])
def test_grouped_ragged_rows_and_long_rows(N):
    # a last group shorter than 128; rows long enough for more than 4
    # vectors per lane (65536) take the element-wise path
    inp = synth.add_rmsnorm_fwd_inputs(9 if N < 65536 else 3, N, torch.bfloat16, seed=N)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"N={N} g128", group=128)


@pytest.mark.parametrize("wpr", [1, 2, 4, 8, 16])
def test_grouped_forced_waves_per_row(knobs, wpr):
    knobs.setenv("ADDRMS_FWD_WPR", str(wpr))
    inp = synth.add_rmsnorm_fwd_inputs(37, 4096, torch.bfloat16, seed=wpr + 50)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"wpr={wpr} g128", group=128)


def test_grouped_elementwise_forced(knobs):
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    inp = synth.add_rmsnorm_fwd_inputs(11, 4096, torch.bfloat16, seed=77)
    run(inp["x"], inp["r"], inp["w"], 1e-6, "elem g128", group=128)
    run(inp["x"], None, inp["w"], 1e-6, "elem g64", group=64)


def test_grouped_special_groups():
    N = 1024
    inp = synth.add_rmsnorm_fwd_inputs(3, N, torch.bfloat16, seed=79)
    x = inp["x"].clone()
    x[0, :128] = 0            # a zero group: scale 1, codes 0
    x[1, 300] = float("nan")  # a NaN makes the whole row NaN (rstd is NaN)
    x[2, 512:640] = 2.0       # a constant group
    q, s = ar.rmsnorm_fwd_fp8(x.to(DEV), inp["w"].to(DEV), 1e-6, group=128)
    torch.cuda.synchronize()
    qb = q.view(torch.uint8).cpu()
    assert s.shape == (3, 8)
    assert s[0, 0].item() == 1.0 and torch.all(qb[0, :128] == 0)
    assert torch.isfinite(s).all()
    # NaN row: every code NaN; the maximum ignores NaNs, so every scale is 1
    assert torch.all((qb[1] & 0x7F) == 0x7F) and torch.all(s[1].cpu() == 1.0)
    # an ordinary group: its largest value encodes as +-448
    assert int((qb[0, 128:256].to(torch.int32) & 0x7F).max()) == 0x7E
    amax = 512 + int(torch.argmax(inp["w"][512:640].float().abs()))
    assert (int(qb[2, amax]) & 0x7F) == 0x7E
    run(x, None, inp["w"], 1e-6, "special groups", group=128)


def test_custom_ops_match_the_binding_and_compile():
    import add_rmsnorm_amd.autograd as ag
    inp = synth.add_rmsnorm_fwd_inputs(64, 4096, torch.bfloat16, seed=81)
    x, r, w = (inp[k].to(DEV) for k in ("x", "r", "w"))
    for group in (None, 128):
        a = ar.add_rmsnorm_fwd_fp8(x, r, w, 1e-6, group=group)
        b = ag.add_rms_norm_fp8(x, r, w, 1e-6, group=group)
        f = torch.compile(lambda x, r, w: ag.add_rms_norm_fp8(x, r, w, 1e-6, group=group),
                          backend="aot_eager", fullgraph=True)
        c = f(x, r, w)
        torch.cuda.synchronize()
        for u, v, z in zip(a, b, c):
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))
            assert torch.equal(u.view(torch.uint8), z.view(torch.uint8))
    q1, s1 = ar.rmsnorm_fwd_fp8(x, w, 1e-6)
    q2, s2 = ag.rms_norm_fp8(x, w, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8)) and torch.equal(s1, s2)
