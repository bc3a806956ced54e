"""GPU parity of the MXFP4-output RMSNorm (rmsnorm_fwd_mxfp4 /
add_rmsnorm_fwd_mxfp4 through the C ABI) against the CPU oracle.

The residual is compared bit for bit. The GPU computes y in float32; the
oracle rounds a binary64 y once to float32. Their block scales and element
codes can therefore differ only where a decision is within a relative 2^-20
of its boundary: a block maximum next to a power of two (the scale), or a
scaled value next to an E2M1 midpoint (the code). Every decision away from a
boundary must match exactly. Every scale must be within one of the oracle's.
Every element must decode, at the GPU's own scale, to within half a grid
step of the binary64 y (or to +-6 times the scale when saturated). NaN rows
give NaN scales (0xFF) and zero codes.

At 16384x7168 the GPU runs the whole matrix and 2048 of its rows (the first
and last 64, the rest seeded random) are checked against the oracle."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_bits_equal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REL = 2.0 ** -20


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def check_mx(q_gpu, s_gpu, q_ref, s_ref, y64, what):
    assert q_gpu.dtype == torch.float4_e2m1fn_x2 and s_gpu.dtype == torch.float8_e8m0fnu
    # the scale bytes decode through torch's own E8M0 type as 2^(byte - 127)
    sb = s_gpu.view(torch.uint8).cpu().numpy().astype(np.int64)
    with np.errstate(invalid="ignore"):     # byte 255 is E8M0's NaN, left out below
        sf = s_gpu.cpu().float().numpy().astype(np.float64)
    fin = sb != 255
    np.testing.assert_array_equal(sf[fin], np.exp2(sb[fin] - 127.0))
    codes = oracle.unpack_fp4(q_gpu.view(torch.uint8).cpu())
    rcodes = oracle.unpack_fp4(q_ref)
    rs = s_ref.numpy().astype(np.int64)
    y = y64.numpy()
    M, N = y.shape
    nb = (N + 31) // 32
    assert sb.shape == rs.shape == (M, nb)
    nanrow = np.isnan(y).any(axis=1)
    assert np.all(sb[nanrow] == 255) and np.all(codes[nanrow] == 0), f"NaN rows {what}"
    assert np.all(sb[~nanrow] != 255), f"finite rows {what}"
    yf = y.astype(np.float32).astype(np.float64)
    blk = np.arange(N) // 32
    for b in range(nb):
        cols = blk == b
        amax = np.abs(yf[:, cols]).max(axis=1)
        e_lo = np.floor(np.log2(np.maximum(amax * (1 - REL), 1e-300)))
        e_hi = np.floor(np.log2(np.maximum(amax * (1 + REL), 1e-300)))
        robust = (e_lo == e_hi) | (amax == 0)
        ok = ~nanrow
        bad = ok & robust & (sb[:, b] != rs[:, b])
        assert not bad.any(), (f"scales {what}: block {b}, rows {np.nonzero(bad)[0][:5]}, "
                               f"gpu {sb[bad, b][:5]} ref {rs[bad, b][:5]}")
        assert np.all(np.abs(sb[ok, b] - rs[ok, b]) <= 1), f"scales {what}: block {b} off by > 1"
        # codes: exact where the block scale agrees and the scaled value is not
        # next to a midpoint
        X = np.exp2(rs[:, b] - 127.0)[:, None]
        v = yf[:, cols] / X
        lo = oracle.fp4e2m1_encode(v * (1 - REL))
        hi = oracle.fp4e2m1_encode(v * (1 + REL))
        same = (sb[:, b] == rs[:, b])[:, None] & (lo == hi) & ok[:, None]
        cg, cr = codes[:, cols], rcodes[:, cols]
        canon = lambda c: np.where((c & 0x7) == 0, 0, c)   # a zero may carry either sign
        mism = same & (canon(cg) != canon(cr))
        assert not mism.any(), (f"codes {what}: block {b}, {int(mism.sum())} differ; "
                                f"first gpu {cg[mism][0]:#x} ref {cr[mism][0]:#x}")
        # every element at the GPU's own scale
        Xg = np.exp2(sb[:, b] - 127.0)[:, None]
        vg = y[:, cols] / Xg
        deq = oracle.fp4e2m1_decode(cg)
        spacing = np.where(np.abs(vg) < 2, 0.5, np.where(np.abs(vg) < 4, 1.0, 2.0))
        sat = np.abs(vg) > 6
        err_ok = np.where(sat, deq == np.sign(vg) * 6,
                          np.abs(deq - vg) <= spacing / 2 * (1 + 1e-5) + 1e-5 * np.abs(vg))
        assert np.all(err_ok[ok]), f"dequantised {what}: block {b}"


def run(x, r, w, eps, what, rows=None):
    """The GPU over all of x (and r); the oracle over all rows, or over the
    rows `rows` only, compared with the same rows of the GPU's outputs."""
    g = lambda t: t.to(DEV)
    pick = (lambda t: t) if rows is None else (lambda t: t[rows.to(t.device)])
    xs, rs_ = pick(x), None if r is None else pick(r)
    if r is None:
        q, s = ar.rmsnorm_fwd_mxfp4(g(x), g(w), eps)
        qr, sr, _ = by_rows(oracle.rmsnorm_fwd_mxfp4, xs, w, eps)
        y64, _ = by_rows(oracle.rmsnorm_fwd, xs, w, eps, y_dtype=torch.float64)
    else:
        q, s, res = ar.add_rmsnorm_fwd_mxfp4(g(x), g(r), g(w), eps)
        qr, sr, rres, _ = by_rows(oracle.rmsnorm_fwd_mxfp4, xs, w, eps, residual=rs_)
        torch.cuda.synchronize()
        assert_bits_equal(pick(res).cpu(), rres, f"residual_out {what}")
        y64, _ = by_rows(oracle.rmsnorm_fwd, rres, w, eps, y_dtype=torch.float64)
    torch.cuda.synchronize()
    # index the codes and scales as bytes (4- and 8-bit float tensors need
    # not support indexing)
    q = pick(q.view(torch.uint8)).view(q.dtype)
    s = pick(s.view(torch.uint8)).view(s.dtype)
    check_mx(q, s, qr, sr, y64, what)


@pytest.mark.parametrize("fused", [True, False])
def test_full_shape(fused):
    # the whole matrix on the GPU, in the launch the library takes for this
    # shape; 2048 rows checked against the oracle (every row is computed on
    # its own)
    from test_gpu_fp8 import sample_rows
    inp = synth.add_rmsnorm_fwd_inputs(16384, 7168, torch.bfloat16, seed=91, r_std=0.5)
    run(inp["x"], inp["r"] if fused else None, inp["w"], 1e-6, "16384x7168",
        rows=sample_rows(16384, seed=91))


@pytest.mark.parametrize("fused", [True, False])
def test_four_waves_of_three(fused):
    # 513 to 640 vectors a row with 8 or more rows per CU: 4 waves of 3
    # vectors a lane
    inp = synth.add_rmsnorm_fwd_inputs(2048, 4608, torch.bfloat16, seed=93, r_std=0.5)
    run(inp["x"], inp["r"] if fused else None, inp["w"], 1e-6, "2048x4608")


@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.float32, torch.float32),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("N", [32, 48, 64, 1000, 4096, 8192, 16384, 24576, 65536])
def test_shapes_and_dtypes(dtype, wdtype, N):
    # 48 and 1000: a ragged last block; 65536: more than 4 vectors per lane,
    # the element-wise path
    M = max(2, min(40, (1 << 20) // N))
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=N + 7)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"{dtype} N={N}")


@pytest.mark.parametrize("M", [1, 32, 512])
def test_decode_with_outliers(M):
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_decode_n8192", M=M)
    run(inp["x"], inp["r"], inp["w"], 1e-5, f"decode M={M}")


@pytest.mark.parametrize("wpr", [1, 2, 4, 8, 16])
def test_forced_waves_per_row(knobs, wpr):
    knobs.setenv("ADDRMS_FWD_WPR", str(wpr))
    inp = synth.add_rmsnorm_fwd_inputs(37, 4096, torch.bfloat16, seed=wpr + 90)
    run(inp["x"], inp["r"], inp["w"], 1e-6, f"wpr={wpr}")


def test_elementwise_forced(knobs):
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    inp = synth.add_rmsnorm_fwd_inputs(13, 4096, torch.bfloat16, seed=93)
    run(inp["x"], inp["r"], inp["w"], 1e-6, "elem")
    run(inp["x"], None, inp["w"], 1e-6, "elem plain")


def test_special_rows():
    N = 1024
    inp = synth.add_rmsnorm_fwd_inputs(4, N, torch.bfloat16, seed=95)
    x = inp["x"].clone()
    x[0] = 0                   # zero row: every scale 2^-127 (byte 0), codes 0
    x[1, 77] = float("nan")    # NaN row
    x[2] = 2.0                 # constant row
    q, s = ar.rmsnorm_fwd_mxfp4(x.to(DEV), inp["w"].to(DEV), 1e-6)
    torch.cuda.synchronize()
    sb = s.view(torch.uint8).cpu()
    qb = q.view(torch.uint8).cpu()
    assert torch.all(sb[0] == 0) and torch.all(qb[0] == 0)
    assert torch.all(sb[1] == 255) and torch.all(qb[1] == 0)
    run(x, None, inp["w"], 1e-6, "special rows")


def test_custom_ops_match_the_binding():
    import add_rmsnorm_amd.autograd as ag
    inp = synth.add_rmsnorm_fwd_inputs(64, 4096, torch.bfloat16, seed=97)
    x, r, w = (inp[k].to(DEV) for k in ("x", "r", "w"))
    a = ar.add_rmsnorm_fwd_mxfp4(x, r, w, 1e-6)
    b = ag.add_rms_norm_mxfp4(x, r, w, 1e-6)
    c = ag.rms_norm_mxfp4(x, w, 1e-6)
    d = ar.rmsnorm_fwd_mxfp4(x, w, 1e-6)
    torch.cuda.synchronize()
    for u, v in list(zip(a, b)) + list(zip(c, d)):
        assert u.dtype == v.dtype and torch.equal(u.view(torch.uint8), v.view(torch.uint8))


def _tie_rows(dtype):
    """Two rows of 512 columns whose y is exact on both sides, so that every
    E2M1 decision, ties included, must match bit for bit: block 0 holds the
    seven E2M1 midpoints and their negatives (scale 2^0), block 1 twice them
    (2^1), block 2 sixteen times them (2^4), block 3 grid points, values just
    off midpoints and a saturating 7; the rest are zeros.  eps tops the mean
    square up to 4^k and w = 2^k, so rstd = 2^-k and y = x exactly."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    row = np.zeros(512)
    row[0:14] = mids + [-m for m in mids]
    row[32:46] = [2 * m for m in mids] + [-2 * m for m in mids]
    row[64:78] = [16 * m for m in mids] + [-16 * m for m in mids]
    row[96:112] = [0.5, 1, 1.5, 2, 3, 4, 6, 7, -0.5, -1, -3, -6, 0.3125, 0.6875, 2.25, -4.5]
    ms = float((row ** 2).sum() / row.size)
    k = 0
    while 4.0 ** k < ms:
        k += 1
    eps = 4.0 ** k - ms
    assert np.float32(eps) == eps and np.float32(ms) == ms
    x = torch.tensor(np.stack([row, -row]), dtype=torch.float64).to(dtype)
    assert torch.equal(x.double(), torch.tensor(np.stack([row, -row])))
    w = torch.full((512,), 2.0 ** k, dtype=dtype)
    return x, w, eps


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("force_elem", ["0", "1"])
@pytest.mark.parametrize("fused", [False, True])
def test_e2m1_ties_exact(knobs, dtype, force_elem, fused):
    """Round-half-to-even and saturation of the E2M1 encoding (on the GPU the
    hardware conversion), bit for bit against the oracle."""
    knobs.setenv("ADDRMS_FORCE_ELEM", force_elem)
    x, w, eps = _tie_rows(dtype)
    if fused:
        r = torch.zeros_like(x)
        q, s, res = ar.add_rmsnorm_fwd_mxfp4(x.to(DEV), r.to(DEV), w.to(DEV), eps)
        qr, sr, _, _ = by_rows(oracle.rmsnorm_fwd_mxfp4, x, w, eps, residual=r)
    else:
        q, s = ar.rmsnorm_fwd_mxfp4(x.to(DEV), w.to(DEV), eps)
        qr, sr, _ = by_rows(oracle.rmsnorm_fwd_mxfp4, x, w, eps)
    torch.cuda.synchronize()
    sb = s.view(torch.uint8).cpu()
    assert torch.equal(sb, sr), (sb[:, :4], sr[:, :4])
    assert list(sr[0, :4]) == [127, 128, 131, 127]
    codes = oracle.unpack_fp4(q.view(torch.uint8).cpu())
    rcodes = oracle.unpack_fp4(qr)
    assert np.array_equal(codes, rcodes), np.nonzero(codes != rcodes)
    # the ties themselves, read from the pages' grid: 0.25 -> 0, 0.75 -> 1.0,
    # 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0
    assert list(codes[0, :7]) == [0, 2, 2, 4, 4, 6, 6]
    assert list(codes[0, 7:14]) == [8, 10, 10, 12, 12, 14, 14]
    assert list(codes[1, :7]) == [8, 10, 10, 12, 12, 14, 14]
