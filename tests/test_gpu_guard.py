"""Guard bands around every output of every entry point (through the C ABI).

Each output buffer (y, residual_out, rstd, mean, E4M3 codes and scales, MXFP4
codes and E8M0 scales, dx / dh, dw, db, the backward's workspace, RoPE's
query and key outputs) is a view into a larger device allocation filled with
a seeded random byte pattern: 4 KiB before it, 4 KiB after it, and the output
region itself.  After the call
- every byte outside the output region is unchanged (no store lands before,
  after or, for RoPE's strided outputs, between the rows of an output), and
- the output region equals, bit for bit, the result of the same call into
  ordinary allocations (so every element of the output was written; the
  values themselves are checked against the oracle by the parity tests).
The inputs must also be unchanged.  Shapes are ragged: single rows, row
counts that leave a partial last block or step, widths that are not a
multiple of a vector, a wave, a block of 32 or a scale group, and outputs
offset by one element so that the element-wise path runs (the ordinary call
then takes that path too, forced by the FORCE_ELEM knob: the two paths reduce
in different orders).  rstd and mean for the backwards come from the oracle."""
import contextlib
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BAND = 4096  # bytes on each side; a multiple of 256, so offset 0 keeps 16-byte alignment


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


class Guarded:
    """An output of `shape` and `dtype` inside a banded allocation; `offset`
    bytes (a multiple of the element size) shift it off 16-byte alignment."""

    def __init__(self, shape, dtype, seed, offset=0):
        es = torch.empty(0, dtype=dtype).element_size()
        assert offset % es == 0
        nbytes = int(np.prod(shape, dtype=np.int64)) * es
        self.lo, self.hi = BAND + offset, BAND + offset + nbytes
        pattern = np.random.default_rng(seed).integers(0, 256, self.hi + BAND, dtype=np.uint8)
        self.pattern = torch.from_numpy(pattern)
        self.full = self.pattern.to(DEV)
        self.t = self.full[self.lo:self.hi].view(dtype).view(shape)

    def check(self, expect: torch.Tensor, what: str):
        full = self.full.cpu()
        for name, sl in (("before", slice(0, self.lo)), ("after", slice(self.hi, None))):
            diff = (full[sl] != self.pattern[sl]).nonzero()
            assert diff.numel() == 0, \
                f"{what}: {diff.numel()} guard bytes {name} the output changed, first at " \
                f"offset {int(diff[0]) + sl.start - self.lo} from the output's start"
        got = full[self.lo:self.hi]
        want = expect.detach().contiguous().cpu().view(-1).view(torch.uint8)
        diff = (got != want).nonzero()
        assert diff.numel() == 0, \
            f"{what}: output differs from an ordinary call at {diff.numel()} bytes, first {int(diff[0])}"


def _inputs_unchanged(before, after, what):
    for k, (a, b) in enumerate(zip(before, after)):
        assert torch.equal(a.contiguous().view(torch.uint8), b.cpu().contiguous().view(torch.uint8)), \
            f"{what}: input {k} changed"


def _dev_inputs(*ts):
    return [t.to(DEV) if t is not None else None for t in ts]


DTYPES = [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
          (torch.bfloat16, torch.float32), (torch.float16, torch.float16)]
FWD_SHAPES = [(1, 8), (37, 1000), (70, 1001), (129, 7168), (3, 16392), (1500, 2056)]


def _off(dtype, misalign):
    return torch.empty(0, dtype=dtype).element_size() if misalign else 0


def _ref(misalign):
    """Context of the ordinary calls: the element-wise path when the guarded
    outputs are off alignment (and so take it)."""
    return ar.tuning(FORCE_ELEM=1) if misalign else contextlib.nullcontext()


# ---- RMSNorm / LayerNorm forwards -----------------------------------------------------

@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("dtype,wdtype", DTYPES)
@pytest.mark.parametrize("M,N", FWD_SHAPES)
def test_norm_forwards(M, N, dtype, wdtype, misalign):
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, wdtype, seed=M + N, r_std=0.5)
    b = synth.store(synth.normal(1, "b", (N,), std=0.1), wdtype)
    x, r, w, bb = _dev_inputs(inp["x"], inp["r"], inp["w"], b)
    host = [inp["x"], inp["r"], inp["w"], b]
    o = _off(dtype, misalign)
    what = f"{M}x{N} {dtype} w {wdtype} offset {o}"
    s = M * 7 + N

    y, rstd = Guarded((M, N), dtype, s, o), Guarded((M,), torch.float32, s + 1)
    with _ref(misalign):
        ry, rrs = ar.rmsnorm_fwd(x, w, 1e-6, return_rstd=True)
    ar.rmsnorm_fwd(x, w, 1e-6, y=y.t, rstd=rstd.t)
    torch.cuda.synchronize()
    y.check(ry, "rmsnorm_fwd y " + what)
    rstd.check(rrs, "rmsnorm_fwd rstd " + what)

    y, res = Guarded((M, N), dtype, s + 2, o), Guarded((M, N), dtype, s + 3, o)
    rstd = Guarded((M,), torch.float32, s + 4)
    with _ref(misalign):
        ry, rres, rrs = ar.add_rmsnorm_fwd(x, r, w, 1e-6, return_rstd=True)
    ar.add_rmsnorm_fwd(x, r, w, 1e-6, y=y.t, residual_out=res.t, rstd=rstd.t)
    torch.cuda.synchronize()
    y.check(ry, "add_rmsnorm_fwd y " + what)
    res.check(rres, "add_rmsnorm_fwd residual_out " + what)
    rstd.check(rrs, "add_rmsnorm_fwd rstd " + what)

    y, mean = Guarded((M, N), dtype, s + 5, o), Guarded((M,), torch.float32, s + 6)
    rstd = Guarded((M,), torch.float32, s + 7)
    with _ref(misalign):
        ry, rm, rrs = ar.layernorm_fwd(x, w, bb, 1e-5, return_stats=True)
    ar.layernorm_fwd(x, w, bb, 1e-5, y=y.t, mean=mean.t, rstd=rstd.t)
    torch.cuda.synchronize()
    y.check(ry, "layernorm_fwd y " + what)
    mean.check(rm, "layernorm_fwd mean " + what)
    rstd.check(rrs, "layernorm_fwd rstd " + what)

    y, res = Guarded((M, N), dtype, s + 8, o), Guarded((M, N), dtype, s + 9, o)
    mean, rstd = Guarded((M,), torch.float32, s + 10), Guarded((M,), torch.float32, s + 11)
    with _ref(misalign):
        ry, rres, rm, rrs = ar.add_layernorm_fwd(x, r, w, bb, 1e-5, return_stats=True)
    ar.add_layernorm_fwd(x, r, w, bb, 1e-5, y=y.t, residual_out=res.t, mean=mean.t, rstd=rstd.t)
    torch.cuda.synchronize()
    y.check(ry, "add_layernorm_fwd y " + what)
    res.check(rres, "add_layernorm_fwd residual_out " + what)
    mean.check(rm, "add_layernorm_fwd mean " + what)
    rstd.check(rrs, "add_layernorm_fwd rstd " + what)
    _inputs_unchanged(host, [x, r, w, bb], what)


# ---- quantised outputs ------------------------------------------------------------------

@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("group", [None, 128, 48, 32])
@pytest.mark.parametrize("M,N", [(1, 8), (37, 1000), (70, 1001), (129, 7168), (3, 16392),
                                 (1500, 2056)])
def test_fp8_outputs(M, N, group, misalign):
    dtype = torch.bfloat16
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, seed=M + 3 * N, r_std=0.5)
    x, r, w = _dev_inputs(inp["x"], inp["r"], inp["w"])
    ns = 1 if group is None else (N + min(group, N) - 1) // min(group, N)
    sshape = (M,) if group is None else (M, ns)
    o = 1 if misalign else 0
    what = f"{M}x{N} group {group} offset {o}"
    s = M * 11 + N + (group or 0)

    q, sc, rstd = Guarded((M, N), torch.uint8, s, o), Guarded(sshape, torch.float32, s + 1), \
        Guarded((M,), torch.float32, s + 2)
    rrs = torch.empty(M, device=DEV)
    with _ref(misalign):
        rq, rsc = ar.rmsnorm_fwd_fp8(x, w, 1e-6, group=group, rstd=rrs)
    ar.rmsnorm_fwd_fp8(x, w, 1e-6, group=group, y_fp8=q.t, y_scale=sc.t, rstd=rstd.t)
    torch.cuda.synchronize()
    q.check(rq.view(torch.uint8), "rmsnorm_fwd_fp8 codes " + what)
    sc.check(rsc, "rmsnorm_fwd_fp8 scales " + what)
    rstd.check(rrs, "rmsnorm_fwd_fp8 rstd " + what)

    q, sc = Guarded((M, N), torch.uint8, s + 3, o), Guarded(sshape, torch.float32, s + 4)
    res = Guarded((M, N), dtype, s + 5, 2 * o)
    with _ref(misalign):
        rq, rsc, rres = ar.add_rmsnorm_fwd_fp8(x, r, w, 1e-6, group=group)
    ar.add_rmsnorm_fwd_fp8(x, r, w, 1e-6, group=group, y_fp8=q.t, y_scale=sc.t,
                           residual_out=res.t)
    torch.cuda.synchronize()
    q.check(rq.view(torch.uint8), "add_rmsnorm_fwd_fp8 codes " + what)
    sc.check(rsc, "add_rmsnorm_fwd_fp8 scales " + what)
    res.check(rres, "add_rmsnorm_fwd_fp8 residual_out " + what)
    _inputs_unchanged([inp["x"], inp["r"], inp["w"]], [x, r, w], what)


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("M,N", [(1, 8), (37, 1000), (70, 1002), (129, 7168), (3, 16392),
                                 (1500, 2056)])
def test_mxfp4_outputs(M, N, misalign):
    dtype = torch.bfloat16
    inp = synth.add_rmsnorm_fwd_inputs(M, N, dtype, seed=M + 5 * N, r_std=0.5)
    x, r, w = _dev_inputs(inp["x"], inp["r"], inp["w"])
    o = 1 if misalign else 0
    what = f"{M}x{N} offset {o}"
    s = M * 13 + N
    cshape, sshape = (M, N // 2), (M, (N + 31) // 32)

    q, sc, rstd = Guarded(cshape, torch.uint8, s, o), Guarded(sshape, torch.uint8, s + 1, o), \
        Guarded((M,), torch.float32, s + 2)
    rrs = torch.empty(M, device=DEV)
    with _ref(misalign):
        rq, rsc = ar.rmsnorm_fwd_mxfp4(x, w, 1e-6, rstd=rrs)
    ar.rmsnorm_fwd_mxfp4(x, w, 1e-6, y_fp4=q.t, y_scale=sc.t, rstd=rstd.t)
    torch.cuda.synchronize()
    q.check(rq.view(torch.uint8), "rmsnorm_fwd_mxfp4 codes " + what)
    sc.check(rsc.view(torch.uint8), "rmsnorm_fwd_mxfp4 scales " + what)
    rstd.check(rrs, "rmsnorm_fwd_mxfp4 rstd " + what)

    q, sc = Guarded(cshape, torch.uint8, s + 3, o), Guarded(sshape, torch.uint8, s + 4, o)
    res = Guarded((M, N), dtype, s + 5, 2 * o)
    with _ref(misalign):
        rq, rsc, rres = ar.add_rmsnorm_fwd_mxfp4(x, r, w, 1e-6)
    ar.add_rmsnorm_fwd_mxfp4(x, r, w, 1e-6, y_fp4=q.t, y_scale=sc.t, residual_out=res.t)
    torch.cuda.synchronize()
    q.check(rq.view(torch.uint8), "add_rmsnorm_fwd_mxfp4 codes " + what)
    sc.check(rsc.view(torch.uint8), "add_rmsnorm_fwd_mxfp4 scales " + what)
    res.check(rres, "add_rmsnorm_fwd_mxfp4 residual_out " + what)
    _inputs_unchanged([inp["x"], inp["r"], inp["w"]], [x, r, w], what)


# ---- backwards ----------------------------------------------------------------------------

BWD_SHAPES = [(1, 8), (37, 1000), (300, 1001), (1000, 4104), (129, 7168), (5, 16392)]


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("dtype,wdtype", DTYPES)
@pytest.mark.parametrize("M,N", BWD_SHAPES)
def test_rms_backwards(M, N, dtype, wdtype, misalign):
    inp = synth.rmsnorm_bwd_inputs(M, N, dtype, wdtype, seed=M + 7 * N)
    dres = synth.store(synth.normal(M, "dres", (M, N)), dtype)
    rstd = by_rows(oracle.rmsnorm_fwd, inp["x"], inp["w"], 1e-6)[1]
    dy, x, w, rs, dr = _dev_inputs(inp["dy"], inp["x"], inp["w"], rstd, dres)
    host = [inp["dy"], inp["x"], inp["w"], rstd, dres]
    o = _off(dtype, misalign)
    what = f"{M}x{N} {dtype} w {wdtype} offset {o}"
    s = M * 17 + N
    need = ar.rmsnorm_bwd_workspace_bytes(M, N)

    with _ref(misalign):
        rdx, rdw = ar.rmsnorm_bwd(dy, x, w, rs)
    dx, dw, ws = Guarded((M, N), dtype, s, o), Guarded((N,), torch.float32, s + 1), \
        Guarded((need,), torch.uint8, s + 2)
    ar.rmsnorm_bwd(dy, x, w, rs, dx=dx.t, dw=dw.t, workspace=ws.t)
    torch.cuda.synchronize()
    dx.check(rdx, "rmsnorm_bwd dx " + what)
    dw.check(rdw, "rmsnorm_bwd dw " + what)
    # the workspace's contents are the call's own; only its bands are checked
    ws.check(ws.full[ws.lo:ws.hi].clone(), "rmsnorm_bwd workspace " + what)

    # its dw partials may be fewer than rmsnorm_bwd's: compared with itself
    with _ref(misalign):
        ndx, ndw = ar.rmsnorm_bwd_noalloc(dy, x, w, rs)
    dx, dw = Guarded((M, N), dtype, s + 3, o), Guarded((N,), torch.float32, s + 4)
    ar.rmsnorm_bwd_noalloc(dy, x, w, rs, dx=dx.t, dw=dw.t)
    torch.cuda.synchronize()
    dx.check(ndx, "rmsnorm_bwd_noalloc dx " + what)
    dw.check(ndw, "rmsnorm_bwd_noalloc dw " + what)

    with _ref(misalign):
        rdh, rdw = ar.add_rmsnorm_bwd(dy, dr, x, w, rs)
    dh, dw, ws = Guarded((M, N), dtype, s + 5, o), Guarded((N,), torch.float32, s + 6), \
        Guarded((need,), torch.uint8, s + 7)
    ar.add_rmsnorm_bwd(dy, dr, x, w, rs, dh=dh.t, dw=dw.t, workspace=ws.t)
    torch.cuda.synchronize()
    dh.check(rdh, "add_rmsnorm_bwd dh " + what)
    dw.check(rdw, "add_rmsnorm_bwd dw " + what)
    ws.check(ws.full[ws.lo:ws.hi].clone(), "add_rmsnorm_bwd workspace " + what)
    _inputs_unchanged(host, [dy, x, w, rs, dr], what)


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("dtype,wdtype", DTYPES)
@pytest.mark.parametrize("M,N", BWD_SHAPES)
def test_layernorm_backwards(M, N, dtype, wdtype, misalign):
    inp = synth.rmsnorm_bwd_inputs(M, N, dtype, wdtype, seed=M + 9 * N)
    dres = synth.store(synth.normal(M, "dres", (M, N)), dtype)
    _, mean, rstd = by_rows(oracle.layernorm_fwd, inp["x"], inp["w"], None, 1e-5)
    dy, x, w, mu, rs, dr = _dev_inputs(inp["dy"], inp["x"], inp["w"], mean, rstd, dres)
    host = [inp["dy"], inp["x"], inp["w"], mean, rstd, dres]
    o = _off(dtype, misalign)
    what = f"{M}x{N} {dtype} w {wdtype} offset {o}"
    s = M * 19 + N
    need = ar.layernorm_bwd_workspace_bytes(M, N)

    with _ref(misalign):
        rdx, rdw, rdb = ar.layernorm_bwd(dy, x, w, mu, rs)
    dx, dw, db = Guarded((M, N), dtype, s, o), Guarded((N,), torch.float32, s + 1), \
        Guarded((N,), torch.float32, s + 2)
    ws = Guarded((need,), torch.uint8, s + 3)
    ar.layernorm_bwd(dy, x, w, mu, rs, dx=dx.t, dw=dw.t, db=db.t, workspace=ws.t)
    torch.cuda.synchronize()
    dx.check(rdx, "layernorm_bwd dx " + what)
    dw.check(rdw, "layernorm_bwd dw " + what)
    db.check(rdb, "layernorm_bwd db " + what)
    ws.check(ws.full[ws.lo:ws.hi].clone(), "layernorm_bwd workspace " + what)

    with _ref(misalign):
        rdh, rdw, rdb = ar.add_layernorm_bwd(dy, dr, x, w, mu, rs)
    dh, dw, db = Guarded((M, N), dtype, s + 4, o), Guarded((N,), torch.float32, s + 5), \
        Guarded((N,), torch.float32, s + 6)
    ws = Guarded((need,), torch.uint8, s + 7)
    ar.add_layernorm_bwd(dy, dr, x, w, mu, rs, dh=dh.t, dw=dw.t, db=db.t, workspace=ws.t)
    torch.cuda.synchronize()
    dh.check(rdh, "add_layernorm_bwd dh " + what)
    dw.check(rdw, "add_layernorm_bwd dw " + what)
    db.check(rdb, "add_layernorm_bwd db " + what)
    ws.check(ws.full[ws.lo:ws.hi].clone(), "add_layernorm_bwd workspace " + what)

    # without db (no db buffer), dx allocated by the call: aligned, so both
    # calls take the default path
    _, rdw2, none = ar.layernorm_bwd(dy, x, w, mu, rs, with_db=False)
    assert none is None
    dw = Guarded((N,), torch.float32, s + 8)
    ar.layernorm_bwd(dy, x, w, mu, rs, dw=dw.t, with_db=False)
    torch.cuda.synchronize()
    dw.check(rdw2, "layernorm_bwd dw without db " + what)
    _inputs_unchanged(host, [dy, x, w, mu, rs, dr], what)


# ---- RMSNorm + RoPE on a packed buffer ------------------------------------------------------

@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("T,Hq,Hk,D", [(1, 1, 1, 64), (37, 4, 2, 128), (130, 8, 1, 64),
                                       (9, 3, 0, 128), (65, 2, 2, 96)])
def test_rope_outputs_in_a_packed_buffer(T, Hq, Hk, D, interleaved):
    """q_out and k_out are views into a guarded packed [T, (Hq + 2 Hk) * D]
    buffer (the value heads between token rows are guard bytes too), written
    out of place from separate q, k inputs and in place."""
    dtype = torch.bfloat16
    inp = synth.rmsnorm_rope_inputs(T, Hq, Hk, D, dtype, seed=T + D, P=512)
    W = (Hq + 2 * Hk) * D
    qkv = inp["qkv"].to(DEV)
    q = qkv[:, :Hq * D].view(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D) if Hk else None
    wq, wk, cos, sin, pos = _dev_inputs(inp["wq"], inp["wk"], inp["cos"], inp["sin"], inp["pos"])
    wk = wk if Hk else None
    rq, rk = ar.rmsnorm_rope_qk(q, k, wq, wk, cos, sin, pos, 1e-6, interleaved=interleaved)
    what = f"T={T} Hq={Hq} Hk={Hk} D={D} il={interleaved}"
    def expected(g):
        e = g.pattern.clone()  # the value heads and the bands keep the pattern
        body = e[g.lo:g.hi].view(dtype).view(T, W)
        body[:, :Hq * D] = rq.reshape(T, Hq * D).cpu()
        if Hk:
            body[:, Hq * D:(Hq + Hk) * D] = rk.reshape(T, Hk * D).cpu()
        return e

    # out of place into the packed buffer
    g = Guarded((T, W), dtype, T * 23 + D)
    oq = g.t[:, :Hq * D].view(T, Hq, D)
    ok = g.t[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D) if Hk else None
    ar.rmsnorm_rope_qk(q, k, wq, wk, cos, sin, pos, 1e-6, interleaved=interleaved, q_out=oq,
                       k_out=ok)
    torch.cuda.synchronize()
    diff = (g.full.cpu() != expected(g)).nonzero()
    assert diff.numel() == 0, f"out of place {what}: {diff.numel()} bytes differ, first " \
                              f"{int(diff[0]) - g.lo} from the buffer's start"
    # in place: the packed buffer holds q and k, updated where they are
    g = Guarded((T, W), dtype, T * 23 + D)
    body = g.t
    body[:, :(Hq + Hk) * D] = qkv[:, :(Hq + Hk) * D]
    gq = body[:, :Hq * D].view(T, Hq, D)
    gk = body[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D) if Hk else None
    ar.rmsnorm_rope_qk(gq, gk, wq, wk, cos, sin, pos, 1e-6, interleaved=interleaved, q_out=gq,
                       k_out=gk)
    torch.cuda.synchronize()
    diff = (g.full.cpu() != expected(g)).nonzero()
    assert diff.numel() == 0, f"in place {what}: {diff.numel()} bytes differ, first " \
                              f"{int(diff[0]) - g.lo} from the buffer's start"
    assert torch.equal(qkv.cpu().view(torch.uint8), inp["qkv"].view(torch.uint8)), \
        f"{what}: input changed"
