"""The native binding of the two latency-bound forwards against the ctypes
binding (both through the C ABI): bit-identical outputs for every argument
form (outputs given or allocated, rstd requested, given or absent, in place,
batched leading dimensions), and the same exception type and message for
every bad argument."""
import sys

import pytest
import torch

import add_rmsnorm_amd as ar
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _same(a, b):
    a = a if isinstance(a, tuple) else (a,)
    b = b if isinstance(b, tuple) else (b,)
    assert len(a) == len(b)
    for u, v in zip(a, b):
        assert u.dtype == v.dtype and u.shape == v.shape and u.is_contiguous()
        assert torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8))


def test_native_binding_is_loaded():
    assert ar.native is not None
    assert ar.add_rmsnorm_fwd is ar.native.add_rmsnorm_fwd


@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.float16, torch.float16),
                                          (torch.float16, torch.float32),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32)])
def test_results_match_the_ctypes_binding(dtype, wdtype):
    inp = synth.add_rmsnorm_fwd_inputs(3 * 40, 1032, dtype, wdtype, seed=5)
    x = inp["x"].to(DEV).view(3, 40, 1032)
    r = inp["r"].to(DEV).view(3, 40, 1032)
    w = inp["w"].to(DEV)
    for kw in ({}, {"return_rstd": True}):
        _same(ar.add_rmsnorm_fwd(x, r, w, 1e-6, **kw), ar.add_rmsnorm_fwd_ctypes(x, r, w, 1e-6, **kw))
        _same(ar.rmsnorm_fwd(x, w, 1e-6, **kw), ar.rmsnorm_fwd_ctypes(x, w, 1e-6, **kw))
    # outputs and rstd given, y over x and residual_out over r
    outs = []
    for fn in (ar.add_rmsnorm_fwd, ar.add_rmsnorm_fwd_ctypes):
        xx, rr = x.clone(), r.clone()
        rs = torch.empty(3, 40, device=DEV)
        got = fn(xx, rr, w, 1e-6, y=xx, residual_out=rr, rstd=rs)
        assert got[0].data_ptr() == xx.data_ptr() and got[1].data_ptr() == rr.data_ptr()
        assert got[2].data_ptr() == rs.data_ptr()
        outs.append(got)
    _same(outs[0], outs[1])


def _error(fn, *a, **k):
    with pytest.raises(Exception) as e:
        fn(*a, **k)
    return type(e.value), str(e.value)


def test_errors_match_the_ctypes_binding():
    bf = torch.bfloat16
    x = torch.ones(4, 64, dtype=bf, device=DEV)
    w = torch.ones(64, dtype=bf, device=DEV)
    buf = torch.ones(5, 64, dtype=bf, device=DEV)
    strided = torch.empty(64, 4, dtype=bf, device=DEV).t()
    # (what, x, r, w, keywords); cases that name no r or residual_out run on
    # rmsnorm_fwd too, with (x, w)
    cases = [
        ("x on the CPU", x.cpu(), x, w, {}),
        ("x strided", strided, x, w, {}),
        ("x float64", x.double(), x.double(), w, {}),
        ("x empty rows", x[:, :0], x[:, :0], w[:0], {}),
        ("r dtype", x, x.float(), w, {}),
        ("r shape", x, x[:3], w, {}),
        ("r strided", x, strided, w, {}),
        ("w shape", x, x, w[:63], {}),
        ("w 2-d", x, x, w.view(1, 64), {}),
        ("w on the CPU", x, x, w.cpu(), {}),
        ("w float64", x, x, w.double(), {}),
        ("y shape", x, x, w, {"y": x[:2]}),
        ("y dtype", x, x, w, {"y": x.float()}),
        ("y strided", x, x, w, {"y": strided}),
        ("residual_out strided", x, x, w, {"residual_out": strided}),
        ("residual_out dtype", x, x, w, {"residual_out": x.float()}),
        ("rstd dtype", x, x, w, {"rstd": torch.empty(4, dtype=bf, device=DEV)}),
        ("rstd shape", x, x, w, {"rstd": torch.empty(5, device=DEV)}),
        ("rstd on the CPU", x, x, w, {"rstd": torch.empty(4)}),
        ("negative eps", x, x, w, {"eps": -1.0}),
        ("y overlapping x", buf[:4], x, w, {"y": buf[1:]}),
        ("residual_out over y", x, x, w, {"y": buf[:4], "residual_out": buf[:4]}),
    ]
    for what, xa, ra, wa, kw in cases:
        a = _error(ar.add_rmsnorm_fwd, xa, ra, wa, **kw)
        b = _error(ar.add_rmsnorm_fwd_ctypes, xa, ra, wa, **kw)
        assert a == b, (what, a, b)
        if what.startswith(("r ", "residual_out")) or "residual_out" in kw:
            continue
        a = _error(ar.rmsnorm_fwd, xa, wa, **kw)
        b = _error(ar.rmsnorm_fwd_ctypes, xa, wa, **kw)
        assert a == b, (what, a, b)
