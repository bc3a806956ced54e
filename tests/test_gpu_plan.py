"""The kernel each call launches (its template arguments, read from a
torch.profiler trace of the call) is the one addrms_plan names: waves per row,
vectors a lane and, for the backwards, the wide block and the prefetch."""
import re
import sys

import pytest
import torch
from torch.profiler import ProfilerActivity, profile

import add_rmsnorm_amd as ar

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF, F32 = torch.bfloat16, torch.float32


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _kernels(fn):
    fn()                         # warm: the first call's lazy set-up stays out of the trace
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    return [e.name for e in prof.events() if "vec_kernel<" in e.name]


def _targs(name):
    args = [a.strip() for a in re.search(r"<(.*)>", name).group(1).split(",")]
    return [{"true": 1, "false": 0}.get(a, a) for a in args]


FWD = [  # (M, N, dtype, w_dtype, norm, fused, qmode, group)
    (16384, 7168, BF, BF, "rms", True, None, 0),
    (4096, 4096, BF, BF, "rms", True, None, 0),
    (4096, 2560, BF, BF, "rms", True, None, 0),
    (256, 4096, F32, F32, "rms", False, None, 0),
    (1, 8192, BF, F32, "rms", True, None, 0),
    (128, 8192, BF, F32, "rms", True, None, 0),
    (16384, 7168, BF, BF, "layer", True, None, 0),
    (16384, 5120, BF, BF, "layer", False, None, 0),
    (2048, 5120, BF, BF, "rms", True, "fp8", 0),
    (2048, 6144, BF, BF, "rms", True, "fp8_group", 128),
    (4096, 7168, BF, BF, "rms", True, "mxfp4", 0),
]


@pytest.mark.parametrize("M,N,dt,wdt,norm,fused,qmode,group", FWD)
def test_forward_launch_is_the_plan(M, N, dt, wdt, norm, fused, qmode, group):
    x = torch.randn(M, N, device=DEV).to(dt)
    r = torch.randn(M, N, device=DEV).to(dt)
    w = torch.randn(N, device=DEV).to(wdt)
    b = torch.randn(N, device=DEV).to(wdt)
    if qmode == "fp8":
        fn = lambda: ar.add_rmsnorm_fwd_fp8(x, r, w, 1e-6)
    elif qmode == "fp8_group":
        fn = lambda: ar.add_rmsnorm_fwd_fp8(x, r, w, 1e-6, group=group)
    elif qmode == "mxfp4":
        fn = lambda: ar.add_rmsnorm_fwd_mxfp4(x, r, w, 1e-6)
    elif norm == "layer":
        fn = (lambda: ar.add_layernorm_fwd(x, r, w, b, 1e-5)) if fused else \
            (lambda: ar.layernorm_fwd(x, w, b, 1e-5))
    else:
        fn = (lambda: ar.add_rmsnorm_fwd(x, r, w, 1e-6)) if fused else \
            (lambda: ar.rmsnorm_fwd(x, w, 1e-6))
    names = _kernels(fn)
    assert len(names) == 1, names
    t = _targs(names[0])
    p = ar.plan("fwd", M, N, dt, wdt, norm=norm, fused=fused, qmode=qmode, group=group)
    assert (int(t[5]), int(t[6])) == (p["waves_per_row"], p["vectors_per_lane"]), names[0]


BWD = [  # (M, N, dtype, norm, fused)
    (32768, 4096, BF, "rms", False),
    (8191, 4096, BF, "rms", False),
    (2047, 4096, BF, "rms", False),
    (8192, 2560, BF, "rms", True),
    (16384, 7168, BF, "rms", True),
    (32768, 4096, BF, "layer", False),
    (8192, 3584, BF, "layer", True),
    (8192, 2048, F32, "rms", False),
    (8192, 1536, F32, "rms", False),
]


@pytest.mark.parametrize("M,N,dt,norm,fused", BWD)
def test_backward_launch_is_the_plan(M, N, dt, norm, fused):
    x = torch.randn(M, N, device=DEV).to(dt)
    dy = torch.randn(M, N, device=DEV).to(dt)
    dres = torch.randn(M, N, device=DEV).to(dt)
    w = torch.randn(N, device=DEV).to(dt)
    stat = torch.rand(M, device=DEV) + 0.5
    mean = torch.randn(M, device=DEV)
    if norm == "rms":
        fn = (lambda: ar.add_rmsnorm_bwd(dy, dres, x, w, stat)) if fused else \
            (lambda: ar.rmsnorm_bwd(dy, x, w, stat))
    else:
        fn = (lambda: ar.add_layernorm_bwd(dy, dres, x, w, mean, stat)) if fused else \
            (lambda: ar.layernorm_bwd(dy, x, w, mean, stat))
    names = [n for n in _kernels(fn) if "bwd_vec_kernel<" in n]
    assert len(names) == 1, names
    t = _targs(names[0])
    p = ar.plan("bwd", M, N, dt, norm=norm, fused=fused)
    assert (int(t[4]), int(t[5]), t[6], t[7]) == (
        p["waves_per_row"], p["vectors_per_lane"], p["wide"], p["prefetch"]), names[0]
