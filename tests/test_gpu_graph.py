"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph).

Every entry point is captured once into one graph with static buffers:
- fused Add+RMSNorm forward and backward;
- the FP8 forward;
- fused Add+LayerNorm forward and backward.

The graph is then replayed on four sets of inputs, which are copied into the
captured buffers eagerly between replays. The outputs are poisoned before
each replay. Every replay must equal, bit for bit, the same calls made
eagerly on the same inputs (the kernels are deterministic). The first replay
is also checked against the oracle. The library records no memset, so no
replay depends on state left by an earlier one."""
import sys

import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
from oracle_rows import by_rows
import synth
from parity import assert_bits_equal, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 1e-6


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def _poison(t):
    if t.dtype in (torch.float32, torch.bfloat16):
        t.fill_(float("nan"))
    else:
        t.view(torch.uint8).fill_(0xAB)


@pytest.mark.parametrize("M,N", [(2048, 4096), (77, 7168)])
def test_graph_replays_match_eager(M, N):
    bf = torch.bfloat16
    e = lambda *s, dtype=bf: torch.empty(*s, dtype=dtype, device=DEV)
    x, r, dy, dres = e(M, N), e(M, N), e(M, N), e(M, N)
    w, b = e(N), e(N)
    y, res, rstd = e(M, N), e(M, N), e(M, dtype=torch.float32)
    dh, dw = e(M, N), e(N, dtype=torch.float32)
    ws = e(ar.rmsnorm_bwd_workspace_bytes(M, N), dtype=torch.uint8)
    q, qs, qres = e(M, N, dtype=torch.float8_e4m3fn), e(M, dtype=torch.float32), e(M, N)
    yl, resl, mean, rstdl = e(M, N), e(M, N), e(M, dtype=torch.float32), e(M, dtype=torch.float32)
    dhl, dwl, dbl = e(M, N), e(N, dtype=torch.float32), e(N, dtype=torch.float32)
    wsl = e(ar.layernorm_bwd_workspace_bytes(M, N), dtype=torch.uint8)
    outputs = {"y": y, "res": res, "rstd": rstd, "dh": dh, "dw": dw, "q": q, "qs": qs,
               "qres": qres, "yl": yl, "resl": resl, "mean": mean, "rstdl": rstdl, "dhl": dhl,
               "dwl": dwl, "dbl": dbl}

    def step():
        ar.add_rmsnorm_fwd(x, r, w, EPS, y=y, residual_out=res, rstd=rstd)
        ar.add_rmsnorm_bwd(dy, dres, res, w, rstd, dh=dh, dw=dw, workspace=ws)
        ar.add_rmsnorm_fwd_fp8(x, r, w, EPS, y_fp8=q, y_scale=qs, residual_out=qres)
        ar.add_layernorm_fwd(x, r, w, b, EPS, y=yl, residual_out=resl, mean=mean, rstd=rstdl)
        ar.add_layernorm_bwd(dy, dres, resl, w, mean, rstdl, dh=dhl, dw=dwl, db=dbl,
                             workspace=wsl)

    def load(seed):
        inp = synth.add_rmsnorm_fwd_inputs(M, N, bf, seed=seed, r_std=0.5)
        x.copy_(inp["x"].to(DEV))
        r.copy_(inp["r"].to(DEV))
        w.copy_(inp["w"].to(DEV))
        b.copy_(synth.store(synth.normal(seed, "b", (N,), std=0.1), bf).to(DEV))
        dy.copy_(synth.store(synth.normal(seed, "dy", (M, N)), bf).to(DEV))
        dres.copy_(synth.store(synth.normal(seed + 1, "dy", (M, N)), bf).to(DEV))
        torch.cuda.synchronize()
        return inp

    # warm up on a side stream (default priority), then capture
    load(100)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for k in range(4):
        inp = load(k)
        for t in outputs.values():
            _poison(t)
        g.replay()
        torch.cuda.synchronize()
        got = {n: t.clone() for n, t in outputs.items()}
        for t in outputs.values():
            _poison(t)
        step()
        torch.cuda.synchronize()
        for n, t in outputs.items():
            assert torch.equal(got[n].view(torch.uint8), t.view(torch.uint8)), \
                f"replay {k}: {n} differs from the eager call"
        if k == 0:
            ry, rres, rrstd = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], EPS)
            assert_bits_equal(got["res"].cpu(), rres, "residual_out (replay)")
            assert_close(got["y"].cpu(), ry, "y (replay)")
            assert_close(got["rstd"].cpu(), rrstd, "rstd (replay)", atol=0, rtol=1e-5)
            assert_bits_equal(got["qres"].cpu(), rres, "fp8 residual_out (replay)")
    del g


# torch warns when a leaf's gradient node, made under capture on the capture
# stream, later serves an eager backward on the default stream; here that is
# intended (the eager call is the reference)
@pytest.mark.filterwarnings("ignore:The AccumulateGrad node's stream:UserWarning")
def test_graph_capture_through_implicit_workspace():
    """Forward and backward of the autograd ops captured in one graph, the
    backward's workspace taken implicitly (no workspace argument).  Between
    replays, eager backwards at larger sizes grow and replace the binding's
    cached workspace; each replay must still equal the eager result bit for
    bit, so the graph does not write into a cached buffer that was freed."""
    from add_rmsnorm_amd import autograd as ag
    M, N = 512, 4096
    bf = torch.bfloat16
    x = torch.empty(M, N, dtype=bf, device=DEV, requires_grad=True)
    w = torch.empty(N, dtype=bf, device=DEV, requires_grad=True)
    dy = torch.empty(M, N, dtype=bf, device=DEV)

    def load(seed):
        inp = synth.rmsnorm_bwd_inputs(M, N, bf, seed=seed)
        with torch.no_grad():
            x.copy_(inp["x"].to(DEV))
            w.copy_(inp["w"].to(DEV))
            dy.copy_(inp["dy"].to(DEV))
        torch.cuda.synchronize()

    def step():
        y = ag.rms_norm(x, w, EPS)
        gx, gw = torch.autograd.grad(y, (x, w), grad_outputs=dy)
        return y, gx, gw

    load(200)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static = step()
    torch.cuda.synchronize()
    for k in range(4):
        load(k)
        # eager backwards that grow the cached workspace in between
        big = synth.rmsnorm_bwd_inputs(M * (k + 2), N, bf, seed=300 + k)
        bx, bw, bdy = (big[n].to(DEV) for n in ("x", "w", "dy"))
        _, brstd = ar.rmsnorm_fwd(bx, bw, EPS, return_rstd=True)
        ar.rmsnorm_bwd(bdy, bx, bw, brstd)
        g.replay()
        torch.cuda.synchronize()
        got = [t.detach().clone() for t in static]
        ref = [t.detach() for t in step()]
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "dx", "dw"), got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                f"replay {k}: {name} differs from the eager call"
    del g
