"""GPU parity of per-head RMSNorm + RoPE (rmsnorm_rope_qk through the C ABI)
against the CPU oracle on seeded inputs.

The outputs are checked to the bf16 / float32 tolerances. bf16 outputs must
also lie within one bf16 ulp (plus 1e-5 for float32 cancellation) of the
oracle's binary64 value. Coverage:
- the full prefill shape, in place on a packed query/key/value buffer, where
  the value heads must be left untouched;
- every lane-group width of the vector path, for both pair layouts and every
  dtype pair;
- the element-wise path: other head sizes, odd strides, and the forced
  switch;
- separate buffers with their own strides;
- key heads absent;
- positions outside the table, which give NaN heads."""
import sys

import numpy as np
import pytest
import torch

import add_rmsnorm_amd as ar
import oracle
import synth
from parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 1e-6


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def near_exact(gpu, y64, what):
    """bf16 output against the oracle's binary64 value: at most one bf16 ulp
    of it plus 1e-5.  The 1e-5 covers float32 error where a*c and b*s
    nearly cancel; it is |n| * 2^-22 at most, and |n| < 8 here."""
    g = gpu.detach().cpu().float().numpy().astype(np.float64)
    r = y64.detach().cpu().numpy()
    fin = np.isfinite(r)
    mag = np.maximum(np.abs(r[fin]), 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
    err = np.abs(g[fin] - r[fin])
    bad = err > ulp + 1e-5
    assert not bad.any(), (f"{what}: {int(bad.sum())} values more than one bf16 ulp away, "
                           f"worst excess {float((err - ulp).max())}")


def check(got, ref, what, y64=None):
    assert_close(got, ref, what)
    if ref.dtype == torch.bfloat16 and y64 is not None:
        near_exact(got, y64, what)


def references(v, w, inp, interleaved, dtype):
    args = (v, w, inp["cos"], inp["sin"], inp["pos"], EPS)
    ref = oracle.rmsnorm_rope(*args, interleaved=interleaved)
    y64 = oracle.rmsnorm_rope(*args, interleaved=interleaved, y_dtype=torch.float64) \
        if dtype == torch.bfloat16 else None
    return ref, y64


def run_packed(T, Hq, Hk, D, dtype, wdtype, interleaved, seed, P=4096, seq_len=None, pos=None):
    """In place on a packed [T, (Hq + 2Hk) * D] buffer; returns nothing, asserts."""
    inp = synth.rmsnorm_rope_inputs(T, Hq, Hk, D, dtype, wdtype, seed=seed, P=P, seq_len=seq_len)
    if pos is not None:
        inp["pos"] = pos
    qkv = inp["qkv"]
    q = qkv[:, :Hq * D].view(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D)
    rq, q64 = references(q, inp["wq"], inp, interleaved, dtype)
    rk, k64 = references(k, inp["wk"], inp, interleaved, dtype)
    g = qkv.to(DEV)
    gq = g[:, :Hq * D].view(T, Hq, D)
    gk = g[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D)
    oq, ok = ar.rmsnorm_rope_qk(gq, gk, inp["wq"].to(DEV), inp["wk"].to(DEV), inp["cos"].to(DEV),
                                inp["sin"].to(DEV), inp["pos"].to(DEV), EPS,
                                interleaved=interleaved, q_out=gq, k_out=gk)
    assert oq.data_ptr() == gq.data_ptr() and ok.data_ptr() == gk.data_ptr()
    torch.cuda.synchronize()
    out = g.cpu()
    what = f"T={T} Hq={Hq} Hk={Hk} D={D} {dtype} w {wdtype} il={interleaved}"
    check(out[:, :Hq * D].view(T, Hq, D), rq, "q " + what, q64)
    check(out[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D), rk, "k " + what, k64)
    v = slice((Hq + Hk) * D, None)
    assert torch.equal(out[:, v].view(torch.uint8), qkv[:, v].contiguous().view(torch.uint8)), \
        "value heads changed"


@pytest.mark.parametrize("interleaved", [False, True])
def test_full_prefill_shape_in_place(interleaved):
    c = synth.WORKLOADS["rmsnorm_rope_bf16_t16384_q32_k8_d128"]
    run_packed(c["T"], c["Hq"], c["Hk"], c["D"], c["dtype"], c["w_dtype"], interleaved, 0,
               P=c["P"], seq_len=c["seq_len"])


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("dtype,wdtype", [(torch.bfloat16, torch.bfloat16),
                                          (torch.bfloat16, torch.float32),
                                          (torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32, 64])
def test_every_lane_group_width(interleaved, dtype, wdtype, G):
    E = 8 if dtype == torch.bfloat16 else 4
    D = 2 * E * G
    T = max(3, 2048 // D)
    run_packed(T, 3, 2, D, dtype, wdtype, interleaved, seed=G)


@pytest.mark.parametrize("hpl", [1, 2, 4])
@pytest.mark.parametrize("D", [16, 128, 1024])
def test_heads_per_group_with_ragged_tails(knobs, hpl, D):
    # head counts that leave a partial final step: 37 tokens x (5 + 2) heads
    knobs.setenv("ADDRMS_ROPE_HPL", str(hpl))
    run_packed(37, 5, 2, D, torch.bfloat16, torch.bfloat16, hpl == 2, seed=hpl * D)


@pytest.mark.parametrize("D", [2, 6, 96, 130, 200])
@pytest.mark.parametrize("interleaved", [False, True])
def test_other_head_sizes_take_the_elementwise_path(D, interleaved):
    run_packed(37, 4, 1, D, torch.bfloat16, torch.bfloat16, interleaved, seed=D)


@pytest.mark.parametrize("interleaved", [False, True])
def test_forced_elementwise_and_odd_strides(knobs, interleaved):
    run_packed(65, 2, 2, 128, torch.float32, torch.float32, interleaved, seed=3)
    knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    run_packed(65, 5, 3, 128, torch.bfloat16, torch.bfloat16, interleaved, seed=4)


def test_odd_token_stride_is_elementwise():
    # a 3-element gap between tokens: strides are not multiples of 16 bytes
    T, H, D = 50, 4, 64
    base = synth.store(synth.normal(5, "x", (T, H * D + 3)), torch.bfloat16)
    q = base[:, :H * D].view(T, H, D)
    w = synth.weight(5, D, torch.bfloat16, "wq")
    cos, sin = synth.rope_table(256, D)
    pos = synth.positions(5, T, 256)
    ref = oracle.rmsnorm_rope(q, w, cos, sin, pos, EPS)
    g = base.to(DEV)
    gq = g[:, :H * D].view(T, H, D)
    out, none = ar.rmsnorm_rope_qk(gq, None, w.to(DEV), None, cos.to(DEV), sin.to(DEV),
                                   pos.to(DEV), EPS)
    torch.cuda.synchronize()
    assert none is None and out.is_contiguous()
    check(out.cpu(), ref, "odd stride")
    assert torch.equal(g.cpu().view(torch.int16), base.view(torch.int16)), "input changed"


def test_separate_buffers_with_their_own_strides():
    T, Hq, Hk, D = 300, 6, 2, 128
    q = synth.store(synth.normal(7, "x", (T, Hq, D)), torch.bfloat16)
    k = synth.store(synth.normal(7, "r", (T, Hk, D)), torch.bfloat16)
    wq = synth.weight(7, D, torch.bfloat16, "wq")
    wk = synth.weight(7, D, torch.bfloat16, "wk")
    cos, sin = synth.rope_table(1000, D)
    pos = synth.positions(7, T, 1000)
    rq = oracle.rmsnorm_rope(q, wq, cos, sin, pos, EPS)
    rk = oracle.rmsnorm_rope(k, wk, cos, sin, pos, EPS)
    # outputs are views into wider buffers (token strides 1024 and 512 elements)
    qo_buf = torch.full((T, 1024), 7.0, dtype=torch.bfloat16, device=DEV)
    ko_buf = torch.full((T, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    qo = qo_buf[:, 128:128 + Hq * D].view(T, Hq, D)
    ko = ko_buf[:, 256:256 + Hk * D].view(T, Hk, D)
    ar.rmsnorm_rope_qk(q.to(DEV), k.to(DEV), wq.to(DEV), wk.to(DEV), cos.to(DEV), sin.to(DEV),
                       pos.to(DEV), EPS, q_out=qo, k_out=ko)
    torch.cuda.synchronize()
    check(qo.cpu(), rq, "q")
    check(ko.cpu(), rk, "k")
    # nothing outside the output views was written
    qb = qo_buf.cpu().float()
    assert torch.all(qb[:, :128] == 7) and torch.all(qb[:, 128 + Hq * D:] == 7)
    kb = ko_buf.cpu().float()
    assert torch.all(kb[:, :256] == 7) and torch.all(kb[:, 256 + Hk * D:] == 7)


@pytest.mark.parametrize("vec", [True, False])
def test_positions_outside_the_table_give_nan_heads(knobs, vec):
    if not vec:
        knobs.setenv("ADDRMS_FORCE_ELEM", "1")
    T, P = 9, 64
    pos = synth.positions(9, T, P)
    pos[2], pos[5], pos[7] = -1, P, 1 << 40
    run_packed(T, 4, 2, 128, torch.bfloat16, torch.bfloat16, False, seed=9, P=P, pos=pos)


def test_empty_and_one_token():
    D = 128
    e = torch.empty(0, 4, D, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(D, dtype=torch.bfloat16, device=DEV)
    cos, sin = (t.to(DEV) for t in synth.rope_table(8, D))
    oq, ok = ar.rmsnorm_rope_qk(e, None, w, None, cos, sin,
                                torch.empty(0, dtype=torch.int64, device=DEV))
    assert oq.shape == (0, 4, D) and ok is None
    run_packed(1, 1, 1, D, torch.bfloat16, torch.bfloat16, True, seed=11)


def test_repeated_calls_are_bit_identical():
    T, Hq, Hk, D = 512, 8, 2, 128
    inp = synth.rmsnorm_rope_inputs(T, Hq, Hk, D, seed=13)
    qkv = inp["qkv"].to(DEV)
    q = qkv[:, :Hq * D].view(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D)
    args = [inp[n].to(DEV) for n in ("wq", "wk", "cos", "sin", "pos")]
    a = ar.rmsnorm_rope_qk(q, k, args[0], args[1], *args[2:])
    b = ar.rmsnorm_rope_qk(q, k, args[0], args[1], *args[2:])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_custom_ops_out_of_place_and_in_place():
    import add_rmsnorm_amd.autograd as ag
    T, Hq, Hk, D = 256, 8, 2, 128
    inp = synth.rmsnorm_rope_inputs(T, Hq, Hk, D, seed=17)
    args = [inp[n].to(DEV) for n in ("wq", "wk", "cos", "sin", "pos")]
    qkv = inp["qkv"].to(DEV)
    q = qkv[:, :Hq * D].view(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D)
    ref = ar.rmsnorm_rope_qk(q, k, *args, 1e-6, interleaved=True)
    out = ag.rms_norm_rope_qk(q, k, *args, 1e-6, interleaved=True)
    f = torch.compile(lambda q, k: ag.rms_norm_rope_qk(q, k, *args, 1e-6, True),
                      backend="aot_eager", fullgraph=True)
    comp = f(q, k)
    ag.rms_norm_rope_qk(q, k, *args, 1e-6, interleaved=True, inplace=True)
    torch.cuda.synchronize()
    for r_, o_, c_, i_ in zip(ref, out, comp, (q, k)):
        assert torch.equal(r_.view(torch.int16), o_.view(torch.int16))
        assert torch.equal(r_.view(torch.int16), c_.view(torch.int16))
        assert torch.equal(r_.view(torch.int16), i_.view(torch.int16))
