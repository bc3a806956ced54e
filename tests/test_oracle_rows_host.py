"""The row-sliced oracle calls equal one call over all rows, bit for bit, for
every forward the GPU tests slice (float32, bfloat16 and float16 rows, ragged
slice sizes, binary64 outputs), and a function whose outputs do not have one
row per input row is refused."""
import pytest
import torch

import oracle
import synth
from oracle_rows import by_rows

DT = [torch.float32, torch.bfloat16, torch.float16]


def _bits(t):
    ints = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}
    return t.contiguous().view(ints[t.element_size()])


def _same(a, b):
    assert len(a) == len(b)
    for s, t in zip(a, b):
        assert s.shape == t.shape and s.dtype == t.dtype
        assert torch.equal(_bits(s), _bits(t))


def _sliced(fn, *args, **kw):
    return by_rows(fn, *args, threads=5, min_elems=0, **kw)


@pytest.mark.parametrize("dtype", DT)
def test_rms_forwards(dtype):
    inp = synth.add_rmsnorm_fwd_inputs(37, 96, dtype, seed=4, r_std=0.5)
    x, r, w = inp["x"], inp["r"], inp["w"]
    _same(_sliced(oracle.rmsnorm_fwd, x, w, 1e-6), oracle.rmsnorm_fwd(x, w, 1e-6))
    _same(_sliced(oracle.add_rmsnorm_fwd, x, r, w, 1e-6), oracle.add_rmsnorm_fwd(x, r, w, 1e-6))
    _same(_sliced(oracle.add_rmsnorm_fwd, x, r, w, 1e-6, y_dtype=torch.float64),
          oracle.add_rmsnorm_fwd(x, r, w, 1e-6, y_dtype=torch.float64))


@pytest.mark.parametrize("dtype", DT)
def test_layernorm_forwards(dtype):
    inp = synth.add_rmsnorm_fwd_inputs(29, 64, dtype, seed=5, r_std=0.5)
    x, r, w = inp["x"], inp["r"], inp["w"]
    b = synth.store(synth.normal(5, "b", (64,)), dtype)
    _same(_sliced(oracle.layernorm_fwd, x, w, b, 1e-5), oracle.layernorm_fwd(x, w, b, 1e-5))
    _same(_sliced(oracle.add_layernorm_fwd, x, r, w, None, 1e-5),
          oracle.add_layernorm_fwd(x, r, w, None, 1e-5))


@pytest.mark.parametrize("group", [0, 32])
def test_quantised_forwards(group):
    inp = synth.add_rmsnorm_fwd_inputs(23, 128, torch.bfloat16, seed=6, r_std=0.5)
    x, r, w = inp["x"], inp["r"], inp["w"]
    _same(_sliced(oracle.rmsnorm_fwd_fp8, x, w, 1e-6, group=group),
          oracle.rmsnorm_fwd_fp8(x, w, 1e-6, group=group))
    _same(_sliced(oracle.rmsnorm_fwd_fp8, x, w, 1e-6, residual=r, group=group),
          oracle.rmsnorm_fwd_fp8(x, w, 1e-6, residual=r, group=group))
    _same(_sliced(oracle.rmsnorm_fwd_mxfp4, x, w, 1e-6, residual=r),
          oracle.rmsnorm_fwd_mxfp4(x, w, 1e-6, residual=r))


def test_small_inputs_take_one_call():
    calls = []

    def fn(x):
        calls.append(x.shape[0])
        return (x,)

    by_rows(fn, torch.zeros(64, 8), threads=4)
    assert calls == [64]
    by_rows(fn, torch.zeros(64, 8), threads=4, min_elems=0)
    assert sorted(calls[1:]) == [16, 16, 16, 16]


def test_outputs_must_follow_the_rows():
    with pytest.raises(ValueError):
        by_rows(lambda x: (x.sum(0),), torch.ones(8, 3), threads=2, min_elems=0)
