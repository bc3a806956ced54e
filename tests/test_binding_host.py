"""The native binding of the latency-bound forwards against the ctypes
binding, on the CPU: both are present, take the same parameters in the same
order with the same defaults and keyword-only split, and reject a tensor off
the GPU with the same exception and message before any GPU call.  Their
results and every other error are compared on the GPU
(tests/test_gpu_binding.py)."""
import inspect
import re

import pytest
import torch

import add_rmsnorm_amd as ar


def _native_params(fn):
    """(name, default or None, keyword-only) from pybind11's signature line."""
    line = fn.__doc__.splitlines()[0]
    body = line[line.index("(") + 1:line.rindex(")")]
    out, kw = [], False
    for part in (p.strip() for p in re.split(r",\s*(?![^\[]*\])", body)):
        if part == "*":
            kw = True
            continue
        name = part.split(":")[0].strip()
        default = part.split("=")[1].strip() if "=" in part else None
        out.append((name, default, kw))
    return out


def _python_params(fn):
    out = []
    for p in inspect.signature(fn).parameters.values():
        d = None if p.default is inspect.Parameter.empty else repr(p.default)
        out.append((p.name, d, p.kind == inspect.Parameter.KEYWORD_ONLY))
    return out


def test_native_binding_is_built_and_used():
    assert ar.native is not None, "add_rmsnorm_amd/_native*.so is not built"
    assert ar.add_rmsnorm_fwd is ar.native.add_rmsnorm_fwd
    assert ar.rmsnorm_fwd is ar.native.rmsnorm_fwd


@pytest.mark.parametrize("name", ["rmsnorm_fwd", "add_rmsnorm_fwd"])
def test_same_parameters(name):
    native = _native_params(getattr(ar.native, name))
    python = _python_params(getattr(ar, name + "_ctypes"))
    assert [(n, k) for n, _, k in native] == [(n, k) for n, _, k in python]
    for (n, dn, _), (_, dp, _) in zip(native, python):
        if dp is None:
            assert dn is None, n
        else:
            assert dn is not None and eval(dn) == eval(dp), (n, dn, dp)


def test_cpu_tensor_rejected_alike():
    x = torch.ones(2, 8, dtype=torch.bfloat16)
    w = torch.ones(8, dtype=torch.bfloat16)
    for a, b, args in ((ar.native.add_rmsnorm_fwd, ar.add_rmsnorm_fwd_ctypes, (x, x, w)),
                       (ar.native.rmsnorm_fwd, ar.rmsnorm_fwd_ctypes, (x, w))):
        with pytest.raises(ValueError) as ea:
            a(*args)
        with pytest.raises(ValueError) as eb:
            b(*args)
        assert str(ea.value) == str(eb.value) == "x must be a GPU tensor"
