"""The GPU parity tests' own checkers, on the CPU: the one-rounding check
(assert_correctly_rounded) accepts a float32 computation of y rounded once
to bf16 or float16 and rejects the same computation with an extra rounding
of h * rstd to that type; the dw check holds columns without cancellation to rtol 1e-3
alone."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_correctly_rounded, assert_dw_close


def _inputs(dtype=torch.bfloat16):
    inp = synth.add_rmsnorm_fwd_inputs(64, 4096, dtype, seed=3, r_std=0.5)
    y64 = oracle.rmsnorm_fwd(inp["x"], inp["w"], 1e-6, y_dtype=torch.float64)[0]
    return inp["x"], inp["w"], y64


def _float32_y(x, w, double_round: bool):
    """The forward as float32 arithmetic: rstd from a float32 sum of squares,
    then (h * rstd) * w, rounded to the storage type once, or with h * rstd
    rounded to it first."""
    h = x.float()
    rs = 1.0 / torch.sqrt((h * h).sum(dim=1, keepdim=True) / h.shape[1] + 1e-6)
    t = h * rs
    if double_round:
        t = t.to(x.dtype).float()
    return (t * w.float()).to(x.dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_single_rounding_passes(dtype):
    x, w, y64 = _inputs(dtype)
    assert_correctly_rounded(_float32_y(x, w, False), y64, None, "y")


@pytest.mark.parametrize("dtype,name", [(torch.bfloat16, "bf16"), (torch.float16, "float16")])
def test_double_rounding_fails(dtype, name):
    x, w, y64 = _inputs(dtype)
    with pytest.raises(AssertionError, match=f"half a {name} ulp"):
        assert_correctly_rounded(_float32_y(x, w, True), y64, None, "y")


def test_dw_check_rejects_rtol_violation_without_cancellation():
    ref = torch.tensor([1.0, 0.25, -3.0], dtype=torch.float32)
    mag = torch.tensor([50.0, 50.0, 3.5], dtype=torch.float64)
    assert_dw_close(ref.clone(), ref, mag)
    # 1.4e-3 on column 0: inside rtol 1e-3 + 1e-5 * mag (1.5e-3), but the
    # column has no cancellation (|dw| >= 1e-2 * mag), where rtol 1e-3 holds alone
    bad = ref.clone()
    bad[0] = 1.0014
    with pytest.raises(AssertionError, match="without cancellation"):
        assert_dw_close(bad, ref, mag)
    # the same error on column 1 (|dw| < 1e-2 * mag: cancellation) is accepted
    ok = ref.clone()
    ok[1] = 0.25 + 4e-4
    assert_dw_close(ok, ref, mag)
