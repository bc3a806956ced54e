"""The library from plain C, with no PyTorch in the process: tests/c_client's
program allocates with hipMalloc, runs the fused forward and the backward on
a stream of its own, replays the forward from a captured HIP graph, and
checks two argument errors (see its header).  Its outputs are compared here
with the oracle: residual_out bit for bit, y and dx to the bf16 tolerance,
rstd to rtol 1e-5, dw to the dw tolerance, and the graph's y bit for bit
with the eager y.  The backward takes the oracle's residual_out and rstd as
its saved inputs, so every expected value comes from the oracle.

The client is built beside its source by add_rmsnorm_amd/build.py."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle_rows import by_rows
import synth
from parity import assert_bits_equal, assert_close, assert_dw_close

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "addrms_client")


def _bf16_bytes(t: torch.Tensor) -> bytes:
    return t.contiguous().view(torch.int16).numpy().tobytes()


@pytest.mark.parametrize("M,N", [(300, 4104), (1, 8192), (1027, 7168)])
def test_c_client(tmp_path, M, N):
    sys.__stderr__.write(f"[gpu case] c client {M}x{N}\n")
    sys.__stderr__.flush()
    assert os.path.exists(CLIENT), f"{CLIENT} is not built; run python add_rmsnorm_amd/build.py"
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=M + N, r_std=0.5)
    dy = synth.store(synth.normal(M + N, "dy", (M, N)), torch.bfloat16)
    ry, rres, rrstd = by_rows(oracle.add_rmsnorm_fwd, inp["x"], inp["r"], inp["w"], 1e-6)
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(np.array([M, N], dtype="<i8").tobytes())
        for t in (inp["x"], inp["r"], inp["w"], dy, rres):
            f.write(_bf16_bytes(t))
        f.write(rrstd.numpy().astype("<f4").tobytes())
    dst = tmp_path / "out.bin"
    run = subprocess.run([CLIENT, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr

    raw = dst.read_bytes()
    off = 0

    def take(n, dtype, shape):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=int(np.prod(shape)), offset=off).reshape(shape)
        off += a.nbytes
        return torch.from_numpy(a.copy())

    bf = lambda: take(M * N, "<i2", (M, N)).view(torch.bfloat16)
    y, res = bf(), bf()
    rstd = take(M, "<f4", (M,))
    dx = bf()
    dw = take(N, "<f4", (N,))
    y2 = bf()
    assert off == len(raw), f"output holds {len(raw)} bytes, expected {off}"

    assert_bits_equal(res, rres, "residual_out")
    assert_close(y, ry, "y")
    assert_close(rstd, rrstd, "rstd", atol=0, rtol=1e-5)
    assert_bits_equal(y2, y, "y from the graph replay")
    rdx, rdw, mag = oracle.rmsnorm_bwd(dy, rres, inp["w"], rrstd)
    assert_close(dx, rdx, "dx")
    assert_dw_close(dw, rdw, mag, "dw")
