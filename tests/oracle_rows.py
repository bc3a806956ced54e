"""Row slices of the oracle's forwards, run in threads, for the full-size
parity tests.

Every forward the oracle offers (RMSNorm, LayerNorm, their residual forms,
the E4M3 and MXFP4 outputs) is row-wise: row i of each output depends only on
row i of x (and r) and on the shared weights.  So the oracle called on
disjoint row slices and concatenated returns the same tensors, bit for bit,
as one call over all rows (tests/test_oracle_rows_host.py checks this for
each function).  The oracle's C runs inside ctypes calls, which release the
GIL, so the slices run at once on the host's cores.  Nothing here touches
the oracle's arithmetic; inputs below MIN_ELEMS elements take one plain call.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import torch

MIN_ELEMS = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def by_rows(fn, *args, threads: int | None = None, min_elems: int = MIN_ELEMS, **kw):
    """fn(*args, **kw) for a row-wise oracle forward whose first argument is
    the 2-D row tensor x [M, N].  Every 2-D tensor argument with M rows (x,
    and r or residual) is cut into the same row slices; everything else (the
    weights, eps, options) is passed whole.  Each output must have one row per
    input row; the slices' outputs are concatenated in row order."""
    x = args[0]
    n = _threads() if threads is None else threads
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.numel() < min_elems or n <= 1 \
            or x.shape[0] < 2:
        return fn(*args, **kw)
    M = x.shape[0]
    k = min(n, M)
    bounds = [M * i // k for i in range(k + 1)]

    def part(i):
        lo, hi = bounds[i], bounds[i + 1]

        def cut(a):
            if isinstance(a, torch.Tensor) and a.dim() == 2 and a.shape[0] == M:
                return a[lo:hi]
            return a

        out = fn(*(cut(a) for a in args), **{name: cut(v) for name, v in kw.items()})
        for t in out:
            if not isinstance(t, torch.Tensor) or t.dim() < 1 or t.shape[0] != hi - lo:
                raise ValueError("oracle_rows: an output without one row per input row")
        return out

    with cf.ThreadPoolExecutor(k) as ex:
        parts = list(ex.map(part, range(k)))
    return tuple(torch.cat([p[j] for p in parts], 0) for j in range(len(parts[0])))
