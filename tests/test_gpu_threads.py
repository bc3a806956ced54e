"""Concurrent callers: four host threads, each on a stream of its own, run
the fused forward, the backward (with its own workspace), the LayerNorm
forward and the E4M3 forward over their own inputs, many times over,
while the GPU overlaps the streams.  The library keeps no per-call state
and calls are documented as thread-safe, so every thread's every result
must equal, bit for bit, the same call made alone on the default stream
(all these results are deterministic: dw too, whose summation order is
fixed).  The ctypes calls release the interpreter lock, so the threads
enter the library at the same time."""
import sys
import threading

import pytest
import torch

import add_rmsnorm_amd as ar
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
THREADS, ROUNDS = 4, 25


def _inputs(k):
    M, N = 1500 + 37 * k, 4096 + 8 * k
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=100 + k, r_std=0.5)
    dy = synth.store(synth.normal(200 + k, "dy", (M, N)), torch.bfloat16)
    b = synth.store(synth.normal(300 + k, "b", (N,), std=0.1), torch.bfloat16)
    return {n: t.to(DEV) for n, t in (("x", inp["x"]), ("r", inp["r"]), ("w", inp["w"]),
                                       ("dy", dy), ("b", b))}


def _work(t, ws=None):
    y, res, rstd = ar.add_rmsnorm_fwd_ctypes(t["x"], t["r"], t["w"], 1e-6, return_rstd=True)
    dx, dw = ar.rmsnorm_bwd(t["dy"], res, t["w"], rstd, workspace=ws)
    ly, _, mean, lrstd = ar.add_layernorm_fwd(t["x"], t["r"], t["w"], t["b"], 1e-5,
                                              return_stats=True)
    q, s, _ = ar.add_rmsnorm_fwd_fp8(t["x"], t["r"], t["w"], 1e-6, group=128)
    return [y, res, rstd, dx, dw, ly, mean, lrstd, q.view(torch.uint8), s]


def test_threads_on_their_own_streams():
    sys.__stderr__.write("[gpu case] threads on their own streams\n")
    sys.__stderr__.flush()
    data = [_inputs(k) for k in range(THREADS)]
    want = [[o.clone() for o in _work(d)] for d in data]
    torch.cuda.synchronize()
    errors = []
    barrier = threading.Barrier(THREADS)

    def run(k):
        try:
            s = torch.cuda.Stream()
            M, N = data[k]["x"].shape
            ws = torch.empty(ar.rmsnorm_bwd_workspace_bytes(M, N), dtype=torch.uint8, device=DEV)
            barrier.wait(timeout=60)
            with torch.cuda.stream(s):
                for i in range(ROUNDS):
                    got = _work(data[k], ws)
                    s.synchronize()
                    for j, (g, w_) in enumerate(zip(got, want[k])):
                        if not torch.equal(g.view(torch.uint8), w_.view(torch.uint8)):
                            errors.append(f"thread {k} round {i} output {j} differs")
                            return
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {k}: {type(e).__name__}: {e}")

    threads = [threading.Thread(target=run, args=(k,), daemon=True) for k in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=300)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors[:4]
