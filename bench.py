"""Throughput of fused residual-Add + RMSNorm on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only-headline] [--no-cpu-baseline]

A step is one fused Add+RMSNorm forward over the whole batch: bf16 x, r
[16384, 7168], bf16 w, eps 1e-6, writing y and residual_out (bf16).  Inputs
are seeded synthetic data (the shared generator), resident in HBM before the
timed region; two input/output sets alternate so that no step reads data the
previous step left in the 256 MB last-level cache.

Prints ONE JSON line on stdout: achieved GB/s over the algorithmic bytes
(every tensor read or written once: 8*M*N + 2*N bytes), its fraction of the
8 TB/s HBM peak, rows/s, the copy-kernel ceiling measured in the same run, the
roofline of the dominant kernel, the CPU oracle's throughput on a bounded
sample, and secondary figures (backward, decode latency) unless
--only-headline.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "achieved HBM GB/s (% of peak) + rows/s, bf16 fused Add+RMSNorm M=16384 N=7168"
WORKLOAD = "add_rmsnorm_fwd_bf16_16384x7168"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_vec_kernel_add_rmsnorm_bf16_16384x7168.md")
HEADLINE_KERNEL = "fwd_vec_kernel<addrms::bf16_t, addrms::bf16_t, 0, true, 0, 16, 1>"
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_vec_kernel_rmsnorm_bf16_32768x4096.md")
BWD_KERNEL = "bwd_vec_kernel<addrms::bf16_t, addrms::bf16_t, 0, false, 8, 1, false, false>"
COLREDUCE_KERNEL = "dw_colreduce_vec_kernel"
KERNEL_SOURCES = ["add_rmsnorm_amd/csrc/kernels.hpp", "add_rmsnorm_amd/csrc/device.hpp",
                  "add_rmsnorm_amd/csrc/tables.hip", "add_rmsnorm_amd/csrc/internal.hpp",
                  "add_rmsnorm_amd/csrc/api.hip"]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def timed(fn, steps: int, warmup: int):
    """Run fn() warmup times, then time `steps` calls bracketed by device
    synchronisation.  Returns (wall seconds, event seconds) for the K calls;
    the events are recorded on the current stream, where fn launches."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / 1e3


def graph_time(call, per_graph: int = 50, replays: int = 10) -> float:
    """Device seconds per call: `per_graph` calls captured in one graph,
    replayed; launch gaps between kernels in a graph are those of the device,
    not of the Python host loop."""
    import torch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            call()
    best = None
    for _ in range(3):
        _, ev = timed(g.replay, replays, 2)
        best = ev if best is None else min(best, ev)
    return best / (replays * per_graph)


def copy_ceiling(nbytes: int, steps: int = 20):
    """GB/s of torch's device copy moving nbytes/2 read + nbytes/2 written."""
    import torch
    n = nbytes // 2
    a = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(2)]
    b = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for t in a:
        t.fill_(1)
    i = [0]

    def step():
        k = i[0] & 1
        b[k].copy_(a[k])
        i[0] += 1

    _, ev = timed(step, steps, 3)
    return 2 * n * steps / ev / 1e9


def per_call(fn, calls: int, warmup: int = 5) -> dict:
    """Device time of each of `calls` calls of fn(), from a pair of HIP events
    recorded around each call on the current stream (where fn launches):
    median, 10th and 90th percentile and mean, in microseconds."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for a, b in ev:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)

    def pct(q):
        return us[min(len(us) - 1, int(round(q * (len(us) - 1))))]

    return {"median_us": round(pct(0.5), 3), "p10_us": round(pct(0.1), 3),
            "p90_us": round(pct(0.9), 3), "mean_us": round(sum(us) / len(us), 3), "calls": calls}


def figure(fn, nb: int, calls: int, **extra) -> dict:
    """One secondary figure: per-call event pairs around `calls` calls of fn
    (after 5 warm-up calls); GB/s over the algorithmic bytes nb at the median
    call, and the median, 10th and 90th percentile call times.  Then the same
    number of calls back to back between one pair of events: for short
    kernels an event pair per call also times the launch, which back-to-back
    calls overlap with the previous kernel."""
    t = per_call(fn, calls, 5)
    _, ev = timed(fn, calls, 0)
    gbps = nb / t["median_us"] / 1e3
    d = {"GBps": round(gbps, 1), "pct_of_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
         "us_per_call": t["median_us"], "median_us": t["median_us"], "p10_us": t["p10_us"],
         "p90_us": t["p90_us"], "mean_us": t["mean_us"], "calls": calls,
         "us_per_call_back_to_back": round(ev / calls * 1e6, 3),
         "GBps_back_to_back": round(nb * calls / ev / 1e9, 1), "bytes": nb}
    d.update(extra)
    return d


ROW_SWEEP_N = (4096, 7168)
ROW_SWEEP_M = (512, 1024, 2048, 4096, 8192, 16384)
ROW_SWEEP_CALLS = 100
ROW_SWEEP_WARMUP = 5
ROW_SWEEP_PROBE = "r2w2_b1024_u1"       # the 2R2W probe timed beside each shape
ROW_SWEEP_PROBE_KERNEL = "mix_kernel<2, 2, 1024, 1,"


def row_sweep(calls: int = ROW_SWEEP_CALLS) -> dict:
    """The fused bf16 forward at fixed widths over a range of row counts, in
    the order ROW_SWEEP_N x ROW_SWEEP_M, ROW_SWEEP_WARMUP + `calls` calls
    each; enough rotating input/output sets that the calls of one shape
    stream at least 1 GB (never from the 256 MB last-level cache).  Per-call
    event pairs per shape, and the least-squares line t = t0 + bytes / B over
    the medians: B is the marginal stream rate, t0 the fixed cost of a launch
    (the ramp to a full device and the tail of the last blocks).  After each
    shape, the 2-read/2-write stream probe ROW_SWEEP_PROBE over the same
    buffers, the same number of calls, and its own line: the launch cost of
    streaming alone."""
    import numpy as np
    import torch
    import add_rmsnorm_amd as ar
    import synth
    import ctypes
    lib = _probe_lib()
    pid = None
    if lib is not None:
        names = [lib.addrms_probe_name(k).decode() for k in range(lib.addrms_probe_count())]
        pid = names.index(ROW_SWEEP_PROBE)
    out = {}
    for N in ROW_SWEEP_N:
        pts, ppts = [], []
        for M in ROW_SWEEP_M:
            inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.bfloat16, seed=1, r_std=0.5)
            w = inp["w"].cuda()
            x0, r0 = inp["x"].cuda(), inp["r"].cuda()
            nb = 8 * M * N + 2 * N
            nsets = max(2, min(64, -(-(1 << 30) // nb)))
            sets = [(x0.clone(), r0.clone(), torch.empty_like(x0), torch.empty_like(x0))
                    for _ in range(nsets)]
            i = [0]

            def step():
                x, r, y, ro = sets[i[0] % nsets]
                ar.add_rmsnorm_fwd(x, r, w, 1e-6, y=y, residual_out=ro)
                i[0] += 1

            t = per_call(step, calls, ROW_SWEEP_WARMUP)
            out[f"{M}x{N}"] = dict(t, bytes=nb, GBps=round(nb / t["median_us"] / 1e3, 1),
                                   sets=nsets)
            pts.append((nb, t["median_us"]))
            log(f"row sweep {M}x{N}: median {t['median_us']} us")
            # the 2-read/2-write stream probe over the same buffers: the
            # launch cost of pure streaming at this size
            if lib is not None:
                vp = ctypes.c_void_p
                pargs = [((vp * 3)(x.data_ptr(), r.data_ptr(), None),
                          (vp * 2)(y.data_ptr(), ro.data_ptr())) for x, r, y, ro in sets]
                j = [0]

                def pstep():
                    a_in, a_out = pargs[j[0] % nsets]
                    rc = lib.addrms_probe_run(pid, a_in, a_out, 2 * M * N, None,
                                              torch.cuda.current_stream().cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"probe {ROW_SWEEP_PROBE} failed: hipError {rc}")
                    j[0] += 1

                tp = per_call(pstep, calls, ROW_SWEEP_WARMUP)
                out[f"{M}x{N}"]["probe_median_us"] = tp["median_us"]
                ppts.append((8 * M * N, tp["median_us"]))
            del sets, x0, r0
            torch.cuda.empty_cache()
        b, a = np.polyfit([p[0] for p in pts], [p[1] for p in pts], 1)
        out[f"fit_N{N}"] = {"t0_us": round(float(a), 3), "marginal_GBps": round(1e-3 / float(b), 1)}
        if ppts:
            b, a = np.polyfit([p[0] for p in ppts], [p[1] for p in ppts], 1)
            out[f"probe_fit_N{N}"] = {"t0_us": round(float(a), 3),
                                      "marginal_GBps": round(1e-3 / float(b), 1)}
    return out


def summarize_row_sweep(trace_dir: str, out_path: str, commands: dict):
    """Profile summary of a traced --row-sweep run: the fused forward's and
    the stream probe's traced durations grouped by shape (dispatches in the
    sweep's order, one group per shape, the warm-up calls dropped), the
    median per shape, and per width the least-squares line t = t0 + bytes / B
    over those medians for each."""
    import numpy as np
    all_rows, _ = _csv_rows(trace_dir, "kernel_trace.csv")
    all_rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    fwd = [r for r in all_rows if "fwd_vec_kernel" in r["Kernel_Name"]]
    probe = [r for r in all_rows if ROW_SWEEP_PROBE_KERNEL in r["Kernel_Name"]]
    per = ROW_SWEEP_WARMUP + ROW_SWEEP_CALLS
    shapes = [(M, N) for N in ROW_SWEEP_N for M in ROW_SWEEP_M]
    if len(fwd) != per * len(shapes):
        raise SystemExit(f"expected {per * len(shapes)} forward dispatches, found {len(fwd)}")
    if probe and len(probe) != per * len(shapes):
        raise SystemExit(f"expected {per * len(shapes)} probe dispatches, found {len(probe)}")

    def stats(rows, k):
        grp = rows[k * per + ROW_SWEEP_WARMUP:(k + 1) * per]
        d = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp)
        return grp[0], d[len(d) // 2], d[int(0.1 * (len(d) - 1))], d[int(0.9 * (len(d) - 1))]

    lines = ["# Fused Add+RMSNorm forward, bf16: launch time against rows",
             "",
             "Traced kernel durations of the fused forward over a range of row counts at",
             "two widths, and per width the least-squares line t = t0 + bytes / B over",
             "the medians: B is the marginal stream rate of one more row, t0 the fixed",
             "cost of a launch (the ramp to a full device plus the tail of the last",
             "blocks).  Bytes are the algorithmic 8 M N + 2 N.  Beside each shape, the",
             f"2-read/2-write stream probe ({ROW_SWEEP_PROBE}: pure streaming, no reduction)",
             "over the same buffers (8 M N bytes), with its own line.",
             "",
             "Commands:", ""]
    for k, v in commands.items():
        lines.append(f"- {k}: `{v}`")
    lines += [""]
    for N in ROW_SWEEP_N:
        lines += [f"## N = {N}", "",
                  "| M | kernel | blocks x threads | median us | p10 us | p90 us | GB/s | fit us |"
                  + (" probe median us | probe GB/s |" if probe else ""),
                  "|---|---|---|---|---|---|---|---|" + ("---|---|" if probe else "")]
        pts, ppts, info = [], [], []
        for k, (M, NN) in enumerate(shapes):
            if NN != N:
                continue
            first, med, p10, p90 = stats(fwd, k)
            wg = int(first["Workgroup_Size_X"])
            blocks = int(first["Grid_Size_X"]) // wg
            name = first["Kernel_Name"]
            targs = name[name.find("<") + 1:name.rfind(">")].split(",")
            nb = 8 * M * N + 2 * N
            pts.append((nb, med))
            pmed = None
            if probe:
                pmed = stats(probe, k)[1]
                ppts.append((8 * M * N, pmed))
            info.append((M, f"WPR {targs[-2].strip()}, VPL {targs[-1].strip()}", blocks, wg,
                         med, p10, p90, nb, pmed))
        b, a = np.polyfit([p[0] for p in pts], [p[1] for p in pts], 1)
        for M, kern, blocks, wg, med, p10, p90, nb, pmed in info:
            row = (f"| {M} | {kern} | {blocks} x {wg} | {med:.2f} | {p10:.2f} | {p90:.2f} | "
                   f"{nb / med / 1e3:.0f} | {a + b * nb:.2f} |")
            if pmed is not None:
                row += f" {pmed:.2f} | {8 * M * N / pmed / 1e3:.0f} |"
            lines.append(row)
        lines += ["", f"Fit: t0 = {a:.2f} us, B = {1e-3 / b:.0f} GB/s "
                      f"({100e-3 / b / HBM_PEAK_GBPS:.1f} % of 8 TB/s)."]
        if ppts:
            pb, pa = np.polyfit([p[0] for p in ppts], [p[1] for p in ppts], 1)
            lines += ["", f"Probe fit: t0 = {pa:.2f} us, B = {1e-3 / pb:.0f} GB/s "
                          f"({100e-3 / pb / HBM_PEAK_GBPS:.1f} % of 8 TB/s)."]
        lines += [""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out_path}")


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "add_rmsnorm_amd", "libaddrms_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.addrms_probe_count.restype = ctypes.c_int
    lib.addrms_probe_name.restype = ctypes.c_char_p
    lib.addrms_probe_name.argtypes = [ctypes.c_int]
    lib.addrms_probe_streams.restype = ctypes.c_int
    lib.addrms_probe_streams.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int)] * 3
    lib.addrms_probe_run.restype = ctypes.c_int
    lib.addrms_probe_run.argtypes = [ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                     ctypes.c_size_t, vp, vp]
    lib.addrms_probe_floor.restype = ctypes.c_int
    lib.addrms_probe_floor.argtypes = [ctypes.c_int, vp, vp, vp]
    return lib


def launch_floor() -> dict:
    """Device time per call, replaying a captured graph of 50 calls, of an
    empty one-block kernel and of one 1024-thread block copying 16 KiB: the
    floor under a one-row call."""
    import torch
    lib = _probe_lib()
    if lib is None:
        return {}
    a = torch.zeros(16384, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    out = {}
    for kind, name in ((0, "empty_kernel_us"), (1, "row_copy_16KiB_us")):
        def call(kind=kind):
            rc = lib.addrms_probe_floor(kind, a.data_ptr(), b.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"addrms_probe_floor({kind}) failed: hipError {rc}")
        out[name] = round(graph_time(call) * 1e6, 3)
    return out


# 2R2W probes that also run in place (outputs = inputs)
INPLACE_PROBES = {"r2w2_b256_u4", "r2w2_b512_u2", "r2w2_lds_b256_u4"}


def probe_matrix(each_bytes: int, calls: int = 30, only=None, inplace: bool = True) -> dict:
    """The stream probes of libaddrms_probe.so (pure streaming kernels; see
    add_rmsnorm_amd/csrc/stream_probe.hip), each stream `each_bytes` long,
    two buffer sets alternating so that no call reads what the previous one
    left in the 256 MB last-level cache.  Per probe: GB/s over the bytes it
    moves at the median, 10th and 90th percentile call time.  With `inplace`
    the 2R2W probes also run with the inputs passed as the outputs.  `only`:
    names to run (None: all)."""
    import ctypes
    import torch
    lib = _probe_lib()
    if lib is None:
        return {}
    vp = ctypes.c_void_p
    each = each_bytes // 16 * 16
    pool = [[torch.empty(each, dtype=torch.uint8, device="cuda") for _ in range(4)]
            for _ in range(2)]
    for st in pool:
        for k, t in enumerate(st):
            t.fill_(k + 1)
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = {}
    for pid in range(lib.addrms_probe_count()):
        name = lib.addrms_probe_name(pid).decode()
        if only is not None and name not in only:
            continue
        nin, nout, needs_ctr = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        lib.addrms_probe_streams(pid, ctypes.byref(nin), ctypes.byref(nout), ctypes.byref(needs_ctr))
        # work-counter probes: a fresh zeroed word for every call
        ctrs = (torch.zeros(2 * (calls + 8), dtype=torch.int32, device="cuda")
                if needs_ctr.value else None)
        modes = [False] + ([True] if inplace and name in INPLACE_PROBES else [])
        for ip in modes:
            args = []
            for st in pool:
                ins = [st[k].data_ptr() for k in range(nin.value)]
                if ip:
                    outs = ins[:]
                elif nout.value:
                    outs = [st[nin.value + k].data_ptr() for k in range(nout.value)]
                else:
                    outs = [sink.data_ptr()]
                args.append(((vp * 3)(*ins, *([None] * (3 - len(ins)))),
                             (vp * 2)(*outs, *([None] * (2 - len(outs))))))
            i = [0]
            if ctrs is not None:
                ctrs.zero_()

            def step():
                a_in, a_out = args[i[0] & 1]
                ctr = ctrs[i[0]].data_ptr() if ctrs is not None else None
                rc = lib.addrms_probe_run(pid, a_in, a_out, each, ctr,
                                          torch.cuda.current_stream().cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"probe {name} failed: hipError {rc}")
                i[0] += 1

            t = per_call(step, calls, 3)
            nb = (nin.value + nout.value) * each
            key = name + ("_inplace" if ip else "")
            out[key] = {"GBps": round(nb / t["median_us"] / 1e3, 1),
                        "GBps_p10_call": round(nb / t["p90_us"] / 1e3, 1),
                        "GBps_p90_call": round(nb / t["p10_us"] / 1e3, 1),
                        "median_us": t["median_us"], "bytes": nb, "calls": calls}
            log(f"probe {key}: {out[key]['GBps']} GB/s")
    del pool
    return out


def fused_fwd_inplace_compare(calls: int) -> dict:
    """The headline fused forward beside the probes: out of place (the
    workload) and in place (y written over x, residual_out over r, the form
    an inference engine's residual stream uses), same bytes and protocol."""
    import torch
    import add_rmsnorm_amd as ar
    import synth
    inp = synth.workload_inputs(WORKLOAD)
    cfg = synth.WORKLOADS[WORKLOAD]
    M, N, eps = cfg["M"], cfg["N"], cfg["eps"]
    w = inp["w"].cuda()
    sets = [(inp["x"].cuda(), inp["r"].cuda()) for _ in range(2)]
    outs = [(torch.empty_like(x), torch.empty_like(x)) for x, _ in sets]
    nb = 8 * M * N + 2 * N
    res = {}
    i = [0]

    def oop():
        (x, r), (y, ro) = sets[i[0] & 1], outs[i[0] & 1]
        ar.add_rmsnorm_fwd(x, r, w, eps, y=y, residual_out=ro)
        i[0] += 1

    def inp_():
        x, r = sets[i[0] & 1]
        ar.add_rmsnorm_fwd(x, r, w, eps, y=x, residual_out=r)
        i[0] += 1

    for name, fn in (("kernel_fused_fwd", oop), ("kernel_fused_fwd_inplace", inp_)):
        t = per_call(fn, calls, 3)
        res[name] = {"GBps": round(nb / t["median_us"] / 1e3, 1),
                     "GBps_p10_call": round(nb / t["p90_us"] / 1e3, 1),
                     "GBps_p90_call": round(nb / t["p10_us"] / 1e3, 1),
                     "median_us": t["median_us"], "bytes": nb, "calls": calls}
        log(f"{name}: {res[name]['GBps']} GB/s")
    return res


def stream_ceiling(nbytes: int, calls: int = 30):
    """GB/s of the probe kernels that only stream two reads and two writes of
    nbytes/4 each (libaddrms_probe.so), in the two launch shapes the row
    kernels use and 1024 x 1 (the fastest shapes of the probe matrix): the
    practical ceiling of the fused forward's access mix, measured in the same
    run.  The best median is reported."""
    res = probe_matrix(nbytes // 4, calls, only={"r2w2_b256_u4", "r2w2_b512_u2", "r2w2_b1024_u1"},
                       inplace=False)
    return max((v["GBps"] for v in res.values()), default=None)


def headline(steps: int, warmup: int):
    import torch
    import add_rmsnorm_amd as ar
    import synth

    cfg = synth.WORKLOADS[WORKLOAD]
    M, N, eps = cfg["M"], cfg["N"], cfg["eps"]
    log(f"generating {WORKLOAD} inputs")
    inp = synth.workload_inputs(WORKLOAD)
    sets = []
    for k in range(2):
        x = inp["x"].to("cuda")
        r = inp["r"].to("cuda")
        sets.append((x, r, torch.empty_like(x), torch.empty_like(x)))
    w = inp["w"].to("cuda")
    nbytes = 8 * M * N + 2 * N
    i = [0]

    def step():
        x, r, y, res = sets[i[0] & 1]
        ar.add_rmsnorm_fwd(x, r, w, eps, y=y, residual_out=res)
        i[0] += 1

    log(f"timing {steps} steps after {warmup} warmup")
    wall, ev = timed(step, steps, warmup)
    return dict(M=M, N=N, eps=eps, nbytes=nbytes, wall=wall, ev=ev, inputs=inp, step=step)


def traffic_from_profile(nbytes_alg: int):
    """HBM bytes per launch from the committed counter summary, or None when
    absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        if ln.startswith("- ") and ": " in ln:
            k, v = ln[2:].split(": ", 1)
            kv[k.strip("`")] = v.strip("`")
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    newest = max(files, key=os.path.getmtime)
    with open(newest) as f:
        return list(csv.DictReader(f)), newest


def summarize_profiles(trace_dir: str, fetch_dir: str, write_dir: str, commands: dict):
    """Write the committed profile summaries from rocprofv3 CSV output:
    kernel-trace statistics of the bench command, and the headline kernel's
    FETCH_SIZE / WRITE_SIZE scaled by the same counters of a device copy of
    known size."""
    stats, _ = _csv_rows(trace_dir, "kernel_stats.csv")
    fetch, _ = _csv_rows(fetch_dir, "counter_collection.csv")
    write, _ = _csv_rows(write_dir, "counter_collection.csv")

    def counter(rows, name_part, min_kib=0.0):
        return [float(r["Counter_Value"]) for r in rows
                if name_part in r["Kernel_Name"] and float(r["Counter_Value"]) > min_kib]

    # calibration: the device copies of nb/2 bytes that copy_ceiling() runs
    nb = 8 * 16384 * 7168 + 2 * 7168
    copy_kib = (nb // 2) / 1024.0
    cf = counter(fetch, "copyBuffer", copy_kib / 4)
    cw = counter(write, "copyBuffer", copy_kib / 4)
    f_scale = copy_kib / (sum(cf) / len(cf))
    w_scale = copy_kib / (sum(cw) / len(cw))
    kf = counter(fetch, HEADLINE_KERNEL)
    kw = counter(write, HEADLINE_KERNEL)
    fetch_b = sum(kf) / len(kf) * f_scale * 1024
    write_b = sum(kw) / len(kw) * w_scale * 1024
    alg_read, alg_write = 4 * 16384 * 7168 + 2 * 7168, 4 * 16384 * 7168
    # the headline's own dispatches (warm-up and timed steps) come first; the
    # same kernel also serves the per-call and in-place figures later
    first = _trace_durations(trace_dir, HEADLINE_KERNEL)[:commands.get("headline_dispatches", 10 ** 9)]
    avg_us = sum(first) / len(first)

    out = [f"# {HEADLINE_KERNEL}: fused Add+RMSNorm, bf16, M=16384 N=7168", "",
           "Kernel trace (rocprofv3 --kernel-trace --stats) of the default bench command:", "",
           f"    {commands['trace']}", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:24]:
        out.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f} |")
    out += ["", "HBM traffic of the headline kernel (two counter runs, one counter each):", "",
            f"    {commands['fetch']}", f"    {commands['write']}", "",
            f"Calibration: a device copy of {nb // 2} bytes reads FETCH_SIZE "
            f"{sum(cf) / len(cf):.1f} KiB and WRITE_SIZE {sum(cw) / len(cw):.1f} KiB per "
            f"dispatch, so FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by "
            f"{w_scale:.4f} to bytes moved.", "",
            f"| | counter KiB/dispatch | scaled bytes | algorithmic bytes | ratio |",
            f"|---|---|---|---|---|",
            f"| read | {sum(kf) / len(kf):.1f} | {fetch_b:.0f} | {alg_read} | {fetch_b / alg_read:.4f} |",
            f"| write | {sum(kw) / len(kw):.1f} | {write_b:.0f} | {alg_write} | {write_b / alg_write:.4f} |",
            "", f"Kernel average over the headline's {len(first)} dispatches (warm-up and timed "
                f"steps) in the trace: {avg_us:.2f} us.",
            "", "Values read by bench.py:", "",
            f"- kernel_source_digest: {kernel_source_digest()}",
            f"- traffic_bytes_per_launch: {int(round(fetch_b + write_b))}",
            f"- kernel_avg_us_rocprof: {avg_us:.3f}",
            f"- achieved_GBps_rocprof: {nb / avg_us / 1e3:.1f}", ""]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out))
    log(f"wrote {TRAFFIC_FILE}")
    if counter(fetch, BWD_KERNEL):
        summarize_bwd(stats, fetch, write, f_scale, w_scale, commands)
    summarize_secondary(trace_dir, fetch, write, f_scale, w_scale, commands)
    summarize_decode(trace_dir, commands)


def _following_durations(trace_dir: str, name_part: str, follow: str):
    """Durations (us) of the first `follow` kernel dispatched after each
    dispatch of `name_part` (the column reduce that completes a backward)."""
    rows, _ = _csv_rows(trace_dir, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    out = []
    for k, r in enumerate(rows):
        if name_part in r["Kernel_Name"]:
            nxt = next((q for q in rows[k + 1:] if follow in q["Kernel_Name"]), None)
            if nxt is not None:
                out.append((int(nxt["End_Timestamp"]) - int(nxt["Start_Timestamp"])) / 1e3)
    return out


def _trace_durations(trace_dir: str, name_part: str):
    """Durations (us) of a kernel's dispatches in dispatch order, from a
    rocprofv3 kernel trace."""
    rows, _ = _csv_rows(trace_dir, "kernel_trace.csv")
    rows = [r for r in rows if name_part in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]


# Secondary workloads whose kernels each serve one figure of the bench line:
# (profile file stem, title, kernel name, follow-up kernel or None,
#  algorithmic read bytes, algorithmic write bytes)
def _secondary_specs():
    B = "addrms::bf16_t"
    M, N = 16384, 7168
    m2, n2 = 4096, 4096
    mb, nbk = 32768, 4096
    return [
        ("fwd_vec_kernel_add_rmsnorm_bf16_4096x4096", "fused Add+RMSNorm, bf16, M=4096 N=4096",
         f"fwd_vec_kernel<{B}, {B}, 0, true, 0, 4, 2>", None, 4 * m2 * n2 + 2 * n2, 4 * m2 * n2),
        ("fwd_vec_kernel_add_rmsnorm_fp8_row_bf16_16384x7168",
         "fused Add+RMSNorm with E4M3 output, one scale per row, bf16, M=16384 N=7168",
         f"fwd_vec_kernel<{B}, {B}, 0, true, 1, 8, 2>", None, 4 * M * N + 2 * N,
         3 * M * N + 4 * M),
        ("fwd_vec_kernel_add_rmsnorm_fp8_g128_bf16_16384x7168",
         "fused Add+RMSNorm with E4M3 output, one scale per 128 columns, bf16, M=16384 N=7168",
         f"fwd_vec_kernel<{B}, {B}, 0, true, 2, 8, 2>", None, 4 * M * N + 2 * N,
         3 * M * N + 4 * M * (N // 128)),
        ("fwd_vec_kernel_add_rmsnorm_mxfp4_bf16_16384x7168",
         "fused Add+RMSNorm with MXFP4 output, bf16, M=16384 N=7168",
         f"fwd_vec_kernel<{B}, {B}, 0, true, 3, 8, 2>", None, 4 * M * N + 2 * N,
         2 * M * N + M * N // 2 + M * (N // 32)),
        ("fwd_vec_kernel_add_layernorm_bf16_16384x7168",
         "fused Add+LayerNorm with bias, bf16, M=16384 N=7168",
         f"fwd_vec_kernel<{B}, {B}, 1, true, 0, 4, 4>", None, 4 * M * N + 4 * N, 4 * M * N),
        ("bwd_vec_kernel_layernorm_bf16_32768x4096", "LayerNorm backward (dx, dw, db), bf16, "
         "M=32768 N=4096", f"bwd_vec_kernel<{B}, {B}, 1, false, 8, 1, false, false>",
         COLREDUCE_KERNEL, 4 * mb * nbk + 8 * mb + 2 * nbk, 2 * mb * nbk + 8 * nbk),
        ("bwd_vec_kernel_add_rmsnorm_bf16_16384x7168", "fused Add+RMSNorm backward (dh, dw), "
         "bf16, M=16384 N=7168", f"bwd_vec_kernel<{B}, {B}, 0, true, 8, 2, false, false>",
         COLREDUCE_KERNEL, 6 * M * N + 4 * M + 2 * N, 2 * M * N + 4 * N),
    ]


def summarize_secondary(trace_dir: str, fetch, write, f_scale: float, w_scale: float,
                        commands: dict):
    """One profile summary per secondary workload: its kernel's traced
    duration in the default bench command, and its HBM bytes per call from the
    counter runs (the main kernel plus, for the backwards, the column reduce
    that follows it), against the algorithmic bytes."""
    def seq(rows, name, follow):
        rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
        main, red = [], []
        for k, r in enumerate(rows):
            if name in r["Kernel_Name"]:
                main.append(float(r["Counter_Value"]))
                if follow:
                    nxt = next((q for q in rows[k + 1:] if follow in q["Kernel_Name"]), None)
                    red.append(float(nxt["Counter_Value"]) if nxt else 0.0)
        return main, red

    for stem, title, name, follow, alg_r, alg_w in _secondary_specs():
        fm, fr = seq(fetch, name, follow)
        wm, wr = seq(write, name, follow)
        durs = _trace_durations(trace_dir, name)
        red = _following_durations(trace_dir, name, follow) if follow else []
        if not fm or not wm or not durs:
            log(f"no dispatches of {name}; {stem} not written")
            continue
        rd = (sum(fm) / len(fm) + (sum(fr) / len(fr) if fr else 0.0)) * f_scale * 1024
        wt = (sum(wm) / len(wm) + (sum(wr) / len(wr) if wr else 0.0)) * w_scale * 1024
        us = sum(durs) / len(durs)
        srt = sorted(durs)
        med = srt[len(srt) // 2]
        out = [f"# {name}: {title}", "",
               "Kernel trace of the default bench command:", "", f"    {commands['trace']}", "",
               f"- dispatches: {len(durs)}; average {us:.2f} us, median {med:.2f} us, "
               f"min {srt[0]:.2f} us, max {srt[-1]:.2f} us",
               f"- algorithmic bytes {alg_r + alg_w} -> {(alg_r + alg_w) / us / 1e3:.1f} GB/s at "
               f"the average ({100 * (alg_r + alg_w) / us / 1e3 / HBM_PEAK_GBPS:.1f} % of 8 TB/s), "
               f"{(alg_r + alg_w) / med / 1e3:.1f} GB/s at the median"]
        if red:
            ra = sum(red) / len(red)
            out.append(f"- the column reduce after each: average {ra:.2f} us; the call "
                       f"(main kernel + column reduce) {us + ra:.2f} us -> "
                       f"{(alg_r + alg_w) / (us + ra) / 1e3:.1f} GB/s")
        out += ["",
               "HBM traffic per call from the counter runs"
               + (" (the main kernel plus the column reduce after it)" if follow else "")
               + ", with the device-copy calibration of the headline summary (FETCH_SIZE x "
               f"{f_scale:.4f}, WRITE_SIZE x {w_scale:.4f}):", "",
               f"    {commands['fetch']}", f"    {commands['write']}", "",
               "| | bytes per call | algorithmic bytes | ratio |", "|---|---|---|---|",
               f"| read | {rd:.0f} | {alg_r} | {rd / alg_r:.4f} |",
               f"| write | {wt:.0f} | {alg_w} | {wt / alg_w:.4f} |", ""]
        path = os.path.join(ROOT, "profiles", stem + ".md")
        with open(path, "w") as fh:
            fh.write("\n".join(out))
        log(f"wrote {path}")


DECODE_KERNEL = "fwd_vec_kernel<addrms::bf16_t, float, 0, true, 0, "
DECODE_N = 8192


def summarize_decode(trace_dir: str, commands: dict):
    """Profile summary of the decode workload (bf16 rows of 8192 with float32
    weights, the only workload of the bench with float32 weights): the traced
    kernel durations per batch size M, which the trace gives as the number of
    one-row blocks; kernel execution only, without the launch."""
    rows, _ = _csv_rows(trace_dir, "kernel_trace.csv")
    by_m = {}
    for r in rows:
        name = r["Kernel_Name"]
        if DECODE_KERNEL not in name:
            continue
        M = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
        targs = name[name.find("<") + 1:name.rfind(">")].split(",")
        kern = f"WPR {targs[-2].strip()}, VPL {targs[-1].strip()}"
        by_m.setdefault(M, (kern, []))[1].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not by_m:
        log("no decode dispatches in the trace; decode summary not written")
        return
    out = [f"# fwd_vec_kernel (bf16 rows, float32 weights): decode-shaped fused Add+RMSNorm, "
           f"N={DECODE_N}", "",
           "Kernel trace of the default bench command (eager calls and graph replays alike):",
           "", f"    {commands['trace']}", "",
           "Traced kernel execution per call, by batch size (one row per block); the bench "
           "line's decode entry gives the device time per call in a graph replay, the host "
           "time per eager call and the launch floor beside it.  Bytes: 8 M N + 4 N "
           "(x, r read; y, residual_out written; float32 w).  The counter runs skip this "
           "loop: at these sizes the bytes are the launch's, not a stream's.", "",
           "| M | kernel | dispatches | median us | p10 us | p90 us | GB/s at the median |",
           "|---|---|---|---|---|---|---|"]
    for M in sorted(by_m):
        kern, d = by_m[M]
        d = sorted(d)
        med, p10, p90 = d[len(d) // 2], d[int(0.1 * (len(d) - 1))], d[int(0.9 * (len(d) - 1))]
        nb = 8 * M * DECODE_N + 4 * DECODE_N
        out.append(f"| {M} | {kern} | {len(d)} | {med:.2f} | {p10:.2f} | {p90:.2f} | "
                   f"{nb / med / 1e3:.1f} |")
    path = os.path.join(ROOT, "profiles", "fwd_vec_kernel_add_rmsnorm_bf16_f32w_decode_n8192.md")
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    log(f"wrote {path}")


def summarize_bwd(stats, fetch, write, f_scale: float, w_scale: float, commands: dict):
    """The RMS backward's traffic (bf16 32768 x 4096): the main kernel and the
    column reduce that follows each of its dispatches, from the same counter
    runs and calibration as the headline."""
    M, N = 32768, 4096

    def seq(rows):
        rows = sorted(rows, key=lambda r: int(r.get("Dispatch_Id", r.get("Correlation_Id", 0))))
        main, red = [], []
        for k, r in enumerate(rows):
            if BWD_KERNEL in r["Kernel_Name"]:
                main.append(float(r["Counter_Value"]))
                nxt = next((q for q in rows[k + 1:] if COLREDUCE_KERNEL in q["Kernel_Name"]), None)
                if nxt is not None:
                    red.append(float(nxt["Counter_Value"]))
        return sum(main) / len(main), sum(red) / len(red)

    fm, fr = seq(fetch)
    wm, wr = seq(write)
    rd_main, wr_main = fm * f_scale * 1024, wm * w_scale * 1024
    rd_red, wr_red = fr * f_scale * 1024, wr * w_scale * 1024
    alg_read = 2 * 2 * M * N + 4 * M + 2 * N
    alg_write = 2 * M * N + 4 * N
    st = {r["Name"]: r for r in stats}
    main_us = next(float(r["AverageNs"]) / 1e3 for n, r in st.items() if BWD_KERNEL in n)
    out = [f"# {BWD_KERNEL}: RMSNorm backward, bf16, M={M} N={N}", "",
           "Kernel time from the kernel trace of the default bench command:", "",
           f"    {commands['trace']}", "",
           f"- main kernel average: {main_us:.2f} us over its dispatches "
           f"(algorithmic bytes {alg_read + alg_write} -> {(alg_read + alg_write) / main_us / 1e3:.1f} GB/s "
           f"for the main kernel alone)", "",
           "HBM traffic per call (the same two counter runs as the headline summary, "
           "with the RMS backward timed after it, and the same device-copy calibration):", "",
           f"    {commands['fetch']}", f"    {commands['write']}", "",
           "| kernel | read bytes | written bytes |", "|---|---|---|",
           f"| main (dy, x, rstd, w in; dx out; one dw partial row per block out) | {rd_main:.0f} | {wr_main:.0f} |",
           f"| column reduce (partial rows in; dw out) | {rd_red:.0f} | {wr_red:.0f} |",
           f"| algorithmic (dy, x, rstd, w in; dx, dw out) | {alg_read} | {alg_write} |", "",
           f"Whole call (main kernel + column reduce) against the algorithmic bytes: read "
           f"{(rd_main + rd_red) / alg_read:.4f}, written {(wr_main + wr_red) / alg_write:.4f}. "
           f"The excess is the dw partial rows, 4 bytes per column per block of the persistent "
           f"grid (here about {(wr_main - 2 * M * N) / (4 * N):.0f} rows), written once by the "
           f"main kernel and read once by the column reduce.", ""]
    with open(BWD_TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out))
    log(f"wrote {BWD_TRAFFIC_FILE}")


PROBE_PROFILE = os.path.join(ROOT, "profiles", "stream_probes_16384x7168.md")
PROBE_KERNELS = ("mix_kernel", "lds_kernel", "pipe_kernel", "pers_kernel", "fwd_vec_kernel")


def _probe_streams(kernel_name: str):
    """(reads, writes) of a probe kernel from its template arguments."""
    import re
    m = re.search(r"(?:mix|pers)_kernel<(\d+), (\d+)", kernel_name)
    if m:
        return int(m.group(1)), int(m.group(2))
    return 2, 2  # lds_kernel, pipe_kernel and the fused forward


def summarize_probes(timing_json: str, trace_dir: str, pmc_dirs: dict, commands: dict):
    """Write profiles/stream_probes_16384x7168.md: for every stream probe (and
    the fused forward beside them) the event-timed bandwidth and, from four
    rocprofv3 counter passes, the bytes moved, the fraction of L2 (TCC)
    cycles its requests to memory were stalled for lack of DRAM credits, the
    average request latency and the L2 busy fraction; then the kernel-trace
    durations and the figures they pin.  The counter runs list the entries
    in dispatch order (bench.py --probe-matrix --probe-calls 4: 3 warm-up and
    4 counted dispatches each); the counted dispatches are averaged."""
    import csv
    import glob
    timing = json.load(open(timing_json))
    tmatrix = timing["probe_matrix"]
    each = timing["bytes_each_stream"]

    def counters(d):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        disp = {}
        for r in csv.DictReader(open(f)):
            if any(k in r["Kernel_Name"] for k in PROBE_KERNELS):
                disp.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = \
                    float(r["Counter_Value"])
        return [disp[k] for k in sorted(disp)]

    log_text = open(pmc_dirs["fetch"] + ".log").read()
    order = list(json.loads(next(ln for ln in log_text.splitlines()
                                 if ln.startswith('{"probe_matrix"')))["probe_matrix"])
    warm, calls = 3, 4
    per = {n: {} for n in order}
    for d in pmc_dirs.values():
        seq = counters(d)
        if len(seq) != len(order) * (warm + calls):
            raise SystemExit(f"{d}: {len(seq)} dispatches, expected {len(order) * (warm + calls)}")
        for i, n in enumerate(order):
            grp = seq[i * (warm + calls) + warm:(i + 1) * (warm + calls)]
            for c in grp[0]:
                per[n][c] = sum(g[c] for g in grp) / len(grp)
    # byte calibration: the one-stream read and write probes of known size
    f_cal = each / (per["r1_b512_u2"]["FETCH_SIZE"] * 1024)
    w_cal = each / (per["w1_b512_u2"]["WRITE_SIZE"] * 1024)
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    traced = [(r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3)
              for r in csv.DictReader(open(f)) if any(k in r["Name"] for k in PROBE_KERNELS)]

    out = ["# Stream probes and the fused forward at the headline byte count (bf16 16384 x 7168)",
           "",
           "Pure streaming kernels (`add_rmsnorm_amd/csrc/stream_probe.hip`), each stream "
           f"{each} bytes (a quarter of the fused forward's 939,538,432), and the fused "
           "forward itself (`kernel_fused_fwd`, in place: `..._inplace`), on one MI355X.",
           "", "Commands (from the repository root):", ""]
    out += [f"    {commands[k]}" for k in ("timing", "trace", "fetch", "write", "level", "busy")
            if k in commands]
    out += ["",
            f"Byte calibration: FETCH_SIZE x {f_cal:.4f} and WRITE_SIZE x {w_cal:.4f} (the "
            "one-stream read and write probes of known size). Stall columns: cycles the L2's "
            "read or write requests to memory waited for DRAM credits, as a fraction of L2 "
            "cycles (TCC_EA0_RDREQ/WRREQ_DRAM_CREDIT_STALL_sum / TCC_CYCLE_sum). Latency: "
            "average L2 cycles a request is in flight (TCC_EA0_*REQ_LEVEL_sum / "
            "TCC_EA0_*REQ_sum). Busy: TCC_BUSY_sum / TCC_CYCLE_sum.", "",
            "| entry | GB/s, event median | read, write bytes / stream | write stall | "
            "read stall | read latency | write latency | L2 busy |",
            "|---|---|---|---|---|---|---|---|"]
    for n in order:
        c = per[n]
        cyc = c.get("TCC_CYCLE_sum") or 1.0
        rl = c["TCC_EA0_RDREQ_LEVEL_sum"] / max(c["TCC_EA0_RDREQ_sum"], 1.0)
        wl = c["TCC_EA0_WRREQ_LEVEL_sum"] / max(c["TCC_EA0_WRREQ_sum"], 1.0)
        out.append(f"| `{n}` | {tmatrix[n]['GBps']:.0f} | "
                   f"{c['FETCH_SIZE'] * 1024 * f_cal / each:.2f}, "
                   f"{c['WRITE_SIZE'] * 1024 * w_cal / each:.2f} | "
                   f"{100 * c['TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum'] / cyc:.1f} % | "
                   f"{100 * c['TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum'] / cyc:.1f} % | "
                   f"{rl:.0f} | {wl:.0f} | {100 * c['TCC_BUSY_sum'] / cyc:.0f} % |")
    out += ["", "Kernel-trace durations (an in-place entry shares its kernel with the "
            "out-of-place one and is averaged in):", "",
            "| kernel | calls | avg us | GB/s |", "|---|---|---|---|"]
    rates = {}
    for name, n_calls, us in sorted(traced):
        rd, wr = _probe_streams(name)
        gbps = (rd + wr) * each / us / 1e3
        rates[name] = (rd, wr, gbps, us)
        short = name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]
        out.append(f"| `{short}` | {n_calls} | {us:.2f} | {gbps:.0f} |")
    best = lambda rd, wr: max((v[2] for k, v in rates.items()
                               if v[0] == rd and v[1] == wr and "fwd_vec" not in k), default=0.0)
    r2, w2 = best(2, 0), best(0, 2)
    bound = 2.0 / (1.0 / r2 + 1.0 / w2)
    fused = next((v for k, v in rates.items() if HEADLINE_KERNEL in k), None)
    out += ["", "Figures these traces pin (GB/s over the bytes each kernel moves):", "",
            f"- read-only, one stream / two streams, best shape: {best(1, 0):.0f} / {r2:.0f}",
            f"- write-only, one stream / two streams, best shape: {best(0, 1):.0f} / {w2:.0f}",
            f"- two reads and two writes if the reads ran at the two-stream read rate, the "
            f"writes at the two-stream write rate, and never both at once "
            f"(2 / (1/read + 1/write)): {bound:.0f}",
            f"- 2 reads / 2 writes, best probe: {best(2, 2):.0f}",
            f"- 2 reads / 1 write, best probe: {best(2, 1):.0f}; 3 reads / 1 write: "
            f"{best(3, 1):.0f}"]
    if fused:
        out.append(f"- the fused forward: {fused[2]:.0f} ({fused[3]:.2f} us), "
                   f"{100 * fused[2] / best(2, 2):.1f} % of the best 2R2W probe, "
                   f"{100 * fused[2] / 8000:.1f} % of 8 TB/s")
    with open(PROBE_PROFILE, "w") as fh:
        fh.write("\n".join(out) + "\n")
    log(f"wrote {PROBE_PROFILE}")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, M: int, N: int, eps: float, target_s: float = 6.0, passes: int = 3):
    """The CPU oracle (single-threaded plain C, binary64) on the first rows of
    the same inputs, the median of `passes` passes; the row count is sized
    for about target_s seconds a pass (all M rows when they fit)."""
    import oracle
    x, r, w = inp["x"], inp["r"], inp["w"]
    probe = 256
    t0 = time.perf_counter()
    oracle.add_rmsnorm_fwd(x[:probe], r[:probe], w, eps)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(min(M, max(probe, target_s / max(per_row, 1e-9))))
    log(f"cpu baseline: oracle on {rows} rows, {passes} passes (~{rows * per_row:.1f} s each)")
    times = []
    for _ in range(passes):
        t0 = time.perf_counter()
        oracle.add_rmsnorm_fwd(x[:rows], r[:rows], w, eps)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    nbytes = 8 * rows * N + 2 * N
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows} of {M} rows of the same inputs, median of {passes} passes "
                      f"({', '.join(f'{t:.2f}' for t in times)} s); rows/s {rows / dt:.0f}",
            "cpu": _cpu_model()}


def cpu_baseline_all_cores(inp, M: int, N: int, eps: float, max_threads: int = 16):
    """The same oracle, unchanged, run on disjoint slices of all M rows by one
    host thread per available core (each slice is one call into the C
    oracle, which releases the GIL), capped at max_threads."""
    import concurrent.futures as cf
    import oracle
    x, r, w = inp["x"], inp["r"], inp["w"]
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    n = max(1, min(avail, max_threads))
    bounds = [(k * M // n, (k + 1) * M // n) for k in range(n)]
    log(f"cpu baseline: oracle on all {M} rows in {n} threads, 3 passes")
    times = []
    with cf.ThreadPoolExecutor(n) as ex:
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(lambda b: oracle.add_rmsnorm_fwd(x[b[0]:b[1]], r[b[0]:b[1]], w, eps),
                        bounds))
            times.append(time.perf_counter() - t0)
    dt = sorted(times)[1]
    nbytes = 8 * M * N + 2 * N
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"all {M} rows in {n} row slices, median of 3 passes "
                      f"({', '.join(f'{t:.2f}' for t in times)} s); rows/s {M / dt:.0f}; "
                      f"{avail} cores available (sched_getaffinity)", "cpu": _cpu_model()}


def rms_bwd(calls: int):
    """The RMS backward, bf16 32768 x 4096, rstd from the GPU forward."""
    import torch
    import add_rmsnorm_amd as ar
    import synth

    out = {}
    cfg = synth.WORKLOADS["rmsnorm_bwd_bf16_32768x4096"]
    M, N = cfg["M"], cfg["N"]
    inp = synth.workload_inputs("rmsnorm_bwd_bf16_32768x4096")
    w = inp["w"].cuda()
    sets = []
    for _ in range(2):
        x, dy = inp["x"].cuda(), inp["dy"].cuda()
        _, rstd = ar.rmsnorm_fwd(x, w, cfg["eps"], return_rstd=True)
        sets.append((dy, x, rstd, torch.empty_like(x), torch.empty(N, device="cuda")))
    ws = torch.empty(ar.rmsnorm_bwd_workspace_bytes(M, N), dtype=torch.uint8, device="cuda")
    i = [0]

    def bstep():
        dy, x, rstd, dx, dw = sets[i[0] & 1]
        ar.rmsnorm_bwd(dy, x, w, rstd, dx=dx, dw=dw, workspace=ws)
        i[0] += 1

    nb = 6 * M * N + 4 * M + 2 * N + 4 * N
    out["rmsnorm_bwd_bf16_32768x4096"] = figure(bstep, nb, calls,
                                                note="dx, dw; main kernel + column reduce")
    del sets
    return out


def cpu_baseline_configs(target_s: float = 1.0):
    """The oracle (single-threaded, unchanged) on each of the other workloads:
    a bounded sample of rows (all rows when they fit in about target_s), the
    median of 3 passes, rows/s and GB/s over the same algorithmic bytes as
    the GPU figures."""
    import oracle
    import synth
    out = {}

    def run(name, fn, per_row_bytes, once_bytes, M):
        probe = min(M, 16)
        t0 = time.perf_counter()
        fn(probe)
        per_row = (time.perf_counter() - t0) / probe
        rows = int(min(M, max(probe, target_s / max(per_row, 1e-9))))
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn(rows)
            times.append(time.perf_counter() - t0)
        dt = sorted(times)[1]
        out[name] = {"rows": rows, "of_rows": M, "seconds": round(dt, 3), "passes": 3,
                     "rows_per_s": round(rows / dt, 1),
                     "GBps": round((per_row_bytes * rows + once_bytes) / dt / 1e9, 4), "cores": 1}

    c = synth.WORKLOADS["rmsnorm_fwd_f32_256x4096"]
    inp = synth.workload_inputs("rmsnorm_fwd_f32_256x4096")
    run("rmsnorm_fwd_f32_256x4096", lambda n: oracle.rmsnorm_fwd(inp["x"][:n], inp["w"], c["eps"]),
        8 * c["N"], 4 * c["N"], c["M"])
    c = synth.WORKLOADS["add_rmsnorm_fwd_bf16_4096x4096"]
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_4096x4096", M=2048)
    run("add_rmsnorm_fwd_bf16_4096x4096",
        lambda n: oracle.add_rmsnorm_fwd(inp["x"][:n], inp["r"][:n], inp["w"], c["eps"]),
        8 * c["N"], 2 * c["N"], 2048)
    out["add_rmsnorm_fwd_bf16_4096x4096"]["of_rows"] = c["M"]
    c = synth.WORKLOADS["add_rmsnorm_fwd_bf16_decode_n8192"]
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_decode_n8192", M=512)
    run("add_rmsnorm_fwd_bf16_decode_n8192_m512",
        lambda n: oracle.add_rmsnorm_fwd(inp["x"][:n], inp["r"][:n], inp["w"], c["eps"]),
        8 * c["N"], 4 * c["N"], 512)
    c = synth.WORKLOADS["rmsnorm_bwd_bf16_32768x4096"]
    inp = synth.workload_inputs("rmsnorm_bwd_bf16_32768x4096", M=2048)
    rstd = oracle.rmsnorm_fwd(inp["x"], inp["w"], c["eps"])[1]
    run("rmsnorm_bwd_bf16_32768x4096",
        lambda n: oracle.rmsnorm_bwd(inp["dy"][:n], inp["x"][:n], inp["w"], rstd[:n]),
        6 * c["N"] + 4, 6 * c["N"], 2048)
    out["rmsnorm_bwd_bf16_32768x4096"]["of_rows"] = c["M"]
    return out


def secondary(calls: int, profile_run: bool = False):
    """Backward, quantised and LayerNorm forwards, RMSNorm + RoPE, smaller
    forward shapes and decode latency: every figure from per-call event
    pairs over `calls` calls (median, p10, p90)."""
    import torch
    import add_rmsnorm_amd as ar
    import synth

    out = rms_bwd(calls)
    # the headline forward in place (y over x, residual_out over r), as an
    # inference engine updates its residual stream
    inp = synth.workload_inputs(WORKLOAD)
    M, N = 16384, 7168
    w = inp["w"].cuda()
    sets = [(inp["x"].cuda(), inp["r"].cuda()) for _ in range(2)]
    i = [0]

    def ipstep():
        x, r = sets[i[0] & 1]
        ar.add_rmsnorm_fwd(x, r, w, 1e-6, y=x, residual_out=r)
        i[0] += 1

    out["add_rmsnorm_fwd_bf16_16384x7168_inplace"] = figure(
        ipstep, 8 * M * N + 2 * N, calls, note="y written over x, residual_out over r")
    del sets
    # the headline shape with float16 storage (x, r, w, y, residual_out)
    inp = synth.add_rmsnorm_fwd_inputs(M, N, torch.float16, seed=0, r_std=0.5)
    w = inp["w"].cuda()
    sets = []
    for _ in range(2):
        x, r = inp["x"].cuda(), inp["r"].cuda()
        sets.append((x, r, torch.empty_like(x), torch.empty_like(x)))

    def h16():
        x, r, y, res = sets[i[0] & 1]
        ar.add_rmsnorm_fwd(x, r, w, 1e-6, y=y, residual_out=res)
        i[0] += 1

    out["add_rmsnorm_fwd_f16_16384x7168"] = figure(
        h16, 8 * M * N + 2 * N, calls, note="float16 x, r, w in; float16 y, residual_out out")
    del sets, inp
    i = [0]
    # backward of the fused op at the headline shape: dy, dres, h read; dh written
    M, N = 16384, 7168
    inp = synth.workload_inputs(WORKLOAD)
    w = inp["w"].cuda()
    h = inp["x"].cuda()
    _, rstd = ar.rmsnorm_fwd(h, w, 1e-6, return_rstd=True)
    dy, dres = inp["r"].cuda(), inp["x"].cuda()
    sets = [(dy, dres, h, torch.empty_like(h)), (dres, dy, h, torch.empty_like(h))]
    ws = torch.empty(ar.rmsnorm_bwd_workspace_bytes(M, N), dtype=torch.uint8, device="cuda")
    dw = torch.empty(N, device="cuda")

    def fbstep():
        a, b, hh, dh = sets[i[0] & 1]
        ar.add_rmsnorm_bwd(a, b, hh, w, rstd, dh=dh, dw=dw, workspace=ws)
        i[0] += 1

    nb = 8 * M * N + 4 * M + 2 * N + 4 * N
    out["add_rmsnorm_bwd_bf16_16384x7168"] = figure(
        fbstep, nb, calls,
        note="reads dy, d(residual_out), residual_out; writes dh (= dx = dr) and dw")
    del sets, ws, h, dy, dres
    # FP8 output: fused Add+RMSNorm at the headline shape writing E4M3 codes
    # and a per-row scale instead of bf16 y
    M, N = 16384, 7168
    inp = synth.workload_inputs(WORKLOAD)
    w = inp["w"].cuda()
    sets = []
    for _ in range(2):
        x, r = inp["x"].cuda(), inp["r"].cuda()
        sets.append((x, r, torch.empty(M, N, dtype=torch.uint8, device="cuda"),
                     torch.empty(M, device="cuda"), torch.empty_like(x)))

    def f8():
        x, r, q, sc, res = sets[i[0] & 1]
        ar.add_rmsnorm_fwd_fp8(x, r, w, 1e-6, y_fp8=q, y_scale=sc, residual_out=res)
        i[0] += 1

    nb = 7 * M * N + 4 * M + 2 * N
    out["add_rmsnorm_fwd_fp8_16384x7168"] = figure(
        f8, nb, calls, note="bf16 x, r in; bf16 residual_out + E4M3 y + fp32 per-row scale out")
    # the same with one scale per 128 columns of a row
    sg = [torch.empty(M, N // 128, device="cuda") for _ in range(2)]

    def f8g():
        x, r, q, _, res = sets[i[0] & 1]
        ar.add_rmsnorm_fwd_fp8(x, r, w, 1e-6, group=128, y_fp8=q, y_scale=sg[i[0] & 1],
                               residual_out=res)
        i[0] += 1

    nb = 7 * M * N + 4 * M * (N // 128) + 2 * N
    out["add_rmsnorm_fwd_fp8_g128_16384x7168"] = figure(
        f8g, nb, calls, note="as above with one fp32 scale per 128 columns (56 per row)")
    # MXFP4: E2M1 codes two per byte, one E8M0 scale byte per 32 values
    mq = [torch.empty(M, N // 2, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ms = [torch.empty(M, N // 32, dtype=torch.uint8, device="cuda") for _ in range(2)]

    def mx():
        x, r, _, _, res = sets[i[0] & 1]
        ar.add_rmsnorm_fwd_mxfp4(x, r, w, 1e-6, y_fp4=mq[i[0] & 1], y_scale=ms[i[0] & 1],
                                 residual_out=res)
        i[0] += 1

    nb = 4 * M * N + 2 * M * N + M * N // 2 + M * (N // 32) + 2 * N
    out["add_rmsnorm_fwd_mxfp4_16384x7168"] = figure(
        mx, nb, calls,
        note="bf16 x, r in; bf16 residual_out + MXFP4 y (E2M1 x2 per byte + E8M0 per 32) out")
    del sets, sg, mq, ms
    # LayerNorm: fused forward with bias at the headline shape, backward (dw, db)
    # at the backward workload's shape
    M, N = 16384, 7168
    inp = synth.workload_inputs(WORKLOAD)
    w = inp["w"].cuda()
    b = (inp["w"].float() - 1.0).to(torch.bfloat16).cuda()
    sets = []
    for _ in range(2):
        x, r = inp["x"].cuda(), inp["r"].cuda()
        sets.append((x, r, torch.empty_like(x), torch.empty_like(x)))

    def lnf():
        x, r, y, res = sets[i[0] & 1]
        ar.add_layernorm_fwd(x, r, w, b, 1e-5, y=y, residual_out=res)
        i[0] += 1

    nb = 8 * M * N + 4 * N
    out["add_layernorm_fwd_bf16_16384x7168"] = figure(lnf, nb, calls, note="with bias")
    del sets
    M, N = 32768, 4096
    inp = synth.workload_inputs("rmsnorm_bwd_bf16_32768x4096")
    w = inp["w"].cuda()
    sets = []
    for _ in range(2):
        x, dy = inp["x"].cuda(), inp["dy"].cuda()
        _, mean, rstd = ar.layernorm_fwd(x, w, None, 1e-5, return_stats=True)
        sets.append((dy, x, mean, rstd, torch.empty_like(x)))
    ws = torch.empty(ar.layernorm_bwd_workspace_bytes(M, N), dtype=torch.uint8, device="cuda")
    dw, db = torch.empty(N, device="cuda"), torch.empty(N, device="cuda")

    def lnb():
        dy, x, mean, rstd, dx = sets[i[0] & 1]
        ar.layernorm_bwd(dy, x, w, mean, rstd, dx=dx, dw=dw, db=db, workspace=ws)
        i[0] += 1

    nb = 6 * M * N + 8 * M + 2 * N + 8 * N
    out["layernorm_bwd_bf16_32768x4096"] = figure(lnb, nb, calls, note="dx, dw, db")
    del sets, ws
    # per-head RMSNorm + RoPE of the query and key heads, in place on a packed
    # projection buffer: 16384 tokens (4 sequences of 4096), 32 + 8 heads of 128
    name = "rmsnorm_rope_bf16_t16384_q32_k8_d128"
    c = synth.WORKLOADS[name]
    inp = synth.workload_inputs(name)
    T, Hq, Hk, D = c["T"], c["Hq"], c["Hk"], c["D"]
    wq, wk, cos, sin, pos = (inp[n].cuda() for n in ("wq", "wk", "cos", "sin", "pos"))
    bufs = [inp["qkv"].cuda() for _ in range(3)]  # 3 x 168 MB of heads: not cache-resident
    views = [(b[:, :Hq * D].view(T, Hq, D), b[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D))
             for b in bufs]
    i = [0]

    def rstep():
        q, k = views[i[0] % 3]
        ar.rmsnorm_rope_qk(q, k, wq, wk, cos, sin, pos, c["eps"], q_out=q, k_out=k)
        i[0] += 1

    npos = int(torch.unique(inp["pos"]).numel())
    # heads read and written; positions; the table rows used (cos and sin,
    # D/2 floats each); both weight vectors
    nb = 4 * T * (Hq + Hk) * D + 8 * T + npos * D * 4 + 2 * D * 2
    dev_s = graph_time(rstep, per_graph=30, replays=5) if not profile_run else None
    out[name] = figure(
        rstep, nb, calls, GBps_graph=round(nb / dev_s / 1e9, 1) if dev_s else None,
        us_per_call_graph=round(dev_s * 1e6, 2) if dev_s else None,
        note="in place on packed qkv [16384, 48*128]; value heads untouched; 3 rotating sets; "
             "_graph: device time from replaying captured calls")
    del bufs, views
    # fused forward, 4096 x 4096 bf16 (134 MB: fits in the last-level cache; rotate 4 sets)
    inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_4096x4096")
    M, N = 4096, 4096
    w = inp["w"].cuda()
    sets = [(inp["x"].cuda(), inp["r"].cuda()) for _ in range(4)]
    sets = [(x, r, torch.empty_like(x), torch.empty_like(x)) for x, r in sets]

    def fstep():
        x, r, y, res = sets[i[0] & 3]
        ar.add_rmsnorm_fwd(x, r, w, 1e-6, y=y, residual_out=res)
        i[0] += 1

    nb = 8 * M * N + 2 * N
    out["add_rmsnorm_fwd_bf16_4096x4096"] = figure(fstep, nb, calls,
                                                   note="4 rotating buffer sets (537 MB)")
    del sets
    # plain fp32 forward 256 x 4096 (8 MB: cache-resident, launch-bound)
    inp = synth.workload_inputs("rmsnorm_fwd_f32_256x4096")
    x, w = inp["x"].cuda(), inp["w"].cuda()
    y = torch.empty_like(x)
    plain = lambda: ar.rmsnorm_fwd(x, w, 1e-6, y=y)
    if profile_run:  # counter runs: no graph replays, no decode loop
        return out
    dev_s = graph_time(plain)
    nb = 8 * 256 * 4096 + 4 * 4096
    out["rmsnorm_fwd_f32_256x4096"] = figure(
        plain, nb, calls, GBps_graph=round(nb / dev_s / 1e9, 1),
        us_per_call_graph=round(dev_s * 1e6, 2),
        note="cache-resident, launch-bound: the event pairs time each eagerly launched call; "
             "_graph: device time per call replaying a captured graph of 50 calls")
    # decode: N = 8192, fp32 w, M in {1, 8, 32, 128, 512}: device time per call
    # (replay of a captured graph of calls) and host wall time per eager call
    dec = {}
    for M in synth.WORKLOADS["add_rmsnorm_fwd_bf16_decode_n8192"]["M_list"]:
        inp = synth.workload_inputs("add_rmsnorm_fwd_bf16_decode_n8192", M=M)
        x, r, w = inp["x"].cuda(), inp["r"].cuda(), inp["w"].cuda()
        y, res = torch.empty_like(x), torch.empty_like(x)
        call = lambda: ar.add_rmsnorm_fwd(x, r, w, 1e-5, y=y, residual_out=res)
        dev_s = graph_time(call)
        n = max(calls, 200)
        wall, _ = timed(call, n, 20)
        nb = 8 * M * 8192 + 4 * 8192
        t = per_call(call, calls, 5)
        dec[str(M)] = {"us_per_call_device": round(dev_s * 1e6, 2),
                       "us_per_call_host": round(wall / n * 1e6, 2),
                       "GBps_device": round(nb / dev_s / 1e9, 1), "bytes": nb,
                       "event_pair_median_us": t["median_us"], "event_pair_p10_us": t["p10_us"],
                       "event_pair_p90_us": t["p90_us"], "calls": calls}
    dec["binding"] = "native" if ar.add_rmsnorm_fwd is getattr(ar.native, "add_rmsnorm_fwd", 0) \
        else "ctypes"
    dec["launch_floor"] = launch_floor()
    out["add_rmsnorm_fwd_bf16_decode_n8192"] = dec
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-headline", action="store_true",
                    help="skip the secondary figures (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="for counter runs: secondary figures over 6 calls each, without graph "
                         "replays or the decode loop")
    ap.add_argument("--with-rms-bwd", action="store_true",
                    help="with --only-headline: also time the RMS backward (for counter runs)")
    ap.add_argument("--probe-matrix", action="store_true",
                    help="time every stream probe over the headline's byte count, print one "
                         "JSON line and exit")
    ap.add_argument("--probe-calls", type=int, default=30)
    ap.add_argument("--row-sweep", action="store_true",
                    help="time the fused forward over a range of row counts at two widths, "
                         "print one JSON line and exit")
    ap.add_argument("--summarize-row-sweep", nargs=2, metavar=("TRACE_DIR", "OUT"),
                    help="write the row-sweep profile summary from a traced --row-sweep run")
    ap.add_argument("--probe-only", default="",
                    help="comma-separated probe names for --probe-matrix (default: all)")
    ap.add_argument("--summarize-probes", nargs=2, metavar=("TIMING_JSON", "OUT_DIR"),
                    help="write the probe profile summary from the timing JSON and the "
                         "trace_probes and pmc_{fetch,write,level,busy} rocprofv3 runs under "
                         "OUT_DIR, and exit")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summary from rocprofv3 CSV output and exit")
    ap.add_argument("--profile-commands", default="{}",
                    help="JSON {trace, fetch, write}: the commands that made the CSVs")
    args = ap.parse_args()
    if args.summarize_probes:
        tj, d = args.summarize_probes
        summarize_probes(tj, os.path.join(d, "trace_probes"),
                         {k: os.path.join(d, f"pmc_{k}") for k in ("fetch", "write", "level", "busy")},
                         json.loads(args.profile_commands))
        return
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, commands=json.loads(args.profile_commands))
        return
    if args.summarize_row_sweep:
        summarize_row_sweep(*args.summarize_row_sweep, commands=json.loads(args.profile_commands))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: rows are independent, so more GPUs would each "
              "run this kernel on their own row block with no exchange; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.probe_matrix:
        each = (8 * 16384 * 7168) // 4
        only = set(args.probe_only.split(",")) if args.probe_only else None
        res = probe_matrix(each, args.probe_calls, only=only)
        if not args.probe_only:
            res.update(fused_fwd_inplace_compare(args.probe_calls))
        print(json.dumps({"probe_matrix": res, "bytes_each_stream": each,
                          "device": torch.cuda.get_device_name(0)}), flush=True)
        return

    if args.row_sweep:
        print(json.dumps({"row_sweep": row_sweep(), "device": torch.cuda.get_device_name(0)}),
              flush=True)
        return

    h = headline(args.steps, args.warmup)
    M, N, nb = h["M"], h["N"], h["nbytes"]
    gbps = nb * args.steps / h["wall"] / 1e9
    achieved = nb * args.steps / h["ev"] / 1e9  # per-launch average from the events
    log(f"fused fwd: {achieved:.1f} GB/s ({100 * achieved / HBM_PEAK_GBPS:.1f}% of 8 TB/s), "
        f"{h['ev'] / args.steps * 1e6:.2f} us per launch")
    per_call_dist = figure(h["step"], nb, max(100, args.steps))
    log(f"fused fwd per call: median {per_call_dist['median_us']} us, p10 {per_call_dist['p10_us']}, "
        f"p90 {per_call_dist['p90_us']}")
    log("copy-kernel and stream ceilings")
    copy = copy_ceiling(nb)
    stream = stream_ceiling(nb)
    traffic = traffic_from_profile(nb)
    rec = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["wall"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "M": M, "N": N, "storage_dtype": "bf16",
                   "w_dtype": "bf16", "eps": h["eps"], "bytes_per_step": nb,
                   "outputs": "y, residual_out (bf16)", "parallelism": "single GPU"},
        "pct_of_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "rows_per_s": round(M * args.steps / h["wall"], 0),
        "copy_ceiling_GBps": round(copy, 1),
        "pct_of_copy_ceiling": round(100 * gbps / copy, 1),
        "stream_2r2w_ceiling_GBps": round(stream, 1) if stream else None,
        "pct_of_stream_ceiling": round(100 * gbps / stream, 1) if stream else None,
        "per_call": per_call_dist,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "fwd_vec_kernel<bf16_t, bf16_t, kRms, fused, bf16 out, 16, 1> (16 waves/row, "
                               "one 16 B vector per lane and tensor, one row per block)",
                     "avg_launch_us": round(h["ev"] / args.steps * 1e6, 3)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(h["inputs"], M, N, h["eps"])
        rec["cpu_baseline_all_cores"] = cpu_baseline_all_cores(h["inputs"], M, N, h["eps"])
        log("cpu baseline: oracle on the other workloads")
        rec["cpu_baseline_configs"] = cpu_baseline_configs()
    del h
    if not args.only_headline:
        log("secondary figures")
        rec["secondary"] = (secondary(6, profile_run=True) if args.profile_run
                            else secondary(max(100, args.steps)))
    elif args.with_rms_bwd:
        rec["secondary"] = rms_bwd(max(100, args.steps))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
