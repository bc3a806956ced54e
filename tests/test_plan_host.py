"""The dispatcher's launch choices, on the CPU (addrms_plan: no HIP call).

addrms_plan runs the same choice helpers as the calls themselves, for
aligned contiguous tensors on a device of a given CU count.  These tests pin
the choices for the named workloads on a 256-CU MI355X, the boundaries of
the measured rules, that the tuning knobs steer the plan, and that the kernel
names the benchmark reads from the profiler traces are the kernels the
dispatcher picks for those workloads (a stale name would leave a profile
summary describing a kernel that no longer runs)."""
import ctypes
import re

import pytest
import torch

import add_rmsnorm_amd as ar
import bench

BF, F32, F16 = torch.bfloat16, torch.float32, torch.float16


def shape(p):
    return (p["waves_per_row"], p["vectors_per_lane"])


def test_named_workloads():
    # the fused bf16 forward of the headline shape: 16 waves of one vector
    assert shape(ar.plan("fwd", 16384, 7168)) == (16, 1)
    assert shape(ar.plan("fwd", 4096, 4096)) == (4, 2)
    # float32 plain forward, 256 x 4096
    assert shape(ar.plan("fwd", 256, 4096, F32, fused=False)) == (8, 2)
    # decode, N = 8192 with float32 weights: one row spread over 16 waves,
    # 128 rows and more over 8 waves of two
    for M in (1, 8, 32):
        assert shape(ar.plan("fwd", M, 8192, BF, F32)) == (16, 1), M
    for M in (128, 512):
        assert shape(ar.plan("fwd", M, 8192, BF, F32)) == (8, 2), M
    # the RMS and LayerNorm backwards of 32768 x 4096: the measured table's 8
    # waves of one vector on 2 blocks per CU, no prefetch
    for norm in ("rms", "layer"):
        p = ar.plan("bwd", 32768, 4096, fused=False, norm=norm)
        assert (shape(p), p["prefetch"], p["wide"], p["blocks_per_cu"]) == ((8, 1), 0, 0, 2), norm
    # the fused backward of 16384 x 7168: 8 waves of two, RMS grid of 2 per CU
    p = ar.plan("bwd", 16384, 7168)
    assert (shape(p), p["prefetch"], p["blocks_per_cu"]) == ((8, 2), 0, 2)
    # the fused LayerNorm forward of 16384 x 7168: 4 waves of up to 4 vectors
    assert shape(ar.plan("fwd", 16384, 7168, norm="layer")) == (4, 4)
    # quantised outputs of 16384 x 7168: 8 waves of two
    for q, g in (("fp8", 0), ("fp8_group", 128), ("mxfp4", 0)):
        assert shape(ar.plan("fwd", 16384, 7168, qmode=q, group=g)) == (8, 2), q
    # a row that is not a whole number of 16-byte vectors: element-wise
    assert ar.plan("fwd", 16384, 7170)["vector"] == 0


def test_forward_rule_boundaries():
    cus = 256
    # fused RMS, one vector a lane in 8 waves from 257 vectors (2056 bf16
    # columns) and 16 rows per CU; two vectors in 4 waves below either
    assert shape(ar.plan("fwd", 16 * cus, 2560)) == (8, 1)
    assert shape(ar.plan("fwd", 15 * cus, 2560)) == (4, 2)
    assert shape(ar.plan("fwd", 16 * cus, 2048)) == (2, 2)
    # 449 to 512 vectors from 64 rows per CU
    assert shape(ar.plan("fwd", 64 * cus, 4096)) == (8, 1)
    assert shape(ar.plan("fwd", 63 * cus, 4096)) == (4, 2)
    # 16 waves of one from 601 vectors and 8 rows per CU
    assert shape(ar.plan("fwd", 8 * cus, 4816)) == (16, 1)
    assert shape(ar.plan("fwd", 8 * cus, 4800)) == (8, 2)
    assert shape(ar.plan("fwd", 8 * cus - 1, 7168)) == (8, 2)
    # the fused RMS forward keeps one or two vectors a lane in every case, as
    # the plain one does (so their row sums agree bit for bit)
    for M in (512, 2048, 4096, 16384, 65536):
        for N in range(1024, 8193, 512):
            assert ar.plan("fwd", M, N)["vectors_per_lane"] <= 2, (M, N)
            assert ar.plan("fwd", M, N, fused=False)["vectors_per_lane"] <= 2, (M, N)
    # plain LayerNorm: up to 4 vectors a lane in the fewest waves (at least 2)
    assert shape(ar.plan("fwd", 16384, 5120, norm="layer", fused=False)) == (4, 3)
    assert shape(ar.plan("fwd", 16384, 3072, norm="layer", fused=False)) == (2, 3)
    # fused LayerNorm: 4 waves up to 960 vectors, 16 waves of one at 961-1024
    assert shape(ar.plan("fwd", 16384, 7680, norm="layer")) == (4, 4)
    assert shape(ar.plan("fwd", 16384, 8192, norm="layer")) == (16, 1)
    # quantised outputs at 513 to 640 vectors (768 for grouped E4M3): 4 waves
    assert shape(ar.plan("fwd", 8 * cus, 5120, qmode="fp8")) == (4, 3)
    assert shape(ar.plan("fwd", 8 * cus, 6144, qmode="fp8_group", group=128)) == (4, 3)
    assert shape(ar.plan("fwd", 8 * cus, 6144, qmode="fp8")) == (8, 2)


def test_backward_table_boundaries():
    cus = 256
    M = 32 * cus
    # below 32 rows per CU the rules decide: 2 waves of 4 vectors, in the
    # 1024-thread wide block up to 32 rows per CU from 8, with the prefetch
    # below that
    p = ar.plan("bwd", M - 1, 4096, fused=False)
    assert (shape(p), p["wide"], p["prefetch"], p["blocks_per_cu"]) == ((2, 4), 1, 0, 0)
    p = ar.plan("bwd", 8 * cus - 1, 4096, fused=False)
    assert (shape(p), p["wide"], p["prefetch"]) == ((2, 4), 0, 1)
    rows = {  # N: (RMS, fused RMS, LayerNorm, fused LayerNorm) as (WPR, prefetch)
        2560: ((2, 0), (2, 1), (2, 1), (2, 1)),
        3584: ((8, 0), (2, 0), (8, 0), (8, 0)),
        4096: ((8, 0), (8, 0), (8, 0), (8, 0)),
    }
    for N, want in rows.items():
        got = []
        for norm, fused in (("rms", False), ("rms", True), ("layer", False), ("layer", True)):
            p = ar.plan("bwd", M, N, norm=norm, fused=fused)
            assert p["blocks_per_cu"] == 2 and p["wide"] == 0, (N, norm, fused)
            got.append((p["waves_per_row"], p["prefetch"]))
        assert tuple(got) == want, N
    # RMS only: 4 waves at 641-768 vectors, 8 at 961-1024
    assert ar.plan("bwd", M, 6144, fused=False)["waves_per_row"] == 4
    assert ar.plan("bwd", M, 8192, fused=False)["waves_per_row"] == 8
    # float32 rows: their own entries
    assert (shape(ar.plan("bwd", M, 2048, F32, fused=False)), ar.plan("bwd", M, 2048, F32,
                                                                      fused=False)["prefetch"]) \
        == ((8, 1), 0)
    assert ar.plan("bwd", M, 1536, F32, fused=False)["prefetch"] == 1
    # float16 rows take the 16-bit table
    assert shape(ar.plan("bwd", M, 4096, F16, fused=False)) == (8, 1)


def test_knobs_steer_the_plan():
    with ar.tuning(FWD_WPR=2):
        assert ar.plan("fwd", 16384, 7168)["waves_per_row"] == 2
    with ar.tuning(BWD_WPR=2, BWD_PREFETCH=2, BWD_WIDE=2):
        p = ar.plan("bwd", 32768, 4096, fused=False)
        assert (p["waves_per_row"], p["prefetch"], p["wide"]) == (2, 0, 0)
    with ar.tuning(FORCE_ELEM=1):
        assert ar.plan("fwd", 16384, 7168)["vector"] == 0
    assert shape(ar.plan("fwd", 16384, 7168)) == (16, 1)


def _template_ints(name):
    args = re.search(r"<(.*)>", name).group(1).split(",")
    out = []
    for a in args:
        a = a.strip()
        out.append({"true": 1, "false": 0}.get(a, a))
    return out


def test_benchmark_kernel_names_are_the_kernels_picked():
    # fwd_vec_kernel<T, WT, NORM, FUSED, QM, WPR, VPL>
    t = _template_ints(bench.HEADLINE_KERNEL)
    assert (int(t[5]), int(t[6])) == shape(ar.plan("fwd", 16384, 7168))
    # bwd_vec_kernel<T, WT, NORM, RES, WPR, VPL, WIDE, PF>
    t = _template_ints(bench.BWD_KERNEL)
    p = ar.plan("bwd", 32768, 4096, fused=False)
    assert (int(t[4]), int(t[5]), t[6], t[7]) == (p["waves_per_row"], p["vectors_per_lane"],
                                                 p["wide"], p["prefetch"])
    # the secondary workloads' kernels, by their profile summaries' stems
    plans = {
        "fwd_vec_kernel_add_rmsnorm_bf16_4096x4096": ar.plan("fwd", 4096, 4096),
        "fwd_vec_kernel_add_rmsnorm_fp8_row_bf16_16384x7168": ar.plan("fwd", 16384, 7168,
                                                                      qmode="fp8"),
        "fwd_vec_kernel_add_rmsnorm_fp8_g128_bf16_16384x7168": ar.plan(
            "fwd", 16384, 7168, qmode="fp8_group", group=128),
        "fwd_vec_kernel_add_rmsnorm_mxfp4_bf16_16384x7168": ar.plan("fwd", 16384, 7168,
                                                                    qmode="mxfp4"),
        "fwd_vec_kernel_add_layernorm_bf16_16384x7168": ar.plan("fwd", 16384, 7168,
                                                                norm="layer"),
        "bwd_vec_kernel_layernorm_bf16_32768x4096": ar.plan("bwd", 32768, 4096, fused=False,
                                                            norm="layer"),
        "bwd_vec_kernel_add_rmsnorm_bf16_16384x7168": ar.plan("bwd", 16384, 7168),
    }
    specs = {s[0]: s[2] for s in bench._secondary_specs()}
    assert set(plans) <= set(specs)
    for stem, p in plans.items():
        t = _template_ints(specs[stem])
        if specs[stem].startswith("fwd"):
            assert (int(t[5]), int(t[6])) == shape(p), stem
        else:
            assert (int(t[4]), int(t[5]), t[6], t[7]) == (
                p["waves_per_row"], p["vectors_per_lane"], p["wide"], p["prefetch"]), stem


def test_plan_errors():
    out = ar._Plan()
    lib = ar.lib
    assert lib.addrms_plan(0, 0, 1, 0, 0, 16, 4096, 1, 1, 256, None) == -1   # NULL out
    assert lib.addrms_plan(0, 0, 1, 0, 0, 16, 4096, 7, 1, 256, ctypes.byref(out)) == -3
    for args in ((2, 0, 1, 0, 0, 16, 4096),     # unknown op
                 (0, 2, 1, 0, 0, 16, 4096),     # unknown norm
                 (0, 0, 1, 4, 0, 16, 4096),     # unknown output mode
                 (1, 0, 1, 1, 0, 16, 4096),     # a quantised backward
                 (0, 1, 1, 1, 0, 16, 4096),     # a quantised LayerNorm
                 (0, 0, 1, 0, 0, 0, 4096),      # no rows
                 (0, 0, 1, 0, 0, 16, 0)):       # no columns
        assert lib.addrms_plan(*args, 1, 1, 256, ctypes.byref(out)) == -2, args
    assert lib.addrms_plan(0, 0, 1, 0, 0, 16, 4096, 1, 1, 0, ctypes.byref(out)) == -2  # no CUs
    with pytest.raises(ValueError):
        ar.plan("sideways", 16, 4096)
