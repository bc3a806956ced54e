"""The C ABI on the host (CPU only): the library loads, exports every entry
point include/addrms.h declares, sizes the backward workspace, and rejects bad
arguments before making any HIP call (fake, never-dereferenced addresses are
passed; on a validation error nothing is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "addrms.h")
# another build of the library (e.g. one with host-side sanitizers) may be tested
LIB = os.environ.get("ADDRMS_TEST_LIB") or os.path.join(ROOT, "add_rmsnorm_amd", "libaddrms.so")

OK, E_NULL, E_SHAPE, E_DTYPE, E_EPS, E_ALIAS, E_WS, E_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -8
F32, BF16 = 0, 1


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libaddrms.so is not built (python -m add_rmsnorm_amd.build)")
    lib = ctypes.CDLL(LIB)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.rmsnorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.add_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.rmsnorm_bwd_workspace_bytes.restype = sz
    lib.rmsnorm_bwd_workspace_bytes.argtypes = [i64, i64]
    lib.rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, i32, vp]
    lib.add_rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, i32, vp]
    lib.rmsnorm_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, vp]
    lib.layernorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.add_layernorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.layernorm_bwd_workspace_bytes.restype = sz
    lib.layernorm_bwd_workspace_bytes.argtypes = [i64, i64]
    lib.layernorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i32, i32, vp]
    lib.rmsnorm_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.add_rmsnorm_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.rmsnorm_fwd_fp8_grouped.argtypes = [vp, vp, vp, vp, i64, vp, i64, i64, f32, i32, i32, vp]
    lib.add_rmsnorm_fwd_fp8_grouped.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, i64, i64, f32,
                                                i32, i32, vp]
    lib.rmsnorm_fwd_mxfp4.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.add_rmsnorm_fwd_mxfp4.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
    lib.rmsnorm_rope_qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, i64, i64, i64, i64,
                                    i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.addrms_status_str.restype = ctypes.c_char_p
    lib.addrms_status_str.argtypes = [i32]
    return lib


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["rmsnorm_fwd", "add_rmsnorm_fwd", "rmsnorm_bwd",
                                  "rmsnorm_bwd_noalloc", "add_rmsnorm_bwd", "rmsnorm_bwd_workspace_bytes",
                                  "layernorm_fwd", "add_layernorm_fwd", "layernorm_bwd",
                                  "layernorm_bwd_workspace_bytes", "add_layernorm_bwd",
                                  "rmsnorm_fwd_fp8", "add_rmsnorm_fwd_fp8", "rmsnorm_fwd_fp8_grouped",
                                  "add_rmsnorm_fwd_fp8_grouped", "rmsnorm_fwd_mxfp4",
                                  "add_rmsnorm_fwd_mxfp4", "rmsnorm_rope_qk",
                                  "addrms_status_str", "addrms_last_hip_error", "addrms_tune",
                                  "addrms_plan"])


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (OK, E_NULL, E_SHAPE, E_DTYPE, E_EPS, E_ALIAS, E_WS, -7, E_SCRATCH):
        assert lib.addrms_status_str(st)
    assert lib.addrms_status_str(12345) == b"unknown status"


def test_workspace_bytes(lib):
    f = lib.rmsnorm_bwd_workspace_bytes
    assert f(0, 4096) == 0 and f(5, 0) == 0 and f(-1, 8) == 0
    assert f(1, 7) == 28
    assert f(32768, 4096) == 1024 * 4096 * 4
    assert f(100, 10) == 100 * 10 * 4
    assert f(1 << 40, 1 << 40) == 1024 * (1 << 40) * 4
    assert f(1 << 40, 1 << 62) == 0  # does not fit in size_t


# fake device addresses, 4 KiB apart blocks; never dereferenced
A, B, C, D, E, W = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000


def fwd(lib, x=A, w=W, y=B, rstd=None, M=4, N=64, eps=1e-6, dt=BF16, wdt=BF16):
    return lib.rmsnorm_fwd(x, w, y, rstd, M, N, eps, dt, wdt, None)


def add(lib, x=A, r=C, w=W, y=B, res=D, rstd=None, M=4, N=64, eps=1e-6, dt=BF16, wdt=BF16):
    return lib.add_rmsnorm_fwd(x, r, w, y, res, rstd, M, N, eps, dt, wdt, None)


def bwd(lib, dy=A, x=C, w=W, rstd=E, dx=B, dw=D, ws=0x70000000, wsb=None, M=4, N=64,
        dt=BF16, wdt=BF16):
    if wsb is None:
        wsb = lib.rmsnorm_bwd_workspace_bytes(M, N)
    return lib.rmsnorm_bwd(dy, x, w, rstd, dx, dw, ws, wsb, M, N, dt, wdt, None)


def abwd(lib, dy=A, dres=0x80000000, h=C, w=W, rstd=E, dh=B, dw=D, ws=0x70000000, wsb=None,
         M=4, N=64, dt=BF16, wdt=BF16):
    if wsb is None:
        wsb = lib.rmsnorm_bwd_workspace_bytes(M, N)
    return lib.add_rmsnorm_bwd(dy, dres, h, w, rstd, dh, dw, ws, wsb, M, N, dt, wdt, None)


def test_fused_backward_validation(lib):
    for k in ("dy", "h", "w", "rstd", "dh", "dw"):
        assert abwd(lib, **{k: None}) == E_NULL, k
    assert abwd(lib, M=-1) == E_SHAPE
    assert abwd(lib, dt=9) == E_DTYPE
    assert abwd(lib, ws=None) == E_WS
    assert abwd(lib, dh=0x80000000 + 2) == E_ALIAS  # dh partially over dres
    assert abwd(lib, dw=0x80000000) == E_ALIAS      # dw inside dres
    assert abwd(lib, ws=0x80000000 + 64) == E_ALIAS


def test_null_pointers(lib):
    assert fwd(lib, x=None) == E_NULL
    assert fwd(lib, w=None) == E_NULL
    assert fwd(lib, y=None) == E_NULL
    for k in ("x", "r", "w", "y", "res"):
        assert add(lib, **{k: None}) == E_NULL, k
    for k in ("dy", "x", "w", "rstd", "dx", "dw"):
        assert bwd(lib, **{k: None}) == E_NULL, k


def test_shapes(lib):
    assert fwd(lib, M=-1) == E_SHAPE
    assert fwd(lib, N=0) == E_SHAPE
    assert fwd(lib, N=-3) == E_SHAPE
    assert fwd(lib, N=1 << 31) == E_SHAPE
    assert fwd(lib, M=1 << 62, N=1 << 20) == E_SHAPE
    assert add(lib, N=0) == E_SHAPE
    assert bwd(lib, M=-2) == E_SHAPE


def test_dtypes(lib):
    assert fwd(lib, dt=3) == E_DTYPE
    assert fwd(lib, wdt=-1) == E_DTYPE
    assert add(lib, dt=7) == E_DTYPE
    assert bwd(lib, wdt=3) == E_DTYPE


def test_eps(lib):
    assert fwd(lib, eps=-1e-6) == E_EPS
    assert fwd(lib, eps=float("nan")) == E_EPS
    assert add(lib, eps=float("inf")) == E_EPS


def test_workspace_errors(lib):
    assert bwd(lib, ws=None) == E_WS
    assert bwd(lib, wsb=10) == E_WS


def test_aliasing(lib):
    mat = 4 * 64 * 2
    # partial overlap of an output with an input
    assert fwd(lib, y=A + 16) == E_ALIAS
    assert fwd(lib, y=W - 8) == E_ALIAS  # y tail overlaps w
    assert fwd(lib, rstd=A + 32) == E_ALIAS
    assert add(lib, y=D) == E_ALIAS  # y == residual_out
    assert add(lib, res=C + 2) == E_ALIAS
    assert add(lib, rstd=D + mat - 4) == E_ALIAS
    assert bwd(lib, dx=A + 2) == E_ALIAS
    assert bwd(lib, dw=A) == E_ALIAS
    assert bwd(lib, ws=C + mat - 16) == E_ALIAS
    assert bwd(lib, dw=E) == E_ALIAS  # dw overlaps rstd


def test_empty_batch_is_a_noop_without_device(lib):
    # M == 0 is valid and the forward returns before touching HIP; exact
    # aliasing of an output with its input is allowed.
    assert fwd(lib, M=0) == OK
    assert add(lib, M=0) == OK
    assert fwd(lib, M=0, y=A) == OK
    assert add(lib, M=0, res=C, y=A) == OK
    # empty matrices may be NULL; w may not
    assert fwd(lib, M=0, x=None, y=None) == OK
    assert add(lib, M=0, x=None, r=None, y=None, res=None) == OK
    assert fwd(lib, M=0, w=None) == E_NULL
    assert bwd(lib, M=0, dw=None) == E_NULL


def test_layernorm_validation(lib):
    WB = 0x68000000  # bias
    ln = lambda **k: lib.layernorm_fwd(k.get("x", A), k.get("w", W), k.get("b", WB),
                                       k.get("y", B), k.get("mean", None), k.get("rstd", None),
                                       k.get("M", 4), k.get("N", 64), k.get("eps", 1e-5),
                                       BF16, BF16, None)
    assert ln(x=None) == E_NULL and ln(w=None) == E_NULL
    assert ln(b=None, M=0) == OK and ln(M=0) == OK
    assert ln(N=0) == E_SHAPE and ln(eps=-1.0) == E_EPS
    assert ln(y=WB) == E_ALIAS            # y over the bias
    assert ln(mean=A + 4) == E_ALIAS      # mean inside x
    assert ln(mean=E, rstd=E + 8) == E_ALIAS  # mean and rstd overlap
    aln = lambda **k: lib.add_layernorm_fwd(A, C, W, k.get("b", WB), B, k.get("res", D), None,
                                            None, 4, 64, 1e-5, BF16, BF16, None)
    assert aln(res=None) == E_NULL and aln(res=WB) == E_ALIAS
    assert lib.layernorm_bwd_workspace_bytes(10, 8) == 2 * 10 * 8 * 4
    assert lib.layernorm_bwd_workspace_bytes(0, 8) == 0
    wsb = lib.layernorm_bwd_workspace_bytes(4, 64)
    lb = lambda **k: lib.layernorm_bwd(A, C, W, k.get("mean", 0x58000000), E, B, D,
                                       k.get("db", 0x48000000), k.get("ws", 0x70000000),
                                       k.get("wsb", wsb), 4, 64, BF16, BF16, None)
    assert lb(mean=None) == E_NULL
    assert lb(wsb=wsb - 1) == E_WS
    assert lb(db=D + 4) == E_ALIAS        # db overlaps dw
    assert lb(db=0x70000000 + 64) == E_ALIAS  # db inside the workspace


def test_fp8_validation(lib):
    Q, S = 0x78000000, 0x7C000000
    f = lambda **k: lib.rmsnorm_fwd_fp8(k.get("x", A), W, k.get("q", Q), k.get("s", S), None,
                                        k.get("M", 4), 64, 1e-6, BF16, BF16, None)
    assert f(q=None) == E_NULL and f(s=None) == E_NULL
    assert f(M=0, q=None, s=None) == OK
    assert f(q=A) == E_ALIAS          # codes over x (even though same start)
    assert f(s=Q + 8) == E_ALIAS      # scale inside the codes
    g = lambda **k: lib.add_rmsnorm_fwd_fp8(A, C, W, k.get("q", Q), S, k.get("res", D), None,
                                            4, 64, 1e-6, BF16, BF16, None)
    assert g(res=None) == E_NULL and g(q=C) == E_ALIAS and g(res=Q) == E_ALIAS


def test_rope_validation(lib):
    # a packed projection buffer of T tokens: Hq query, Hk key, Hk value heads
    T, Hq, Hk, D, P = 4, 4, 2, 64, 100
    S = (Hq + 2 * Hk) * D  # token stride, elements
    QKV, WQ, WK, COS, SIN, POS = 0x10000000, 0x60000000, 0x61000000, 0x62000000, 0x63000000, \
        0x64000000
    KB = QKV + Hq * D * 2  # key heads of token 0 (bf16)
    OUT = 0x70000000

    def rope(**k):
        g = lambda n, d: k.get(n, d)
        return lib.rmsnorm_rope_qk(g("q", QKV), g("k", KB), g("wq", WQ), g("wk", WK),
                                   g("cos", COS), g("sin", SIN), g("pos", POS), g("P", P),
                                   g("qo", OUT), g("ko", OUT + T * Hq * D * 2), g("T", T),
                                   g("Hq", Hq), g("Hk", Hk), g("D", D), g("qs", S), g("ks", S),
                                   g("qos", Hq * D), g("kos", Hk * D), g("eps", 1e-6),
                                   g("il", 0), g("dt", BF16), g("wdt", BF16), None)

    assert rope(dt=3) == E_DTYPE and rope(wdt=-1) == E_DTYPE
    assert rope(D=63) == E_SHAPE and rope(D=0) == E_SHAPE and rope(T=-1) == E_SHAPE
    assert rope(Hk=-1) == E_SHAPE and rope(P=-1) == E_SHAPE
    assert rope(qs=Hq * D - 1) == E_SHAPE     # heads of a token wider than the stride
    assert rope(kos=Hk * D - 8) == E_SHAPE
    assert rope(eps=-1.0) == E_EPS and rope(eps=float("nan")) == E_EPS
    # nothing to do: no launch, NULL pointers allowed
    assert rope(T=0, q=None, k=None, qo=None, ko=None, pos=None, cos=None, sin=None) == OK
    assert rope(Hq=0, Hk=0) == OK
    assert rope(q=None) == E_NULL and rope(pos=None) == E_NULL and rope(cos=None) == E_NULL
    assert rope(k=None) == E_NULL and rope(wk=None) == E_NULL and rope(ko=None) == E_NULL
    # outputs overlapping an input other than their own, or each other
    assert rope(qo=QKV + 2, qos=S) == E_ALIAS          # shifted view of q
    assert rope(qo=KB, qos=S) == E_ALIAS               # query output over the key heads
    assert rope(ko=QKV, kos=S) == E_ALIAS              # key output over the query heads
    assert rope(ko=OUT + 64) == E_ALIAS                # key output inside the query output
    assert rope(qo=COS) == E_ALIAS and rope(ko=POS - 16) == E_ALIAS
    assert rope(qo=WQ - 8) == E_ALIAS


def test_fp8_grouped_validation(lib):
    Q, S = 0x78000000, 0x7C000000
    f = lambda **k: lib.rmsnorm_fwd_fp8_grouped(A, W, k.get("q", Q), k.get("s", S),
                                                k.get("g", 128), None, k.get("M", 4),
                                                k.get("N", 64), 1e-6, BF16, BF16, None)
    assert f(g=0) == E_SHAPE and f(g=-128) == E_SHAPE
    assert f(q=None) == E_NULL and f(s=None) == E_NULL
    assert f(M=0, q=None, s=None) == OK and f(M=0) == OK
    # 4 rows x ceil(64 / 16) = 4 scales per row: 64 bytes of scales
    assert f(g=16, s=Q + 4 * 64 - 8) == E_ALIAS     # scales run into the codes' tail
    assert f(g=16, s=W - 60) == E_ALIAS             # scales run into w
    g = lambda **k: lib.add_rmsnorm_fwd_fp8_grouped(A, C, W, Q, k.get("s", S), k.get("g", 32),
                                                    k.get("res", D), None, 4, 64, 1e-6, BF16,
                                                    BF16, None)
    assert g(g=0) == E_SHAPE and g(res=None) == E_NULL and g(s=D + 8) == E_ALIAS


def test_mxfp4_validation(lib):
    Q, S = 0x78000000, 0x7C000000
    f = lambda **k: lib.rmsnorm_fwd_mxfp4(k.get("x", A), W, k.get("q", Q), k.get("s", S), None,
                                          k.get("M", 4), k.get("N", 64), 1e-6, BF16, BF16, None)
    assert f(N=63) == E_SHAPE                       # two codes per byte: N must be even
    assert f(q=None) == E_NULL and f(s=None) == E_NULL
    assert f(M=0, q=None, s=None) == OK
    # codes: 4 rows x 32 bytes = 128 bytes; scales: 4 x 2 = 8 bytes
    assert f(s=Q + 124) == E_ALIAS                  # scales run into the codes' tail
    assert f(q=A + 64) == E_ALIAS                   # codes inside x
    g = lambda **k: lib.add_rmsnorm_fwd_mxfp4(A, C, W, k.get("q", Q), k.get("s", S),
                                              k.get("res", D), None, 4, 64, 1e-6, BF16, BF16,
                                              None)
    assert g(res=None) == E_NULL and g(q=C) == E_ALIAS and g(s=D + 8) == E_ALIAS


def test_noalloc_validation(lib):
    """rmsnorm_bwd_noalloc rejects bad arguments before any HIP call, rows
    wider than its 16 MiB scratch holds (4 Mi float32 columns) included."""
    f = lib.rmsnorm_bwd_noalloc
    A, B, C, D, E, G = (0x10000 * k for k in range(1, 7))
    assert f(A, B, C, D, E, None, 4, 64, BF16, BF16, None) == E_NULL
    assert f(None, B, C, D, E, G, 4, 64, BF16, BF16, None) == E_NULL
    assert f(A, B, None, D, E, G, 4, 64, BF16, BF16, None) == E_NULL
    assert f(A, B, C, None, E, G, 4, 64, BF16, BF16, None) == E_NULL
    assert f(A, B, C, D, E, G, 4, 64, 7, BF16, None) == E_DTYPE
    assert f(A, B, C, D, E, G, -1, 64, BF16, BF16, None) == E_SHAPE
    assert f(A, B, C, D, E, G, 4, 0, BF16, BF16, None) == E_SHAPE
    assert f(A, B, C, D, E, G, 1, (16 << 20) // 4 + 1, BF16, BF16, None) == E_SCRATCH
    assert f(A, B, C, D, E, G, 1, (16 << 20) // 4 + 8, F32, F32, None) == E_SCRATCH


def test_tuning_knobs(lib):
    """addrms_tune: set returns the previous value, a negative value only
    reads, an unknown knob is ADDRMS_ERR_KNOB; no HIP call."""
    f = lib.addrms_tune
    f.argtypes = [ctypes.c_int, ctypes.c_int]
    E_KNOB = -9
    assert f(10, 1) == E_KNOB and f(-1, 0) == E_KNOB
    for k in range(10):
        prev = f(k, -1)
        assert prev >= 0
        assert f(k, prev + 3) == prev
        assert f(k, -1) == prev + 3
        assert f(k, prev) == prev + 3
        assert f(k, -1) == prev
