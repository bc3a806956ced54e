"""Address and undefined-behaviour sanitizers on the CPU (no GPU).

- The oracle (plain C) built by gcc with -fsanitize=address,undefined runs the
  whole pin suite: no out-of-bounds access, use after free, signed overflow,
  misaligned access or other undefined behaviour on any pin's inputs.
- The library's host code (argument validation, variant choice, the C ABI in
  api.hip) built by hipcc with host-only sanitizers (each -fsanitize= behind
  -Xarch_host; the device code is built as usual) runs the host ABI tests,
  which call every entry point with valid and invalid arguments.
- Canaries: copies of both sources with one planted out-of-bounds access and
  one planted signed overflow must make the same runs fail with the
  sanitizer's report, which shows the sanitizers are live in these builds.
Every build goes to a temporary directory; nothing here touches a GPU."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "addrms_oracle.c")
API_SRC = os.path.join(ROOT, "add_rmsnorm_amd", "csrc", "api.hip")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
PINS = ["tests/test_oracle_bf16.py", "tests/test_oracle_fwd.py", "tests/test_oracle_bwd.py",
        "tests/test_oracle_layernorm.py", "tests/test_oracle_fp8.py", "tests/test_oracle_rope.py",
        "tests/test_oracle_mxfp4.py"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan_rt():
    return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()


def _clang_asan_rt():
    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not found:
        pytest.fail("clang's ASan runtime is not installed under /opt/rocm/llvm")
    return found[0]


def _plant(src: str, anchor: str, new: str) -> str:
    assert src.count(anchor) == 1, f"anchor {anchor!r} occurs {src.count(anchor)} times"
    return src.replace(anchor, new)


def _build_oracle(src_text: str, out: str) -> str:
    c = out[:-3] + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-fast-math", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-o", out, c, "-lm"])
    return out


def _kernel_objects():
    """The library's kernel objects (built without sanitizers), built first if
    absent."""
    objs = sorted(glob.glob(os.path.join(BUILD, "tables_*.o")) +
                  glob.glob(os.path.join(BUILD, "rope_*.o")))
    if len(objs) != 18:  # tables_c.o and rope_c.o for the 9 dtype combinations
        subprocess.check_call([sys.executable, os.path.join(ROOT, "add_rmsnorm_amd", "build.py")])
        objs = sorted(glob.glob(os.path.join(BUILD, "tables_*.o")) +
                      glob.glob(os.path.join(BUILD, "rope_*.o")))
    return objs


def _build_library(src_text: str, out: str) -> str:
    src = out[:-3] + ".hip"
    with open(src, "w") as f:
        f.write(src_text)
    obj = out[:-3] + ".o"
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           *host_san, "-Xarch_host", "-fno-sanitize-recover=all",
                           "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "add_rmsnorm_amd", "csrc"),
                           "-c", src, "-o", obj], stderr=subprocess.DEVNULL)
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san,
                           "-o", out, obj, *_kernel_objects()])
    return out


def _pytest(files, env_extra):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    # -s: a sanitizer report is written to the process's stderr as it aborts,
    # which pytest's own output capture would drop
    run = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                          *files], cwd=ROOT, env=env, capture_output=True, text=True)
    return run.returncode, run.stdout + run.stderr


@pytest.fixture(scope="module")
def work(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitizers"))


# ---- the oracle ------------------------------------------------------------------

ORACLE_OOB = ("        for (int64_t j = 0; j < N; j++) {\n"
              "            double h = load_elem(x, x_dt, i * N + j);\n"
              "            ss += h * h;\n")
ORACLE_OVERFLOW = ("    for (int64_t i = 0; i < M; i++) {\n"
                   "        double ss = 0.0;\n")


def _oracle_run(lib):
    return _pytest(PINS, {"LD_PRELOAD": _gcc_asan_rt(), "ADDRMS_ORACLE_LIB": lib})


def test_oracle_pins_under_asan_and_ubsan(work):
    src = open(ORACLE_SRC).read()
    code, out = _oracle_run(_build_oracle(src, os.path.join(work, "liboracle_san.so")))
    assert code == 0, out[-4000:]
    assert " passed" in out


def test_oracle_canaries_are_caught(work):
    src = open(ORACLE_SRC).read()
    # one element past each row: past the whole matrix on the last row
    oob = _plant(src, ORACLE_OOB, ORACLE_OOB.replace("j < N", "j <= N"))
    code, out = _oracle_run(_build_oracle(oob, os.path.join(work, "liboracle_oob.so")))
    assert code != 0 and "AddressSanitizer" in out, out[-4000:]
    ovf = _plant(src, ORACLE_OVERFLOW, "    { volatile int big = 2147483647; big = big + (M >= 0); }\n"
                 + ORACLE_OVERFLOW)
    code, out = _oracle_run(_build_oracle(ovf, os.path.join(work, "liboracle_ovf.so")))
    assert code != 0 and "runtime error" in out, out[-4000:]


# ---- the library's host code --------------------------------------------------------

API_WS = "size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N)\n{\n"
API_STATUS = "const char *addrms_status_str(int status)\n{\n"


def _library_run(lib):
    return _pytest(["tests/test_abi_host.py"],
                   {"LD_PRELOAD": _clang_asan_rt(), "ADDRMS_TEST_LIB": lib})


def test_library_host_code_under_asan_and_ubsan(work):
    src = open(API_SRC).read()
    code, out = _library_run(_build_library(src, os.path.join(work, "libaddrms_san.so")))
    assert code == 0, out[-4000:]
    assert " passed" in out


def test_library_canaries_are_caught(work):
    src = open(API_SRC).read()
    # one byte past a heap block (past what the bounds check of a fixed array
    # would see, so ASan's redzone catches it)
    oob = _plant(src, API_WS, API_WS + "    { char *p = new char[8]; volatile int i = 8; p[i] = 1; "
                 "delete[] p; }\n")
    code, out = _library_run(_build_library(oob, os.path.join(work, "libaddrms_oob.so")))
    assert code != 0 and "AddressSanitizer" in out, out[-4000:]
    ovf = _plant(src, API_STATUS, API_STATUS + "    { volatile int k = 2147483647; k = k + 1; }\n")
    code, out = _library_run(_build_library(ovf, os.path.join(work, "libaddrms_ovf.so")))
    assert code != 0 and "runtime error" in out, out[-4000:]
