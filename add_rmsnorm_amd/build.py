"""Build libaddrms.so for gfx950 with hipcc, in-tree.

    python add_rmsnorm_amd/build.py        (a script: it must not import the
                                            package, which loads the library)

Compiles csrc/tables.hip and csrc/rope.hip once per (row dtype, weight dtype)
combination and csrc/api.hip, in parallel, then links one shared library next
to this file.  The native Python binding of the latency-bound forwards
(csrc/binding.cpp, host C++ against torch's headers) is compiled in the same
pool and linked against that library as _native*.so.  The plain C client
that the GPU tests run (tests/c_client) is linked against it too.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libaddrms.so")
PROBE_LIB = os.path.join(PKG, "libaddrms_probe.so")

ARCH = os.environ.get("ADDRMS_OFFLOAD_ARCH", "gfx950")
NUM_COMBOS = 9  # (row dtype, weight dtype) pairs of float32, bfloat16, float16
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, obj: str, defines=()):
    cmd = [HIPCC, *CFLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _torch_paths():
    """Include and library directories of the installed torch, and the
    Python extension suffix, for the native binding."""
    import sysconfig
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        return None
    td = os.path.dirname(spec.origin)
    return (td, sysconfig.get_paths()["include"], sysconfig.get_config_var("EXT_SUFFIX"))


NATIVE_SRC = os.path.join(CSRC, "binding.cpp")


def _native_compile(obj: str):
    """Compile the native Python binding (binding.cpp) with the host C++
    compiler against torch's headers: no device code."""
    td, pyinc, _ = _torch_paths()
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", "-DUSE_ROCM",
           "-I", os.path.join(td, "include"),
           "-I", os.path.join(td, "include", "torch", "csrc", "api", "include"),
           "-I", pyinc, "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-c", NATIVE_SRC, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _native_link(obj: str) -> str:
    td, _, suffix = _torch_paths()
    out = os.path.join(PKG, "_native" + suffix)
    lib = os.path.join(td, "lib")
    tmp = out + ".tmp"
    cmd = ["g++", "-shared", "-fPIC", "-o", tmp, obj, "-L", lib, "-lc10", "-lc10_hip", "-ltorch",
           "-ltorch_cpu", "-ltorch_python", f"-Wl,-rpath,{lib}", "-L", PKG, "-l:libaddrms.so",
           "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "addrms_client.c")
CLIENT = os.path.join(ROOT, "tests", "c_client", "addrms_client")


def _client_build() -> str:
    """The plain C client of the library that the GPU tests run (host code
    against the HIP runtime and libaddrms.so, found by a relative rpath)."""
    tmp = CLIENT + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), CLIENT_SRC, "-o", tmp, "-L", PKG, "-l:libaddrms.so",
           "-Wl,-rpath,$ORIGIN/../../add_rmsnorm_amd", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CLIENT)
    return CLIENT


def build(verbose: bool = False, extra_defines=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    # one object per (row dtype, weight dtype) combination: 3 x 3
    jobs = [(os.path.join(CSRC, "tables.hip"), os.path.join(BUILD, f"tables_{c}.o"),
             (f"ADDRMS_COMBO={c}", *extra_defines)) for c in range(NUM_COMBOS)]
    jobs += [(os.path.join(CSRC, "rope.hip"), os.path.join(BUILD, f"rope_{c}.o"),
              (f"ADDRMS_COMBO={c}", *extra_defines)) for c in range(NUM_COMBOS)]
    jobs.append((os.path.join(CSRC, "api.hip"), os.path.join(BUILD, "api.o"),
                 tuple(extra_defines)))
    workers = min(len(jobs) + 1, max(1, min(16, os.cpu_count() or 1)))
    native_obj = os.path.join(BUILD, "binding.o")
    with cf.ThreadPoolExecutor(workers) as ex:
        native = ex.submit(_native_compile, native_obj) if _torch_paths() else None
        objs = list(ex.map(lambda j: _compile(*j), jobs))
        if native is not None:
            native.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if native is not None:
        _native_link(native_obj)
    if os.path.exists(CLIENT_SRC):
        _client_build()
    # the benchmark's stream-ceiling probe: a separate library, never linked
    # into libaddrms.so
    _compile(os.path.join(CSRC, "stream_probe.hip"), os.path.join(BUILD, "stream_probe.o"))
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           os.path.join(BUILD, "stream_probe.o")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {LIB}, {PROBE_LIB}" + (" and the native binding" if native else ""))
    return LIB


if __name__ == "__main__":
    defs = [a[2:] for a in sys.argv[1:] if a.startswith("-D")]
    build(verbose=True, extra_defines=defs)
