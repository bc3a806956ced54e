"""Build libaddrms.so for gfx950 with hipcc, in-tree.

    python add_rmsnorm_amd/build.py        (a script: it must not import the
                                            package, which loads the library)

Compiles csrc/tables.hip and csrc/rope.hip once per (row dtype, weight dtype)
combination and csrc/api.hip, in parallel, then links one shared library next
to this file.
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


def build(verbose: bool = False, extra_defines=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(os.path.join(CSRC, "tables.hip"), os.path.join(BUILD, f"tables_{c}.o"),
             (f"ADDRMS_COMBO={c}", *extra_defines)) for c in range(4)]
    jobs += [(os.path.join(CSRC, "rope.hip"), os.path.join(BUILD, f"rope_{c}.o"),
              (f"ADDRMS_COMBO={c}", *extra_defines)) for c in range(4)]
    jobs.append((os.path.join(CSRC, "api.hip"), os.path.join(BUILD, "api.o"),
                 tuple(extra_defines)))
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
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
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    defs = [a[2:] for a in sys.argv[1:] if a.startswith("-D")]
    build(verbose=True, extra_defines=defs)
