"""The plain C client's own input handling, on the CPU: it rejects a missing
argument, a missing file, a bad header and a short file before any HIP call.
Its --plan mode (no HIP call) prints addrms_plan's answers through the C
header's struct, which must agree with the Python binding's.  Its GPU run is
tests/test_gpu_c_client.py."""
import os
import subprocess

import numpy as np

import add_rmsnorm_amd as ar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "addrms_client")


def _run(*args):
    assert os.path.exists(CLIENT), f"{CLIENT} is not built; run python add_rmsnorm_amd/build.py"
    return subprocess.run([CLIENT, *args], capture_output=True, text=True, timeout=60)


def test_client_rejects_bad_input(tmp_path):
    r = _run()
    assert r.returncode == 1 and "usage" in r.stderr
    r = _run(str(tmp_path / "missing.bin"), str(tmp_path / "out.bin"))
    assert r.returncode == 1 and "cannot open" in r.stderr
    bad = tmp_path / "bad.bin"
    bad.write_bytes(np.array([0, 8], dtype="<i8").tobytes())
    r = _run(str(bad), str(tmp_path / "out.bin"))
    assert r.returncode == 1 and "bad header" in r.stderr
    short = tmp_path / "short.bin"
    short.write_bytes(np.array([2, 8], dtype="<i8").tobytes() + bytes(10))
    r = _run(str(short), str(tmp_path / "out.bin"))
    assert r.returncode == 1 and "short file" in r.stderr
    assert not (tmp_path / "out.bin").exists()


def test_client_prints_the_launch_plans():
    for M, N in ((16384, 7168), (32768, 4096), (1, 8192), (300, 7170)):
        r = _run("--plan", str(M), str(N))
        assert r.returncode == 0, r.stderr
        lines = r.stdout.split("\n")
        for line, (op, fused) in zip(lines, (("fwd", True), ("bwd", False))):
            name, *fields = line.split()
            got = {k: int(v) for k, v in (f.split("=") for f in fields)}
            assert got == ar.plan(op, M, N, fused=fused), (M, N, name)
    r = _run("--plan", "0", "4096")
    assert r.returncode == 1 and "plan" in r.stderr
    r = _run("--plan", "16x", "4096")
    assert r.returncode == 1 and "bad M" in r.stderr
