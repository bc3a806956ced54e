"""Machine-code checks of the built library (CPU only, no GPU).

The gfx950 code objects inside add_rmsnorm_amd/libaddrms.so (built here from
this repository's sources) are taken out of the library's offload bundles and
inspected with LLVM's readelf and objdump:

- no kernel uses scratch memory, spills registers or has a dynamic stack;
- the fused forward of the headline shape (bf16, 8 waves per row, 2 vectors
  per lane) streams rows with 128-bit non-temporal loads and stores and
  converts with the hardware bf16 instruction;
- the FP8 forward converts with the hardware E4M3 instruction;
- the RMSNorm + RoPE kernel for bf16 heads of 128 streams each lane's two
  vectors in and out with 128-bit non-temporal accesses;
- no kernel contains packed fp32 add/mul/fma (the build disables them) or a
  generic (flat) memory access.

The vectorisation success sign the CuTe DSL skill page gives in Workflow 1
(128-bit vector loads) is checked here on AMD code."""
import os
import re
import shutil
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "add_rmsnorm_amd", "libaddrms.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

HEADLINE = "_ZN6addrms14fwd_vec_kernelINS_6bf16_tES1_Li0ELb1ELi0ELi8ELi2EEEvNS_7FwdArgsE"
FP8_FUSED = "_ZN6addrms14fwd_vec_kernelINS_6bf16_tES1_Li0ELb1ELi1ELi8ELi2EEEvNS_7FwdArgsE"
MXFP4_FUSED = "_ZN6addrms14fwd_vec_kernelINS_6bf16_tES1_Li0ELb1ELi3ELi8ELi2EEEvNS_7FwdArgsE"
ROPE_D128 = "_ZN6addrms15rope_vec_kernelINS_6bf16_tES1_Li8ELb0ELi4EEEvNS_8RopeArgsE"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{path} not available")
    return path


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (python add_rmsnorm_amd/build.py)")
    d = tmp_path_factory.mktemp("isa")
    fat = d / "fatbin.bin"
    subprocess.run([_tool("llvm-objcopy"), "-O", "binary", "--only-section=.hip_fatbin", LIB,
                    str(fat)], check=True)
    data = fat.read_bytes()
    objs = []
    at = data.find(MAGIC)
    while at >= 0:
        (n,) = struct.unpack_from("<Q", data, at + len(MAGIC))
        p = at + len(MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tlen].decode()
            p += tlen
            if "amdgcn" in triple:
                assert triple.endswith("gfx950"), triple
                path = d / f"co{len(objs)}.elf"
                path.write_bytes(data[at + off:at + off + size])
                objs.append(path)
        at = data.find(MAGIC, at + 1)
    assert objs, "no gfx950 code object in the library"
    return objs


def _kernels(path):
    notes = subprocess.run([_tool("llvm-readelf"), "--notes", str(path)], check=True,
                           capture_output=True, text=True).stdout
    out = {}
    for block in re.split(r"\n  - \.", notes):
        m = re.search(r"\.name:\s+(\S+)", block)
        if not m or ".symbol:" not in block:
            continue

        def field(k):
            f = re.search(rf"\.{k}:\s+(\S+)", block)
            return f.group(1) if f else None

        out[m.group(1)] = {k: field(k) for k in ("private_segment_fixed_size", "vgpr_spill_count",
                                                 "sgpr_spill_count", "uses_dynamic_stack",
                                                 "vgpr_count")}
    return out


@pytest.fixture(scope="module")
def kernels(code_objects):
    allk = {}
    for co in code_objects:
        for name, meta in _kernels(co).items():
            allk[name] = (co, meta)
    return allk


def _disasm(co, symbol=None):
    cmd = [_tool("llvm-objdump"), "-d", str(co)]
    if symbol:
        cmd.insert(2, f"--disassemble-symbols={symbol}")
    return subprocess.run(cmd, check=True, capture_output=True, text=True).stdout


def test_every_kernel_is_present_and_free_of_scratch(kernels):
    names = list(kernels)
    # forward, backward and column-reduce kernels of every dtype combination
    assert sum("fwd_vec_kernel" in n for n in names) > 100
    assert sum("bwd_vec_kernel" in n for n in names) > 100
    assert any("dw_colreduce_vec_kernel" in n for n in names)
    assert HEADLINE in kernels and FP8_FUSED in kernels
    bad = [(n, m) for n, (_, m) in kernels.items()
           if m["private_segment_fixed_size"] != "0" or m["vgpr_spill_count"] != "0"
           or m["sgpr_spill_count"] != "0" or m["uses_dynamic_stack"] != "false"]
    assert not bad, f"{len(bad)} kernels use scratch or spill, e.g. {bad[:3]}"


def test_headline_kernel_streams_128_bit_non_temporal(kernels):
    co, meta = kernels[HEADLINE]
    asm = _disasm(co, HEADLINE)
    loads = re.findall(r"global_load_dwordx4 [^\n]*", asm)
    stores = re.findall(r"global_store_dwordx4 [^\n]*", asm)
    # x and r: two 16-byte vectors each per lane, non-temporal; w: default policy
    assert sum(l.split("//")[0].rstrip().endswith(" nt") for l in loads) >= 4, loads
    # residual_out and y: two vectors each, non-temporal
    assert len(stores) >= 4 and all(s.split("//")[0].rstrip().endswith(" nt") for s in stores), stores
    assert not re.search(r"global_load_(dword|dwordx2|short|ushort|ubyte|sbyte)\b", asm)
    # the only narrower store is the row's float32 rstd
    assert len(re.findall(r"global_store_(dword|dwordx2|short|byte)\b", asm)) <= 1
    assert "v_cvt_pk_bf16_f32" in asm
    assert "scratch_" not in asm
    assert int(meta["vgpr_count"]) <= 128   # at least 4 waves per SIMD


def test_fp8_kernel_uses_hardware_e4m3_conversion(kernels):
    co, _ = kernels[FP8_FUSED]
    asm = _disasm(co, FP8_FUSED)
    assert "v_cvt_pk_fp8_f32" in asm
    assert re.search(r"global_load_dwordx4 [^\n]* nt", asm)


def test_mxfp4_kernel_uses_hardware_e2m1_conversion(kernels):
    # four packed conversions per 16-byte vector (8 bf16 values), 2 vectors a lane
    co, _ = kernels[MXFP4_FUSED]
    asm = _disasm(co, MXFP4_FUSED)
    assert len(re.findall(r"v_cvt_scalef32_pk_fp4_f32", asm)) >= 8
    assert re.search(r"global_load_dwordx4 [^\n]* nt", asm)


def test_rope_kernel_streams_heads_non_temporal(kernels):
    # bf16 heads of 128, 8 lanes per head, 4 heads per group and step (the
    # default): two 16-byte vectors in and out per lane and head,
    # non-temporal; tables and weights with the default policy
    co, meta = kernels[ROPE_D128]
    asm = _disasm(co, ROPE_D128)
    loads = [l.split("//")[0].rstrip() for l in re.findall(r"global_load_dwordx4 [^\n]*", asm)]
    stores = [l.split("//")[0].rstrip() for l in re.findall(r"global_store_dwordx4 [^\n]*", asm)]
    assert sum(l.endswith(" nt") for l in loads) == 8, loads
    assert len(stores) == 8 and all(l.endswith(" nt") for l in stores), stores
    assert "v_cvt_pk_bf16_f32" in asm and "scratch_" not in asm
    assert int(meta["vgpr_count"]) <= 168   # at least 3 waves per SIMD


def test_no_packed_fp32_arithmetic_and_no_flat_memory_access(code_objects):
    if shutil.which(os.path.join(LLVM, "llvm-objdump")) is None:
        pytest.skip("llvm-objdump not available")
    for co in code_objects:
        asm = _disasm(co)
        hits = re.findall(r"v_pk_(?:add|mul|fma)_f32[^\n]*", asm)
        assert not hits, f"{co.name}: {hits[:3]}"
        # every buffer is global memory: generic (flat) accesses would mean
        # the compiler lost a pointer's address space
        flat = re.findall(r"flat_(?:load|store|atomic)[^\n]*", asm)
        assert not flat, f"{co.name}: {flat[:3]}"
