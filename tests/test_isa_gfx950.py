"""Checks on the gfx950 machine code of our own library (CPU only).

The code object is taken out of libfused_reduce_norm.so (the .hip_fatbin
section, unbundled for gfx950) and disassembled with llvm-objdump.  The
test asserts that the kernels

* never write through the scalar data cache (no scalar stores, scalar
  atomics or scalar-cache write-back): every store is a vector store;
* contain no packed FP32 arithmetic (the build disables it);
* never spill to scratch memory;
* narrow FP32 to BF16 with the hardware round-to-nearest-even conversion.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "libfused_reduce_norm.so")
LLVM = "/opt/rocm/llvm/bin"


@pytest.fixture(scope="module")
def mnemonics(tmp_path_factory):
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.hip_build_module().build()
    d = tmp_path_factory.mktemp("isa")
    fatbin, co = str(d / "fatbin.bin"), str(d / "gfx950.co")
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fatbin}", LIB,
                    str(d / "copy.so")], check=True)
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                    f"--input={fatbin}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    f"--output={co}"], check=True)
    dis = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", co],
                         capture_output=True, text=True, check=True).stdout
    ops = [m.group(1) for m in re.finditer(r"^\s+([a-z_0-9]+)\b", dis, re.M)]
    assert len(ops) > 1000, "disassembly looks empty"
    return ops


def test_no_scalar_cache_writes(mnemonics):
    bad = sorted({op for op in mnemonics
                  if op.startswith(("s_store", "s_buffer_store", "s_scratch_store",
                                    "s_atomic", "s_buffer_atomic", "s_dcache_wb"))})
    assert not bad, f"scalar-cache writes in the kernels: {bad}"


def test_no_packed_fp32(mnemonics):
    bad = sorted({op for op in mnemonics if op in ("v_pk_fma_f32", "v_pk_add_f32",
                                                     "v_pk_mul_f32")})
    assert not bad, f"packed FP32 instructions: {bad}"


def test_no_scratch_spills(mnemonics):
    bad = sorted({op for op in mnemonics if op.startswith("scratch_")})
    assert not bad, f"scratch accesses (register spills): {bad}"


def test_bf16_narrowing_uses_hardware_rne(mnemonics):
    assert "v_cvt_pk_bf16_f32" in set(mnemonics)
