"""Checks on the gfx950 machine code of our own library (CPU only).

The code object is taken out of libfused_reduce_norm.so (the .hip_fatbin
section, unbundled for gfx950) and disassembled with llvm-objdump.  The
test asserts that the kernels

* never write through the scalar data cache (no scalar stores, scalar
  atomics or scalar-cache write-back): every store is a vector store;
* contain no packed FP32 arithmetic (the build disables it);
* never spill to scratch memory, and keep the register budgets their launch
  shapes were measured at;
* narrow FP32 to BF16 with the hardware round-to-nearest-even conversion.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "libfused_reduce_norm.so")
LLVM = "/opt/rocm/llvm/bin"


_DIS = {}


def _code_object(d):
    """Write the library's gfx950 code object into directory d; its path."""
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.hip_build_module().build()
    fatbin, co = os.path.join(d, "fatbin.bin"), os.path.join(d, "gfx950.co")
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fatbin}", LIB,
                    os.path.join(d, "copy.so")], check=True)
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                    f"--input={fatbin}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    f"--output={co}"], check=True)
    return co


def _vgpr_counts():
    """{kernel symbol: VGPRs per lane} from the code object's metadata (cached)."""
    if "vgprs" in _DIS:
        return _DIS["vgprs"]
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", _code_object(d)],
                               capture_output=True, text=True, check=True).stdout
    out = {}
    for block in notes.split("- .agpr_count")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        out[name] = int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1))
    _DIS["vgprs"] = out
    return out


def _disassembly():
    """llvm-objdump of the library's gfx950 code object (cached)."""
    if "text" in _DIS:
        return _DIS["text"]
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        co = _code_object(d)
        _DIS["text"] = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", co],
                                      capture_output=True, text=True, check=True).stdout
    return _DIS["text"]


@pytest.fixture(scope="module")
def mnemonics():
    ops = [m.group(1) for m in re.finditer(r"^\s+([a-z_0-9]+)\b", _disassembly(), re.M)]
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


def test_no_flat_memory_instructions(mnemonics):
    """Every memory access names its address space (global or LDS): a flat
    access would also count against the scalar-load counter, so waiting for
    a scalar load would wait for it too (the expert-parallel work list
    rebuilds row addresses from lanes and must cast them back to global)."""
    bad = sorted({op for op in mnemonics if op.startswith(("flat_load", "flat_store"))})
    assert not bad, f"flat memory instructions: {bad}"


def test_streamed_rows_use_non_temporal_accesses():
    """The streamed tensors are loaded and stored non-temporally (nt bit)."""
    dis = _disassembly()
    assert re.search(r"global_load_dwordx4 .* nt\b", dis), "no non-temporal row loads"
    assert re.search(r"global_store_dwordx4 .* nt\b", dis), "no non-temporal row stores"


def _function(dis, symbol):
    """The disassembly of one kernel (from its label to the next label)."""
    m = re.search(rf"^[0-9a-f]+ <{re.escape(symbol)}>:\n(.*?)(?=^[0-9a-f]+ <|\Z)", dis, re.M | re.S)
    assert m, f"{symbol} not found"
    return m.group(1)


def test_pipelined_kernel_keeps_the_next_row_in_flight():
    """rows_pipelined_kernel (sandwich, two vectors per lane, R = 4): the
    gamma rows go to LDS by direct global->LDS loads; the only full wait on
    the vector memory counter is the one before the first barrier (those
    copies must have landed); in the row loop the partials are consumed
    with the row's four output stores still in flight (vmcnt(4)), so no
    wait covers the stores, and the epilogue never waits on the next row's
    loads (no lane predicate hides a memory access from the count)."""
    f = _function(_disassembly(), "_ZN3frn12_GLOBAL__N_121rows_pipelined_kernelILi1ELi2ELi4EEEvNS_7RowArgsE")
    assert "global_load_lds_dwordx4" in f
    assert len(re.findall(r"s_waitcnt vmcnt\(0\)", f)) == 1
    assert re.search(r"s_waitcnt vmcnt\(4\)", f)
    first_barrier = f.index("s_barrier")
    assert f.index("vmcnt(0)") < first_barrier


def _pipelined_instances():
    """(epilogue, vectors per lane, ranks) of every rows_pipelined_kernel."""
    return [(e, v, r) for e in (0, 1) for v in (1, 2) for r in (1, 2, 3, 4)]


def _pipelined_symbol(e, v, r):
    return f"_ZN3frn12_GLOBAL__N_121rows_pipelined_kernelILi{e}ELi{v}ELi{r}EEEvNS_7RowArgsE"


@pytest.mark.parametrize("epi,vec,ranks", _pipelined_instances())
def test_pipelined_row_sums_alternate_slot_arrays(epi, vec, ranks):
    """A row sum writes one FP64 per wave into an LDS slot array, then one
    barrier, then every lane reads all of them; nothing follows the reads.
    So the next write into the same array must sit behind another barrier,
    or a fast wave could overwrite a slot a slow wave has not read yet.  In
    the row loop the slot writes (ds_write_b64 at offset 0 = slots[0] and
    128 = slots[1]) alternate between the two arrays, each followed by a
    barrier before the next write: two per loop, for the sandwich (two sums
    per row) and for residual + RMSNorm (one sum per row, rows unrolled by
    two)."""
    f = _function(_disassembly(), _pipelined_symbol(epi, vec, ranks))
    events = [m.group(0) for m in re.finditer(
        r"s_barrier|ds_write_b64 v\d+, v\[\d+:\d+\]( offset:\d+)?", f)]
    writes = [e for e in events if e.startswith("ds_write_b64")]
    offsets = [int(e.split("offset:")[1]) if "offset:" in e else 0 for e in writes]
    assert offsets == [0, 128], f"slot writes at offsets {offsets}"
    # every slot write is followed by a barrier before the next slot write
    seq = ["W" if e.startswith("ds_write") else "B" for e in events]
    first = seq.index("W")
    assert seq[first:] == ["W", "B", "W", "B"], seq


@pytest.mark.parametrize("epi,vec,ranks", _pipelined_instances())
def test_pipelined_loop_never_waits_for_everything(epi, vec, ranks):
    """One full wait on the vector memory counter (the gamma copies before
    the first barrier); every other wait leaves the row's 2 x vec output
    stores in flight, so none of them waits for the stores."""
    f = _function(_disassembly(), _pipelined_symbol(epi, vec, ranks))
    waits = [int(n) for n in re.findall(r"s_waitcnt vmcnt\((\d+)\)", f)]
    assert waits.count(0) == 1, waits
    assert f.index("vmcnt(0)") < f.index("s_barrier")
    assert min(w for w in waits if w) >= 2 * vec, waits



def _split_row_symbols(dis):
    return sorted(set(re.findall(r"<(_ZN3frn12_GLOBAL__N_126finalize_sum_slices_kernel\w+)>:", dis)))


def test_split_row_first_kernel_one_barrier_and_no_flat_rank_selection():
    """finalize_sum_slices_kernel (every instance): one barrier, after which
    wave 0 reads the R parked partials; the wave's rank is a scalar
    (readfirstlane), so the per-rank kernel arguments are picked with
    scalar loads, never with a per-lane index."""
    dis = _disassembly()
    syms = _split_row_symbols(dis)
    assert len(syms) == 16, syms
    for sym in syms:
        f = _function(dis, sym)
        assert f.count("s_barrier") == 1, sym
        assert "v_readfirstlane_b32" in f, sym
        assert "scratch_" not in f, sym


def test_sliced_epilogue_loads_the_slice_sums_in_one_round_trip():
    """norm_slices_kernel: the S slice sums of squares come in as one vector
    load (lane q takes sum q), not as S dependent scalar loads, and the
    kernel waits on the vector memory counter once before the rows' norm."""
    f = _function(_disassembly(), "_ZN3frn12_GLOBAL__N_118norm_slices_kernelENS_7RowArgsEi")
    assert len(re.findall(r"global_load_dwordx2 ", f)) == 1
    assert len(re.findall(r"s_waitcnt vmcnt\(0\)", f)) == 1
    loop = f[f.index("vmcnt(0)"):]
    assert "v_readlane_b32" in loop
    assert not re.search(r"s_load_dwordx2 s\[\d+:\d+\], s\[\d+:\d+\], 0x0\b", loop)


def _row_kernel_symbols(dis):
    """{(epilogue, finalize, vectors per lane, chunk): symbol} of every row_kernel."""
    out = {}
    for m in re.finditer(r"<(_ZN3frn12_GLOBAL__N_110row_kernelILi(\d)ELi(\d)ELi(\d)ELi(\d+)EEEvNS_7RowArgsE)>:", dis):
        out[tuple(int(g) for g in m.groups()[1:])] = m.group(1)
    return out


def test_row_kernel_epilogue_loads_nothing_after_its_first_store():
    """row_kernel with two or four vectors per lane and a norm epilogue: no
    vector load follows the first store.  A wave's vector memory operations
    complete in issue order, so a gamma load behind a store would also wait
    for the store; every gamma load goes out before the last row sum and
    both outputs are stored after it.  With one vector per lane the last
    gamma load does follow the residual_out store (one such wait, measured
    faster there), and that layout is checked too."""
    dis = _disassembly()
    syms = _row_kernel_symbols(dis)
    multi = {k: v for k, v in syms.items() if k[0] in (0, 1) and k[2] >= 2}
    assert len(multi) >= 12, sorted(syms)
    for key, sym in multi.items():
        f = _function(dis, sym)
        first_store = f.index("global_store")
        assert not re.search(r"\b(global|buffer)_load", f[first_store:]), (key, sym)
    one = {k: v for k, v in syms.items() if k[0] in (0, 1) and k[2] == 1}
    assert one
    for key, sym in one.items():
        f = _function(dis, sym)
        after = f[f.index("global_store"):]
        assert re.search(r"\bglobal_load_dwordx4\b", after), (key, sym)


# Register budgets the launch shapes were measured at: a SIMD holds
# floor(512 / VGPRs) waves (VGPRs allocated in steps of 8), and a CU four
# SIMDs.  (kernel symbol pattern, most VGPRs, why)
OCCUPANCY = [
    (r"row_kernelILi[01]ELi2ELi1ELi5E", 64,
     "expert-parallel work list: 8 waves per SIMD (two 768-lane or four 512-lane tokens per CU)"),
    (r"row_kernelILi[01]ELi1ELi1ELi8E", 72,
     "TP finalize, k <= 8: 7 waves per SIMD (two 896-lane tokens per CU at H=7168)"),
    (r"finalize_sum_slices_kernelILi[01]ELb1ELi12E", 80,
     "split-row finalize, k <= 12: 6 waves per SIMD (three 8-wave workgroups per CU at R=8)"),
    (r"rows_pipelined_kernelILi1ELi2ELi4E", 128,
     "headline kernel: one 320-lane workgroup per CU needs 2 waves per SIMD"),
    (r"norm_slices_kernel", 64, "sliced epilogue: one wave per workgroup, 8 per SIMD"),
]


@pytest.mark.parametrize("pattern,limit,why", OCCUPANCY, ids=[o[0] for o in OCCUPANCY])
def test_measured_kernels_keep_their_register_budget(pattern, limit, why):
    hits = {k: v for k, v in _vgpr_counts().items() if re.search(pattern, k)}
    assert hits, f"no kernel matches {pattern}"
    over = {k: v for k, v in hits.items() if v > limit}
    assert not over, f"{why}: {over} exceed {limit} VGPRs"
