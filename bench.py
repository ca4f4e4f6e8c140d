"""Benchmark of the fused reduce + norm boundary on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--no-cpu]

One step is one call of the whole fused path on the headline workload: the
sandwich boundary (FP32 sum of R=4 BF16 partials -> RMSNorm(gamma1) ->
+residual -> RMSNorm(gamma2)) at H=5120, T=4096 tokens, inputs resident in
HBM.  Consecutive steps rotate over input/output sets totalling more than
1 GiB so that the 256 MB Infinity Cache cannot serve them.  The K timed
steps are captured in one HIP graph and replayed once between HIP events
(``--eager``: K calls through the Python binding instead); warm-up runs W
steps and at least 100 ms.

Printed: ONE JSON line with the contract fields plus
  * ``roofline``: the fused kernel's achieved algorithmic GB/s (bytes per
    launch / average launch time from HIP events on the launch stream)
    against MI355X's 8 TB/s HBM peak, and the HBM traffic measured with
    rocprofv3 counters when the stored counter summary was taken on the
    current kernel machine code;
  * ``sweep``: µs/call and GB/s over T = 1..4096 at H=5120 (R=4) and H=8192
    (R=8), each the median of 5 replays of a HIP graph holding 20 calls (the
    measuring method of the pages' microbenchmark table, vLLM PR #62366);
  * ``other_configs``: the other workloads at their gated sizes -- the tiny
    call at T=8, the MoE finalize at T=1, 8 and 64, the large-batch MoE call
    fused against the split path at T=4096, the expert-parallel finalize at
    T=8, 64, 1024 and 4096 -- and eager (not graph-captured) µs per call at T=1 and 8;
  * ``cpu_baseline``: the CPU oracle timed on every core of the host's
    affinity mask (and on one) on a bounded sample of the same workload,
    with the largest BF16 ulp distance between its rows and the GPU's timed
    outputs of those rows;
  * ``roofline.access_pattern``: the headline call's access pattern alone
    (bench_probe.hip: the same rows read and written, the same launch
    pattern, no arithmetic) on the same buffers, the practical ceiling of
    this access mix on this GPU, and the call's fraction of it.

The GPU runs one process on one device; ``--gpus N`` with N > 1 exits with a
message (the library runs on one GPU only).
"""
from __future__ import annotations

import argparse
import hashlib
import struct
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of peak) vs tokens T at H=5120/8192"
PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
HEADLINE = (2, 4096)       # sandwich H=5120 R=4, T=4096
SWEEP_T = (1, 8, 64, 256, 1024, 4096)
COLD_BYTES = 1 << 30       # rotate inputs over > 1 GiB where bandwidth is measured
INFINITY_CACHE_BYTES = 256 << 20  # MI355X's last-level cache
# Warm-up before every timed region lasts at least this long.  After idle
# time (input generation, another workload's set-up) MI355X runs the first
# ~10 ms of sustained memory traffic slow: the same graph of 20 sandwich
# calls (H=5120 R=4 T=4096) measured 53.7-54.6 us per call when timed first
# and 49.7-51.7 us once 200 ms of calls had run, whichever kernel went
# first.  Timing after a settled warm-up measures the kernel, not the ramp.
SETTLE_MS = 100.0


def hip_build_module():
    """tp_reduction_rmsnorm_amd/build.py loaded by path (importing it through
    the package would first load the library it builds)."""
    import importlib.util
    path = os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "build.py")
    spec = importlib.util.spec_from_file_location("frn_hip_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_MAX_SRC = 24  # kMaxSrc of bench_probe.hip
PROBE_LIB = os.path.join(ROOT, "bench_probe.so")


def build_probe() -> str:
    """Compile bench_probe.hip (the access pattern alone) with the library's
    code-generation flags."""
    import subprocess
    b = hip_build_module()
    tmp = PROBE_LIB + f".tmp{os.getpid()}"
    proc = subprocess.run([b.HIPCC, *b.CODEGEN_FLAGS, PROBE_SRC, "-o", tmp],
                          capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on bench_probe.hip:\n{proc.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def pattern_probe(dev, cid=2, Ts=(1024, 4096)):
    """A workload's access pattern alone (bench_probe.hip: the same rows read
    and written, the same lanes, no arithmetic, no row-wide sums), graph-timed
    beside the fused call.  Where the call takes the row-pipelined kernel, its
    pattern (one workgroup per CU walking the rows, the next row's loads before
    the current row's stores) is timed as well.  Reduction workloads: on the call's own rotating
    buffers.  Expert-parallel workload: its k routed rows, the shared row and
    the residual of each token read as k + 2 contiguous [T,H] streams of
    their own (the same bytes without the gather, indices or weights); TP
    finalize workloads the same way, R (k + 1) + 1 streams (at most
    PROBE_MAX_SRC)."""
    import ctypes
    import torch
    import tp_reduction_rmsnorm_amd as frn
    if not os.path.exists(PROBE_LIB):
        build_probe()
    lib = ctypes.CDLL(PROBE_LIB)
    lib.probe_rows_mode.restype = ctypes.c_int
    lib.probe_rows_mode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.probe_rows_pipelined.restype = ctypes.c_int
    lib.probe_rows_pipelined.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rows = []
    for T in Ts:
        r = Runner(cid, T, dev, cold=True)
        w = r.w
        arrays, keep = [], []
        if w.ep or w.k:
            # expert-parallel: k routed rows + the shared row + the residual;
            # TP finalize: R (k + shared) rows + the residual
            nsrc = w.k + 2 if w.ep else w.R * (w.k + (1 if w.shared else 0)) + 1
            if nsrc > PROBE_MAX_SRC:
                raise ValueError(f"the pattern probe reads at most {PROBE_MAX_SRC} rows per token")
            vec = frn.launch_shape(w.R, w.k, T, w.H, r.epi, ep=w.ep)[1]
            for o, ro in r.outs:
                bufs = [torch.empty(T, w.H, dtype=torch.bfloat16, device=dev) for _ in range(nsrc)]
                keep.append(bufs)
                arrays.append(((ctypes.c_void_p * nsrc)(*[b.data_ptr() for b in bufs]),
                               (ctypes.c_void_p * 2)(o.data_ptr(), ro.data_ptr())))
        else:
            nsrc = w.R + 1
            vec = frn.launch_shape(w.R, 0, T, w.H, r.epi)[1]
            for d, (o, ro) in zip(r.sets, r.outs):
                srcs = (ctypes.c_void_p * nsrc)(*[p.data_ptr() for p in d.partials],
                                                d.residual.data_ptr())
                arrays.append((srcs, (ctypes.c_void_p * 2)(o.data_ptr(), ro.data_ptr())))

        def probe(i, arrays=arrays, T=T, H=w.H, nsrc=nsrc, vec=vec, mode=0):
            srcs, dsts = arrays[i % len(arrays)]
            st = lib.probe_rows_mode(ctypes.cast(srcs, ctypes.c_void_p), nsrc,
                                     ctypes.cast(dsts, ctypes.c_void_p), 2, T, H, vec, mode,
                                     torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(f"probe_rows_mode failed ({st})")

        def probe_reads(i):
            probe(i, mode=1)

        def probe_writes(i):
            probe(i, mode=2)

        def probe_pipelined(i, arrays=arrays, T=T, H=w.H, nsrc=nsrc, vec=vec):
            srcs, dsts = arrays[i % len(arrays)]
            st = lib.probe_rows_pipelined(ctypes.cast(srcs, ctypes.c_void_p), nsrc,
                                          ctypes.cast(dsts, ctypes.c_void_p), 2, T, H, vec,
                                          min(T, cus), torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(f"probe_rows_pipelined failed ({st})")

        pipelined = not w.k and frn.launch_pipelined(w.R, 0, T, w.H, r.epi)
        kernel_us = r.graph_us()
        call = r.call
        r.call = probe
        probe_us = r.graph_us()
        r.call = probe_reads
        reads_us = r.graph_us()
        r.call = probe_writes
        writes_us = r.graph_us()
        pipe_us = None
        if pipelined:
            r.call = probe_pipelined
            pipe_us = r.graph_us()
        r.call = call
        pattern_bytes = T * w.H * 2 * (nsrc + 2)
        read_bytes, write_bytes = T * w.H * 2 * nsrc, T * w.H * 2 * 2
        rows.append(dict(workload=w.name, T=T, vectors_per_lane=vec, rows_read=nsrc,
                         kernel="rows_pipelined_kernel" if pipelined else "row_kernel",
                         kernel_us=round(kernel_us, 3), kernel_GBps=round(r.bytes / kernel_us / 1e3, 1),
                         pattern_us=round(probe_us, 3),
                         pattern_GBps=round(pattern_bytes / probe_us / 1e3, 1),
                         pattern_frac_of_peak=round(pattern_bytes / probe_us / 1e3 / PEAK_GBS, 4),
                         kernel_over_pattern=round(kernel_us / probe_us, 4),
                         reads_only_us=round(reads_us, 3),
                         reads_only_GBps=round(read_bytes / reads_us / 1e3, 1),
                         writes_only_us=round(writes_us, 3),
                         writes_only_GBps=round(write_bytes / writes_us / 1e3, 1),
                         reads_plus_writes_over_pattern=round((reads_us + writes_us) / probe_us,
                                                              4)))
        if pipelined:
            rows[-1].update(
                pipelined_pattern_us=round(pipe_us, 3),
                pipelined_pattern_frac_of_peak=round(pattern_bytes / pipe_us / 1e3 / PEAK_GBS, 4),
                kernel_over_pipelined_pattern=round(kernel_us / pipe_us, 4))
        print(json.dumps(dict(pattern_probe=rows[-1])), file=sys.stderr, flush=True)
        del r, keep, arrays
        torch.cuda.empty_cache()
    return rows


def _elf_sections(b: bytes) -> dict:
    """{name: bytes} of the sections of a 64-bit little-endian ELF image."""
    shoff, = struct.unpack_from("<Q", b, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQ", b, shoff + i * shentsize) for i in range(shnum)]
    strtab = hdrs[shstrndx][4]
    out = {}
    for name, typ, _flags, _addr, off, size in hdrs:
        n = b[strtab + name:b.index(b"\0", strtab + name)].decode()
        out[n] = b"" if typ == 8 else b[off:off + size]  # SHT_NOBITS holds no bytes
    return out


def kernel_code_digest(lib: str = None) -> str:
    """SHA-256 of the kernels' machine code: the gfx950 code object inside
    the built library (its .hip_fatbin section, a clang offload bundle),
    over the sections that hold the instructions, the kernel descriptors
    and the kernel metadata (.text, .rodata, .note).  Symbol-name tables are
    left out: they carry per-build identifiers.  Comments and documentation
    do not change it; any change to the generated code does, so counter data
    taken on other code is not reported."""
    lib = lib or os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "libfused_reduce_norm.so")
    fat = _elf_sections(open(lib, "rb").read())[".hip_fatbin"]
    if fat[:24] != b"__CLANG_OFFLOAD_BUNDLE__":
        raise RuntimeError("unexpected .hip_fatbin layout")
    n, = struct.unpack_from("<Q", fat, 24)
    p = 32
    for _ in range(n):
        off, size, tlen = struct.unpack_from("<QQQ", fat, p)
        triple = fat[p + 24:p + 24 + tlen].decode()
        p += 24 + tlen
        if triple.endswith("gfx950"):
            secs = _elf_sections(fat[off:off + size])
            h = hashlib.sha256()
            for name in (".text", ".rodata", ".note"):
                h.update(name.encode())
                h.update(secs[name])
            return h.hexdigest()
    raise RuntimeError("no gfx950 code object in the library")


def stored_traffic(workload: str, T: int, digest: str):
    """HBM bytes per launch from profiles/traffic_<workload>_T<T>.md, or None
    when the file is missing or was measured on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_T{T}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_code_sha256:\s*([0-9a-f]{64})", text)
    f = re.search(r"fetch_bytes_per_launch:\s*([0-9.eE+]+)", text)
    w = re.search(r"write_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m and f and w) or m.group(1) != digest:
        return None
    return float(f.group(1)) + float(w.group(1))


class Runner:
    """Rotating input/output sets of one workload and the fused call on them."""

    def __init__(self, cid, T, dev, cold=True, split=False, unfused=False):
        import torch
        import tp_reduction_rmsnorm_amd as frn
        import workloads
        self.frn, self.torch = frn, torch
        self.w = workloads.WORKLOADS[cid]
        self.T = T
        self.split = split
        self.unfused = unfused
        w = self.w
        self.bytes = workloads.algorithmic_bytes(w.R, T, w.H, epilogue=w.epilogue, k=w.k,
                                                 shared=w.shared, ep=w.ep)
        n = max(1, min(32, -(-COLD_BYTES // self.bytes))) if cold else 1
        # the inputs the graph's calls rotate over exceed the Infinity Cache
        self.cold = cold and n * self.bytes > INFINITY_CACHE_BYTES
        self.sets = [workloads.make_workload(cid, T, device=dev, salt=i) for i in range(n)]
        self.outs = [(torch.empty(T, w.H, dtype=torch.bfloat16, device=dev),
                      torch.empty(T, w.H, dtype=torch.bfloat16, device=dev)) for _ in range(n)]
        self.scratch = torch.empty(T, w.H, dtype=torch.bfloat16, device=dev) if split else None
        self.parts = ([torch.empty(T, w.H, dtype=torch.bfloat16, device=dev) for _ in range(w.R)]
                      if unfused else None)
        self.epi = frn.EPI_SANDWICH if w.epilogue == "sandwich" else frn.EPI_RMSNORM

    def call(self, i):
        d = self.sets[i % len(self.sets)]
        o, r = self.outs[i % len(self.outs)]
        f = self.frn
        if self.split:
            return f.split_reduce_norm(d.sources, d.residual, d.gamma1, d.gamma2, d.eps,
                                       topk_weights=d.topk_w if d.k else None,
                                       topk_rows=d.topk_idx if d.k else None,
                                       shared=d.shared if d.k else None, epilogue=self.epi,
                                       scratch=self.scratch, out=o, residual_out=r)
        if d.ep_rows is not None:
            return f.ep_moe_finalize_reduce_norm(d.expert_rows, d.topk_w, d.ep_rows, d.residual,
                                                 d.gamma1, d.gamma2, d.eps, shared=d.shared,
                                                 epilogue=self.epi, out=o, residual_out=r)
        if d.k and self.unfused:
            # the standalone finalize, then the plain reduction of its output
            f.moe_finalize(d.expert_rows, d.topk_w, d.topk_idx, shared=d.shared, out=self.parts)
            if self.epi == f.EPI_SANDWICH:
                return f.reduce_sandwich_norm(self.parts, d.residual, d.gamma1, d.gamma2, d.eps,
                                              out=o, residual_out=r)
            return f.reduce_residual_rmsnorm(self.parts, d.residual, d.gamma1, d.eps,
                                             out=o, residual_out=r)
        if d.k:
            return f.moe_finalize_reduce_norm(d.expert_rows, d.topk_w, d.topk_idx, d.residual,
                                              d.gamma1, d.gamma2, d.eps, shared=d.shared,
                                              epilogue=self.epi, out=o, residual_out=r)
        if self.epi == f.EPI_SANDWICH:
            return f.reduce_sandwich_norm(d.partials, d.residual, d.gamma1, d.gamma2, d.eps,
                                          out=o, residual_out=r)
        return f.reduce_residual_rmsnorm(d.partials, d.residual, d.gamma1, d.eps,
                                         out=o, residual_out=r)

    def graph_us(self, calls=20, replays=5, warm=3):
        """µs per call: a HIP graph of `calls` calls, median over replays."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(3):
                self.call(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                self.call(i)
        for _ in range(warm):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
            for _ in range(10):
                g.replay()
            torch.cuda.synchronize()
        ts = []
        for _ in range(replays):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / calls)
        del g
        return sorted(ts)[len(ts) // 2]


def sweep(dev, cids=(2, 3), Ts=SWEEP_T):
    rows = []
    for cid in cids:
        for T in Ts:
            r = Runner(cid, T, dev, cold=T >= 256)
            us = r.graph_us()
            gbs = r.bytes / us / 1e3
            rows.append(dict(workload=r.w.name, T=T, us_per_call=round(us, 3),
                             GBps=round(gbs, 1), frac_of_peak=round(gbs / PEAK_GBS, 4),
                             cold=r.cold))
            print(json.dumps(dict(sweep=rows[-1])), file=sys.stderr, flush=True)
            del r
    return rows


def extra_configs(dev, full=False):
    """The other workloads at their gated sizes: the tiny call at T=8, the
    MoE finalize at T=1, 8, 64, the expert-parallel finalize at T=8, 64,
    1024 and 4096, and
    the large-batch MoE call fused against the split path at T=4096
    (``full``: more T, and the MoE finalize fused against the standalone
    finalize followed by the plain reduction).  Where two paths compute the
    same call they share one set of inputs and are timed in the order A, B,
    B, A, each reported as the mean of its two medians, so that neither
    gains from running second."""
    rows = []

    def add(r, T, tag, us):
        rows.append(dict(workload=r.w.name + (f"_{tag}" if tag else ""), T=T,
                         us_per_call=round(us, 3), GBps=round(r.bytes / us / 1e3, 1),
                         frac_of_peak=round(r.bytes / us / 1e3 / PEAK_GBS, 4),
                         cold=r.cold))
        print(json.dumps(dict(extra=rows[-1])), file=sys.stderr, flush=True)

    def pair(r, attr):
        t = {False: [], True: []}
        for flag in (False, True, True, False):
            setattr(r, attr, flag)
            t[flag].append(r.graph_us())
        setattr(r, attr, False)
        return sum(t[False]) / 2, sum(t[True]) / 2

    if full:
        singles = ((1, (8,)), (4, (2, 4, 16, 32)), (6, (1, 8, 64, 1024, 4096)))
    else:
        singles = ((1, (8,)), (4, (1, 8, 64)), (6, (8, 64, 1024, 4096)))
    for cid, Ts in singles:
        for T in Ts:
            r = Runner(cid, T, dev, cold=T >= 256)
            add(r, T, "", r.graph_us())
            del r
    if full:
        for T in (1, 8, 64):
            r = Runner(4, T, dev, cold=False, unfused=True)
            fused, unfused = pair(r, "unfused")
            add(r, T, "", fused)
            add(r, T, "unfused", unfused)
            rows[-1]["unfused_over_fused"] = round(unfused / fused, 3)
            del r
    for T in ((4096, 16384) if full else (4096,)):
        r = Runner(5, T, dev, cold=True, split=True)
        fused, split = pair(r, "split")
        add(r, T, "", fused)
        add(r, T, "split", split)
        rows[-1]["split_over_fused"] = round(split / fused, 3)
        rows[-1].update(split_vs_fused_difference(r))
        del r
    return rows


def _ordered_device(t):
    """_ordered on the GPU: a BF16 tensor's bits as integers in the order of
    their values (+0 = -0), so that a difference of n is n ulps."""
    import torch
    b = t.contiguous().view(torch.int16).to(torch.int32)
    return torch.where(b < 0, -(b & 0x7FFF), b)


def split_vs_fused_difference(r):
    """The split path rounds the reduced sum to BF16 before the epilogue and
    the fused call does not, so their outputs may differ by design: reported,
    not gated.  Both are run once on the first input set; over out and
    residual_out, the largest difference in BF16 units in the last place
    and its 99.9th percentile (near zero, where the residual add cancels,
    a small difference in value spans many ulps), the largest difference in
    value, and the share of elements that differ."""
    import torch
    res = {}
    outs = []
    for split in (False, True):
        r.split = split
        r.call(0)
        torch.cuda.synchronize()
        o, ro = r.outs[0]
        outs.append((o.clone(), ro.clone()))
    r.split = False
    for name, a, b in (("out", outs[0][0], outs[1][0]), ("residual_out", outs[0][1], outs[1][1])):
        d = (_ordered_device(a) - _ordered_device(b)).abs().flatten()
        k = max(1, -(-999 * d.numel() // 1000))
        res[f"split_vs_fused_{name}"] = dict(
            max_ulp=int(d.max()), p999_ulp=int(d.kthvalue(k).values),
            differing=round(float((d > 0).float().mean()), 6),
            max_abs=float((a.float() - b.float()).abs().max()))
    return res


def eager_rows(dev, cases=((2, 1), (2, 8), (1, 8), (4, 1), (4, 8)), calls=1000):
    """µs per call of eager calls through the Python binding (no graph), the
    outputs given: the wall time of `calls` back-to-back calls, after a
    warm-up, divided by their number.  At these sizes the host's time per
    call, not the kernel, sets the rate."""
    import torch
    rows = []
    for cid, T in cases:
        r = Runner(cid, T, dev, cold=False)
        t_warm = time.perf_counter()
        while (time.perf_counter() - t_warm) * 1e3 < SETTLE_MS:
            for i in range(50):
                r.call(i)
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(calls):
            r.call(i)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / calls * 1e6
        rows.append(dict(workload=r.w.name, T=T, eager_us_per_call=round(us, 2)))
        print(json.dumps(dict(eager=rows[-1])), file=sys.stderr, flush=True)
        del r
    return rows


def _ordered(bits):
    """BF16 bit patterns -> integers in the order of their values (+0 = -0)."""
    import numpy as np
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(runner, seconds=10.0, single_seconds=5.0):
    """The CPU oracle, as it is, on a bounded sample of the timed workload:
    the first 256 token rows of its first input set, repeated for about
    `seconds` with one thread per core of the process's affinity mask and
    `single_seconds` on one.  The oracle's rows are also compared with the
    GPU's outputs of those rows from the timed calls (the last timed call on
    that set)."""
    import numpy as np
    import oracle
    import workloads
    d = runner.sets[0]
    rows = min(256, runner.T)
    w = runner.w
    args = [workloads.bits(p[:rows]) for p in d.partials]
    kw = dict(residual=workloads.bits(d.residual[:rows]), gamma1=workloads.f32(d.gamma1),
              gamma2=workloads.f32(d.gamma2), eps=d.eps,
              epilogue=oracle.EPI_SANDWICH if w.epilogue == "sandwich" else oracle.EPI_RMSNORM)
    cores = max(1, len(os.sched_getaffinity(0)))
    byts = workloads.algorithmic_bytes(w.R, rows, w.H, epilogue=w.epilogue)

    def rate(threads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            res = oracle.boundary(args, nthreads=threads, **kw)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return res, reps, el

    res, _, _ = rate(cores, 0.0)  # warm
    res, reps, el = rate(cores, seconds)
    _, reps1, el1 = rate(1, single_seconds)
    y_gpu, x_gpu = (workloads.bits(t[:rows]) for t in runner.outs[0])
    ulp = max(int(np.abs(_ordered(res.y) - _ordered(y_gpu)).max()),
              int(np.abs(_ordered(res.xout) - _ordered(x_gpu)).max()))
    return dict(value=round(byts * reps / el / 1e9, 3), unit="GB/s", cores=cores, kind="oracle",
                cpu=cpu_model(), affinity_cores=len(os.sched_getaffinity(0)),
                online_cpus=os.cpu_count(),
                sample=f"{rows} of {runner.T} token rows of {w.name} (R={w.R}, H={w.H}), "
                       f"{reps} repetitions in {el:.1f} s, {cores} threads; "
                       f"{el / reps * 1e6 / rows:.1f} us per row",
                single_thread=dict(value=round(byts * reps1 / el1 / 1e9, 3), unit="GB/s",
                                   sample=f"{reps1} repetitions in {el1:.1f} s"),
                parity=dict(rows=rows, max_ulp_vs_gpu=ulp))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--eager", action="store_true",
                    help="time the K steps as eager calls through the Python binding "
                         "instead of one HIP graph replay (host-bound when a call's "
                         "Python work outlasts the kernel)")
    ap.add_argument("--all", action="store_true",
                    help="more sizes of the other workloads, and the MoE finalize fused "
                         "against finalize-then-reduce")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the other workloads and the eager rows")
    ap.add_argument("--no-pattern", action="store_true",
                    help="skip the access-pattern reference of the headline call")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--workload", default=None,
                    help="time another workload than the headline one (by name; for "
                         "profiling runs -- the contract line is the default)")
    ap.add_argument("--tokens", type=int, default=None, help="T for --workload")
    ap.add_argument("--split", action="store_true", help="with --workload: the split path")
    ap.add_argument("--pattern-probe", action="store_true",
                    help="also time the access pattern alone (bench_probe.hip): the "
                         "headline workload at T=1024 and 4096, or --workload at its T")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    lib = os.path.join(ROOT, "tp_reduction_rmsnorm_amd", "libfused_reduce_norm.so")
    if not os.path.exists(lib):
        hip_build_module().build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cid, T = HEADLINE
    if args.workload is not None:
        import workloads
        byname = {w.name: c for c, w in workloads.WORKLOADS.items()}
        if args.workload not in byname:
            print(f"unknown workload {args.workload!r}; known: {sorted(byname)}", file=sys.stderr)
            sys.exit(2)
        cid = byname[args.workload]
        T = args.tokens or workloads.WORKLOADS[cid].tokens[-1]
    run = Runner(cid, T, dev, cold=True, split=args.split)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    warm_calls = 0
    if args.eager:
        # W warm-up steps, continued in batches of 50 until SETTLE_MS have passed
        t_warm = time.perf_counter()
        while True:
            n = 50 if warm_calls >= args.warmup else min(50, args.warmup - warm_calls)
            for _ in range(n):
                run.call(warm_calls)
                warm_calls += 1
            torch.cuda.synchronize()
            if warm_calls >= args.warmup and (time.perf_counter() - t_warm) * 1e3 >= SETTLE_MS:
                break
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(args.steps):
            run.call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # The K steps captured in one HIP graph (the pages time the operation
        # from graph replays): the Python binding's per-call host work stays
        # out of the timed region.
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(3):
                run.call(i)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                run.call(i)
        # W warm-up steps (whole replays of the K), continued until SETTLE_MS
        t_warm = time.perf_counter()
        while warm_calls < args.warmup or (time.perf_counter() - t_warm) * 1e3 < SETTLE_MS:
            graph.replay()
            warm_calls += args.steps
            torch.cuda.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ev_us = e0.elapsed_time(e1) * 1e3 / args.steps  # average launch duration, µs
    ms_per_step = wall * 1e3 / args.steps
    value = run.bytes / (ms_per_step * 1e-3) / 1e9
    achieved = run.bytes / (ev_us * 1e-6) / 1e9

    if args.copy_calibration:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    digest = kernel_code_digest()
    traffic = stored_traffic(run.w.name + ("_split" if args.split else ""), T, digest)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls_run": warm_calls,
        "launch": "eager" if args.eager else "hip_graph",
        "warmup_min_ms": SETTLE_MS,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "frac_of_peak": round(value / PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": run.w.name + ("_split" if args.split else ""), "T": T,
                   "H": run.w.H, "R": run.w.R, "k": run.w.k,
                   "epilogue": run.w.epilogue, "storage": "bf16",
                   "algorithmic_bytes_per_call": run.bytes,
                   "rotating_sets": len(run.sets), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic, "kernel_us": round(ev_us, 3),
                     "kernel_code_sha256": digest},
    }
    if not args.no_cpu and args.workload is None:
        out["cpu_baseline"] = cpu_baseline(run)
    del run
    torch.cuda.empty_cache()
    if args.workload is None and not args.no_pattern:
        # the access pattern alone on the same kind of buffers: the practical
        # ceiling of this read/write mix and launch pattern on this GPU
        pat = pattern_probe(dev, cid, (T,))[0]
        pat_us = pat.get("pipelined_pattern_us", pat["pattern_us"])
        pat_bytes = T * out["config"]["H"] * 2 * (out["config"]["R"] + 3)
        out["roofline"]["access_pattern"] = dict(
            kernel=pat["kernel"], pattern_us=pat_us,
            pattern_GBps=round(pat_bytes / pat_us / 1e3, 1),
            pattern_frac_of_peak=round(pat_bytes / pat_us / 1e3 / PEAK_GBS, 4),
            call_frac_of_pattern=round(pat_us / ev_us, 4),
            source="bench_probe.hip: the call's rows read and written with its launch "
                   "pattern, no arithmetic")
    if not args.no_sweep:
        out["sweep"] = sweep(dev)
    if not args.no_other and args.workload is None:
        out["other_configs"] = extra_configs(dev, full=args.all)
        out["eager"] = eager_rows(dev)
    if args.pattern_probe:
        out["pattern_probe"] = (pattern_probe(dev, cid, (T,)) if args.workload is not None
                                else pattern_probe(dev))
    if "cpu_baseline" in out:  # keep the contract's key order readable
        out["cpu_baseline"] = out.pop("cpu_baseline")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
