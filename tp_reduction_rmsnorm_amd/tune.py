"""Measure launch shapes on the local GPU and write a launch table.

    python tp_reduction_rmsnorm_amd/tune.py --out frn_launch_table.txt \\
        [--shape H R k epilogue ...] [--tokens T ...] [--calls 20]

With ``--out tp_reduction_rmsnorm_amd/csrc/frn_tuned_mi355x.inc`` it writes
the table the library compiles in as its default tuned rules (rebuild to
use it); any other name gets the plain table text.

For every shape and token count, each launch choice that fits is forced
through ``set_launch_table`` -- the one-row kernel with 1, 2 or 4 vectors
per lane, and for calls without finalize the row-pipelined kernel with 1 or
2 (``p1``, ``p2``) -- and timed the way the pages time this
operation (vLLM PR #62366, kernel microbenchmark table): a HIP graph holding
``--calls`` calls, median of 5 replays after at least 100 ms of replays.
Each choice is timed twice, the choices in order and then in reverse
order, and the two medians are averaged, so that a drift over the run
favours none of them.  The hand-fitted rule's own choice is kept wherever
it is within 1% of the fastest (``TIE``), so that near-equal choices do not
flip the table from run to run.  Inputs rotate over up to 64 sets,
at least 1 GiB where that many sets reach it, so large calls are not served
from the Infinity Cache.  The fastest choice per T becomes a rule covering
the T range up to it; neighbouring ranges with the same choice merge.  Load
the table with ``FRN_LAUNCH_TABLE=<file>`` or ``set_launch_table(text)``.

Shapes with a finalize (k > 0, not ``sum``) are also timed at
``--split-tokens`` (T <= 256) with the split-row finalize forced (a
workspace and a ``split`` rule) against the one-row kernel (no workspace);
the winner per T becomes ``split`` / ``fused`` rules.  The vec rules of a
finalize shape describe the one-row kernel; the split-row finalize's two
kernels take fixed shapes (a wave per rank, then one workgroup per token).  An epilogue
named ``ep-rmsnorm`` or ``ep-sandwich`` tunes the expert-parallel finalize
(``ep_moe_finalize_reduce_norm``): each of the R ranks owns an equal share
of 4R experts (at least k), and each token picks k distinct ones at random.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import tp_reduction_rmsnorm_amd as frn  # noqa: E402

EPI = {"rmsnorm": frn.EPI_RMSNORM, "sandwich": frn.EPI_SANDWICH, "sum": frn.EPI_SUM,
       "ep-rmsnorm": frn.EPI_RMSNORM, "ep-sandwich": frn.EPI_SANDWICH}
DEFAULT_SHAPES = [(5120, 4, 0, "sandwich"), (8192, 8, 0, "sandwich"), (512, 2, 0, "rmsnorm"),
                  (6144, 8, 0, "rmsnorm"), (6144, 8, 10, "rmsnorm"), (7168, 2, 8, "rmsnorm"),
                  (7168, 2, 0, "rmsnorm"), (7168, 2, 8, "sum"), (6144, 8, 10, "ep-rmsnorm"),
                  # residual + RMSNorm without finalize at common hidden sizes and TP degrees
                  (4096, 2, 0, "rmsnorm"), (4096, 4, 0, "rmsnorm"), (4096, 8, 0, "rmsnorm"),
                  (5120, 2, 0, "rmsnorm"), (5120, 4, 0, "rmsnorm"), (5120, 8, 0, "rmsnorm"),
                  (7168, 4, 0, "rmsnorm"), (7168, 8, 0, "rmsnorm"),
                  (8192, 2, 0, "rmsnorm"), (8192, 4, 0, "rmsnorm"), (8192, 8, 0, "rmsnorm")]
DEFAULT_TOKENS = [1, 8, 64, 256, 512, 1024, 2048, 4096, 16384]
DEFAULT_SPLIT_TOKENS = [1, 8, 16, 32, 48, 64, 96, 128, 160, 192, 224, 256]


def _bf16(shape, dev, g):
    return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)


class Call:
    """Rotating input sets of one shape and the library call on them."""

    def __init__(self, H, R, k, epi, T, dev):
        g = torch.Generator(device=dev)
        g.manual_seed(H * 131 + R * 17 + k * 7 + T)
        self.ep = epi.startswith("ep-")
        per_set = T * H * 2 * ((k + 1 if self.ep else R * (k + 1 if k else 1)) + 3)
        n = max(1, min(64, -(-(1 << 30) // per_set)))
        self.H, self.R, self.k, self.epi, self.T = H, R, k, epi, T
        self.workspace = None
        self.sets = []
        for _ in range(n):
            d = dict(residual=_bf16((T, H), dev, g), g1=torch.rand(H, generator=g, device=dev) + 0.5,
                     g2=torch.rand(H, generator=g, device=dev) + 0.5,
                     out=torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                     rout=torch.empty(T, H, dtype=torch.bfloat16, device=dev))
            if self.ep:
                experts = max(4 * R, -(-k // R) * R)
                chosen = torch.rand((T, experts), generator=g, device=dev).topk(k, dim=1).indices
                owner = chosen // (experts // R)
                d["rows"], d["src"] = [], []
                for r in range(R):
                    own = owner == r
                    idx = torch.full((T, k), -1, dtype=torch.int32, device=dev)
                    idx[own] = torch.arange(int(own.sum()), dtype=torch.int32, device=dev)
                    d["rows"].append(idx)
                    d["src"].append(_bf16((max(1, int(own.sum())), H), dev, g))
                d["shared"] = [_bf16((T, H), dev, g) if r == 0 else None for r in range(R)]
                d["w"] = torch.softmax(torch.randn(T, k, generator=g, device=dev), -1)
            elif k:
                d["src"] = [_bf16((T * k, H), dev, g) for _ in range(R)]
                d["shared"] = [_bf16((T, H), dev, g) for _ in range(R)]
                d["w"] = torch.softmax(torch.randn(T, k, generator=g, device=dev), -1)
                d["idx"] = torch.randperm(T * k, generator=g, device=dev).to(torch.int32).reshape(T, k)
            else:
                d["src"] = [_bf16((T, H), dev, g) for _ in range(R)]
            self.sets.append(d)

    def __call__(self, i):
        d = self.sets[i % len(self.sets)]
        if self.ep:
            return frn.ep_moe_finalize_reduce_norm(d["src"], d["w"], d["rows"], d["residual"],
                                                   d["g1"], d["g2"], shared=d["shared"],
                                                   epilogue=EPI[self.epi], out=d["out"],
                                                   residual_out=d["rout"],
                                                   workspace=self.workspace)
        if self.epi == "sum":
            if self.k:
                return frn.moe_finalize_reduce_bf16(d["src"], d["w"], d["idx"], shared=d["shared"],
                                                    out=d["out"])
            return frn.reduce_bf16(d["src"], out=d["out"])
        if self.k:
            return frn.moe_finalize_reduce_norm(d["src"], d["w"], d["idx"], d["residual"], d["g1"],
                                                d["g2"], shared=d["shared"], epilogue=EPI[self.epi],
                                                out=d["out"], residual_out=d["rout"],
                                                workspace=self.workspace)
        if self.epi == "sandwich":
            return frn.reduce_sandwich_norm(d["src"], d["residual"], d["g1"], d["g2"],
                                            out=d["out"], residual_out=d["rout"])
        return frn.reduce_residual_rmsnorm(d["src"], d["residual"], d["g1"], out=d["out"],
                                           residual_out=d["rout"])


# Each graph is replayed for this long before it is timed: after idle time
# (input generation) MI355X runs the first ~10 ms of sustained traffic
# slow, which would penalise whichever choice is timed first.
SETTLE_S = 0.1


def graph_us(call: Call, calls: int) -> float:
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            call(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            call(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / calls)
    del g
    return sorted(ts)[2]


def fits(H, R, k, epi, T, choice):
    """Whether the rule value `choice` ('1', '2', '4', 'p1', 'p2') is what a
    call of these sizes takes once that rule is loaded (a rule that does
    not fit the call is skipped in favour of the built-in rule)."""
    ep = epi.startswith("ep-")
    vec = int(choice[-1])
    pipelined = not ep and frn.launch_pipelined(R, k, T, H, EPI[epi])
    return (frn.launch_shape(R, k, T, H, EPI[epi], ep=ep)[1] == vec and
            pipelined == choice.startswith("p"))


# A measured winner replaces the hand-fitted rule's choice only where it is
# faster by more than this: between near-equal choices the timing order of
# a run, not the kernels, would decide, and the table would change from run
# to run.
TIE = 0.01


def builtin_choice(H, R, k, epi, T):
    """The rule value the hand-fitted rule gives a call ('1', '2', '4', 'p1',
    'p2')."""
    ep = epi.startswith("ep-")
    frn.set_launch_table("* * * * 0 * builtin\n")
    try:
        vec = frn.launch_shape(R, k, T, H, EPI[epi], ep=ep)[1]
        pipe = not ep and frn.launch_pipelined(R, k, T, H, EPI[epi])
    finally:
        frn.set_launch_table(None)
    return ("p" if pipe else "") + str(vec)


def builtin_split(H, R, k, epi, T):
    """'split' or 'fused': the hand-fitted rule's choice for a finalize call."""
    frn.set_launch_table("* * * * 0 * builtin\n")
    try:
        return "split" if frn.split_rows(R, k, T, H, EPI[epi], ep=epi.startswith("ep-")) else "fused"
    finally:
        frn.set_launch_table(None)


def pick(times, default):
    """The fastest choice, unless `default` is within TIE of it."""
    best = min(times, key=times.get)
    if default in times and times[default] <= times[best] * (1 + TIE):
        return default
    return best


def tune_shape(H, R, k, epi, tokens, calls, dev, log=print):
    """[(T, best_choice, {choice: us})] for one shape; a choice is a rule
    value: '1', '2', '4' (one-row kernel) or 'p1', 'p2' (row-pipelined)."""
    rows = []
    for T in tokens:
        call = Call(H, R, k, epi, T, dev)
        choices = []
        for vec in ("1", "2", "4", "p1", "p2"):
            frn.set_launch_table(f"{H} {R} {k} {epi} {T} {T} {vec}")
            if fits(H, R, k, epi, T, vec):  # else the rule is skipped for this call
                choices.append(vec)
        # every choice timed twice, in order and then in reverse order, so
        # that a drift over the run favours none of them
        times = {vec: 0.0 for vec in choices}
        for vec in choices + choices[::-1]:
            frn.set_launch_table(f"{H} {R} {k} {epi} {T} {T} {vec}")
            times[vec] += graph_us(call, calls) / 2
        frn.set_launch_table(None)
        hand = builtin_choice(H, R, k, epi, T)
        best = pick(times, hand)
        rows.append((T, best, times))
        log(f"H={H} R={R} k={k} {epi} T={T}: " +
            ", ".join(f"vec {v}: {us:.2f} us" for v, us in sorted(times.items())) +
            f" -> {best} (hand-fitted rule: {hand})")
        del call
        torch.cuda.empty_cache()
    return rows


def tune_split(H, R, k, epi, tokens, calls, dev, log=print):
    """[(T, 'split' | 'fused', {choice: us})] for one finalize shape: the
    split-row finalize (forced by a rule, with a workspace) against the
    one-row kernel (no workspace)."""
    rows = []
    for T in tokens:
        call = Call(H, R, k, epi, T, dev)
        times = {"split": 0.0, "fused": 0.0}
        for choice in ("split", "fused", "fused", "split"):  # A, B, B, A
            try:
                if choice == "split":
                    frn.set_launch_table(f"{H} {R} {k} {epi} {T} {T} split")
                    call.workspace = "auto"
                else:
                    call.workspace = None
                times[choice] += graph_us(call, calls) / 2
            finally:
                frn.set_launch_table(None)
        best = pick(times, builtin_split(H, R, k, epi, T))
        rows.append((T, best, times))
        log(f"H={H} R={R} k={k} {epi} T={T}: split {times['split']:.2f} us, "
            f"fused {times['fused']:.2f} us -> {best}")
        del call
        torch.cuda.empty_cache()
    return rows


def rules_for(H, R, k, epi, rows, last="*"):
    """Merge per-T winners into 'H R k epilogue Tmin Tmax vec' lines; the
    last range ends at ``last``."""
    out = []
    lo = 0
    for i, (T, best, _) in enumerate(rows):
        hi = last if i == len(rows) - 1 else str(T)
        if out and out[-1][2] == best:
            out[-1][1] = hi
        else:
            out.append([lo, hi, best])
        lo = T + 1
    return [f"{H} {R} {k} {epi} {a} {b} {v}" for a, b, v in out]


INC_HEADER = """\
// frn_tuned_mi355x.inc -- the launch table measured on MI355X (gfx950, 256
// CUs) by tune.py, compiled into the library as its default tuned rules:
// they decide every shape they cover unless a caller's table
// (frn_set_launch_table, FRN_LAUNCH_TABLE) has a rule for it first.  Shapes
// they do not cover take the hand-fitted rule in frn_shapes.hip.  Written
// by `python tp_reduction_rmsnorm_amd/tune.py --out <this file>`; the text
// between the delimiters is the table format of frn_set_launch_table.
"""


def as_inc(text: str) -> str:
    """The table as the C++ raw string literal frn_shapes.hip includes."""
    return INC_HEADER + 'R"FRN_TABLE(\n' + text + ')FRN_TABLE"\n'


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", required=True)
    ap.add_argument("--shape", nargs=4, action="append", metavar=("H", "R", "k", "EPILOGUE"))
    ap.add_argument("--tokens", nargs="+", type=int, default=DEFAULT_TOKENS)
    ap.add_argument("--split-tokens", nargs="+", type=int, default=DEFAULT_SPLIT_TOKENS,
                    help="T values (<= 256) at which finalize shapes time the split-row "
                         "finalize against the one-row kernel")
    ap.add_argument("--calls", type=int, default=20)
    args = ap.parse_args()
    split_tokens = sorted(t for t in set(args.split_tokens) if 1 <= t <= 256)
    shapes = ([(int(h), int(r), int(k), e) for h, r, k, e in args.shape] if args.shape
              else DEFAULT_SHAPES)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    lines = ["# fused_reduce_norm launch table: H R k epilogue Tmin Tmax vec",
             f"# measured on a {props.gcnArchName.split(':')[0]} GPU with {props.multi_processor_count} CUs"
             f" with: python tp_reduction_rmsnorm_amd/tune.py {' '.join(sys.argv[1:])}",
             f"# graph replay of {args.calls} calls, median of 5 after 100 ms of replays;"
             " each choice timed twice (in order, then in reverse order), the two averaged;"
             " the hand-fitted choice kept where within 1% of the fastest."]
    for H, R, k, epi in shapes:
        rows = tune_shape(H, R, k, epi, sorted(set(args.tokens)), args.calls, dev)
        lines += rules_for(H, R, k, epi, rows)
        if k > 0 and epi != "sum" and split_tokens:
            rows = tune_split(H, R, k, epi, split_tokens, args.calls, dev)
            lines += rules_for(H, R, k, epi, rows, last="256")
    text = "\n".join(lines) + "\n"
    frn.set_launch_table(text)  # validates the table
    frn.set_launch_table(None)
    with open(args.out, "w") as f:
        f.write(as_inc(text) if args.out.endswith(".inc") else text)
    print(f"wrote {args.out}", flush=True)


if __name__ == "__main__":
    main()
