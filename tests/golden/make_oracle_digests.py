"""Write tests/golden/oracle_digests.json: SHA-256 digests of the CPU
oracle's outputs on small seeded workloads.

Calls only ``oracle`` and ``workloads``.  The digests guard the oracle
against an unnoticed change of its arithmetic: after any deliberate change,
rerun this script and name the passage that justifies the change in the
commit message.

    python tests/golden/make_oracle_digests.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digests.json")

# (workload id, T, split)
CASES = [(1, 8, False), (2, 8, False), (3, 2, False), (4, 2, False), (5, 3, False),
         (5, 3, True), (2, 3, True), (6, 4, False)]


def run_case(cid, T, split):
    w = workloads.WORKLOADS[cid]
    inp = workloads.make_workload(cid, T)
    epi = oracle.EPI_SANDWICH if w.epilogue == "sandwich" else oracle.EPI_RMSNORM
    kw = dict(residual=workloads.bits(inp.residual), gamma1=workloads.f32(inp.gamma1),
              gamma2=workloads.f32(inp.gamma2) if inp.gamma2 is not None else None,
              eps=inp.eps, epilogue=epi, split=split)
    if w.ep:
        res = oracle.ep_boundary(
            [workloads.bits(e) for e in inp.expert_rows], topk_w=workloads.f32(inp.topk_w),
            topk_rows=[r.numpy() for r in inp.ep_rows], H=w.H,
            shared=[None if s is None else workloads.bits(s) for s in inp.shared], **kw)
        return _digest(res)
    if inp.k:
        kw.update(topk_w=workloads.f32(inp.topk_w),
                  topk_idx=inp.topk_idx.numpy(),
                  shared=[workloads.bits(s) for s in inp.shared] if inp.shared else None)
    res = oracle.boundary([workloads.bits(s) for s in inp.sources], **kw)
    return _digest(res)


def _digest(res):
    h = hashlib.sha256()
    h.update(res.y.tobytes())
    h.update(res.xout.tobytes())
    return h.hexdigest()


def digests():
    return {f"w{cid}_T{T}{'_split' if split else ''}": run_case(cid, T, split)
            for cid, T, split in CASES}


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(digests(), f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", OUT)
