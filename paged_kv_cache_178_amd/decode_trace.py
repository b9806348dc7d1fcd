"""Phase timeline of the uniform-split decode, from the trace build.

Runs the batch-1 decode of the Llama-3.2-1B head shape (Hq 32, Hkv 8, d 64,
bf16, block size 16) through libnp_paged_trace.so, which stamps every
workgroup's phases with s_memrealtime (100 MHz), and prints where the time of
one launch goes: for each phase the median over launches of the median (and
of the latest) workgroup, in microseconds from the first workgroup's start,
and the same for the workgroup that merged the splits of each KV head (the
critical path). Every launch reads its own cold copy of the pool.

    python -m paged_kv_cache_178_amd.decode_trace --history 4096 --reps 40

The trace build waits for all outstanding memory operations at every stamp,
so its total is an upper bound of the product kernel's; the phase split is
what it is for.
"""

from __future__ import annotations

import argparse
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PHASES = ["start", "q/table/length arrived", "first K/V group arrived (wave 0)",
          "blocks computed (wave 0)", "workgroup merged, partial stores issued",
          "stores acknowledged", "ticket known", "split merge done", "end"]
WORDS = 32      # NP_TRACE_UNIFORM_WORDS
STAMPS = 9      # NP_TRACE_STAMPS


def parse_uniform(buf):
    """Records of one launch from the trace words (numpy int32 [wgs, 32]):
    a list of dicts for the workgroups that ran a split."""
    import numpy as np

    recs = []
    for w in buf:
        if (w[0] & 1) == 0 or w[8] == 0:
            continue
        lo = w[10:10 + 2 * STAMPS:2].astype(np.uint32).astype(np.uint64)
        hi = w[11:11 + 2 * STAMPS:2].astype(np.uint32).astype(np.uint64)
        recs.append(dict(flags=int(w[0]), where=int(w[1]), seq=int(w[2]), kvh=int(w[3]),
                         split=int(w[4]), b0=int(w[5]), b1=int(w[6]), ticket=int(w[7]),
                         splits=int(w[8]), t=(hi << np.uint64(32)) | lo))
    return recs


def summarize(launches):
    """Per-phase medians over launches (µs from each launch's first start)."""
    import numpy as np

    med, late, crit = [[] for _ in PHASES], [[] for _ in PHASES], [[] for _ in PHASES]
    for recs in launches:
        t0 = min(int(r["t"][0]) for r in recs)
        for i in range(STAMPS):
            xs = [(int(r["t"][i]) - t0) / 100.0 for r in recs if int(r["t"][i]) != 0]
            if xs:
                med[i].append(float(np.median(xs)))
                late[i].append(float(np.max(xs)))
        mergers = [r for r in recs if r["flags"] & 2]
        if mergers:
            for i in range(STAMPS):
                xs = [(int(r["t"][i]) - t0) / 100.0 for r in mergers if int(r["t"][i]) != 0]
                if xs:
                    crit[i].append(float(np.max(xs)))
    f = lambda v: float(np.median(v)) if v else math.nan
    return [(PHASES[i], f(med[i]), f(late[i]), f(crit[i])) for i in range(STAMPS)]


def xcc_map(recs):
    """{kv head: sorted XCC ids its splits ran on} for one launch."""
    m = {}
    for r in recs:
        m.setdefault(r["kvh"], set()).add(r["where"] >> 6)
    return {k: sorted(v) for k, v in sorted(m.items())}


def run(history: int, reps: int, pool_bytes: float = float(1 << 30), bps: int = 0):
    import numpy as np
    import torch

    from paged_kv_cache_178_amd import binding
    from paged_kv_cache_178_amd import workloads as wl

    lib = binding.trace_library()
    dev = torch.device("cuda:0")
    inp = wl.llama_decode(history)
    q = inp.q.to(dev)
    bt = inp.block_table.to(dev)
    lens = inp.context_lens.to(dev)
    per_copy = 2 * inp.k_pool.numel() * inp.k_pool.element_size()
    copies = max(1, math.ceil(pool_bytes / per_copy))
    kbig = inp.k_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
    vbig = inp.v_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
    out = torch.empty_like(q)
    desc = binding.make_desc(q, kbig[0], bt, out=out, scale=inp.scale)
    plan = binding.np_plan(desc, inp.context_lens.numpy(), None,
                           binding.PlanOpts(force_blocks_per_split=bps), lib=lib)
    ws = binding.workspace_for(plan, dev)
    grid, wg, comb = plan.launch_shape()
    n_wg = grid[0] * grid[1] * grid[2]
    trace = torch.zeros(n_wg * WORDS, dtype=torch.int32, device=dev)
    st = lib.np_debug_set_trace(trace.data_ptr(), trace.numel() * 4)
    if st:
        raise binding.NPError(st, "np_debug_set_trace")
    launches = []
    try:
        for r in range(reps + 2):
            trace.zero_()
            c = r % copies
            binding.np_paged_attention_decode(desc, plan, q, kbig[c], vbig[c], bt, lens, out, ws)
            torch.cuda.synchronize()
            if r >= 2:                                   # first two: code and TLB warm-up
                launches.append(parse_uniform(trace.view(n_wg, WORDS).cpu().numpy()))
    finally:
        lib.np_debug_set_trace(None, 0)
    return dict(history=history, grid=grid, bps=plan.blocks_per_split,
                splits=plan.max_splits, copies=copies, launches=launches,
                rows=summarize(launches), xcc=xcc_map(launches[-1]))


def report(res) -> str:
    lines = [f"decode trace: history {res['history']}, {res['splits']} splits of {res['bps']} "
             f"blocks, grid {list(res['grid'])}, {len(res['launches'])} launches on "
             f"{res['copies']} rotating pool copies",
             "", "| phase | median workgroup (µs) | latest workgroup (µs) | merging workgroup (µs) |",
             "|---|---|---|---|"]
    for name, a, b, c in res["rows"]:
        lines.append(f"| {name} | {a:.2f} | {b:.2f} | {c:.2f} |")
    lines.append("")
    lines.append("XCC of each KV head's splits (last launch): " +
                 ", ".join(f"{k}: {v}" for k, v in res["xcc"].items()))
    return "\n".join(lines)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--history", type=int, default=4096)
    ap.add_argument("--reps", type=int, default=40)
    ap.add_argument("--blocks-per-split", type=int, default=0)
    args = ap.parse_args(argv)
    res = run(args.history, args.reps, bps=args.blocks_per_split)
    print(report(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
