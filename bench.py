#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

Workload: Llama-3.2-1B head shape (Hq=32, Hkv=8, d=64), block size 16, one
sequence with a 4096-token history, one query token, bf16 inputs with fp32
accumulation, one layer's cache (8 MiB of K+V), seeded N(0,1) data in blocks
scattered over a pool twice the size the history needs.

A step is one decode call through the C ABI: the split-KV decode kernel with
its in-launch split merge, on a plan and workspace prepared once (the plan
stays valid while the lengths keep the same split layout). The timed region
replays a HIP graph of K steps; step i reads copy i mod 64 of the pool (1 GiB
of copies), and a 512 MiB read of an unrelated buffer runs between the
untimed warm-up replay and the timed one. So every timed step reads K/V that
at least 504 MiB of other reads have passed through since it was last
touched, twice the 256 MiB Infinity Cache: cold HBM at any K.

Printed: one JSON line with KV GB/s (whole job), microseconds per step, the
decode kernel's roofline against 8 TB/s HBM and the float64 oracle's
throughput on this host's cores. Before any timing the GPU output is checked
against the oracle (atol = rtol = 1e-2). The same line carries, under
"secondary", the continuous-batching decode and the chunked prefill below,
each measured by a child run of this script with its default steps and
warmup (--no-secondary leaves them out).

Other workloads (not the headline, one JSON line each):
  --workload batching  64 sequences, lengths uniform on [128, 8192], Llama head
                       shape, 40000-block pool; KV GB/s against 8 TB/s.
  --workload prefill   4 sequences x (2048 cached + 512 new rows), causal, Llama
                       head shape; TFLOP/s of the exact causal FLOP count
                       against the 2.5 PFLOP/s dense bf16 MFMA peak.
  --workload read-ceiling
                       the single-launch ceiling of a plain read of the
                       headline's 8 MiB: the stream-read probe over 256 ..
                       2048 workgroups of 256 threads (and 512 and 1024
                       threads at 256 workgroups) with 1 .. 16 loads of 16 B
                       in flight per thread, graph-timed on cold copies.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-decode KV GB/s (% HBM peak) and µs/step, Llama-3.2-1B shape @4K history"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "paged_decode_llama_L4096_pmc.md")
PMC_SUMMARY_BATCHING = os.path.join(ROOT, "profiles", "paged_decode_batching_64seq_pmc.md")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_178_amd", "csrc", "np_decode.hip")
HOST_SRC = os.path.join(ROOT, "paged_kv_cache_178_amd", "csrc", "np_host.cpp")
PREFILL_SRC = os.path.join(ROOT, "paged_kv_cache_178_amd", "csrc", "np_prefill.hip")
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "paged_prefill_chunked_4x2560_counters.md")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Digest of the decode kernels' source and of the planner that shapes
    their launches: a counter summary taken on other sources is stale."""
    h = hashlib.sha256()
    for path in (DECODE_SRC, HOST_SRC):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_source_sha() -> str:
    """Digest of the prefill kernel's source and of the planner."""
    h = hashlib.sha256()
    for path in (PREFILL_SRC, HOST_SRC):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_mfma_busy(path=PREFILL_COUNTERS):
    """Fraction of SIMD cycles the matrix cores were busy during the chunked
    prefill, from the committed counter summary, if it was taken on the
    current prefill source; else None."""
    if not os.path.exists(path):
        return None
    m = re.search(r"^counters-json: (\{.*\})\s*$", open(path).read(), re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_sha") != prefill_source_sha():
        return None
    return rec.get("mfma_busy_frac")


def stored_traffic(path=PMC_SUMMARY):
    """HBM bytes per launch from a committed counter summary, if it was
    taken on the current decode kernel source; else None."""
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic-json: (\{.*\})\s*$", open(path).read(), re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_sha") != kernel_source_sha():
        return None
    return rec


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=("decode", "batching", "tiny", "awkward", "prefill",
                                           "append", "splitkv", "fused-prefill",
                                           "read-ceiling"),
                    default="decode")
    ap.add_argument("--history", type=int, default=4096)
    ap.add_argument("--pool-bytes", type=float, default=float(1 << 30),
                    help="total bytes of rotated pool copies (cold-cache measurement)")
    ap.add_argument("--warm", action="store_true",
                    help="one pool copy only (reported as MALL-warm, not the headline)")
    ap.add_argument("--combine-mode", type=int, default=0)
    ap.add_argument("--blocks-per-split", type=int, default=0)
    ap.add_argument("--wgs-per-cu", type=int, default=0)
    ap.add_argument("--schedule", type=int, default=0,
                    help="decode schedule: 0 auto, 1 uniform splits, 2 stream-K")
    ap.add_argument("--segment-cost", type=int, default=0,
                    help="stream-K: fixed cost of a (sequence, KV head) in blocks (0: default)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="headline only: skip the batching and prefill child runs")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="short run for hardware counters: a few decode steps and a plain "
                         "256 MiB copy, no timing")
    return ap.parse_args(argv)


def host_cores():
    """(cores this process may run on, cores of the machine)."""
    return len(os.sched_getaffinity(0)), os.cpu_count()


def time_runs(fn, seconds: float, clock=time.perf_counter, min_runs: int = 3):
    """Call fn until `seconds` of clock time have passed (at least min_runs
    calls); returns the duration of each call."""
    times = []
    t_end = clock() + seconds
    while clock() < t_end or len(times) < min_runs:
        t0 = clock()
        fn()
        times.append(clock() - t0)
    return times


def run_stats(times):
    """Best-of is the headline; median and mean show the spread."""
    xs = sorted(times)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"best": xs[0], "median": med, "mean": sum(xs) / n, "runs": n}


def per_step_us(elapsed_ms: float, steps: int) -> float:
    """Microseconds per step from an event interval (ms) around `steps` steps."""
    return elapsed_ms * 1e3 / steps


def rate(units: float, us: float, scale: float = 1e9) -> float:
    """units per second / scale (GB/s for bytes with scale 1e9) from µs."""
    return units / (us * 1e-6) / scale


def cpu_baseline(inp, seconds: float, seqs=None, prefill=False, threads=None):
    """Time the float64 oracle (gather, then dense softmax attention) on the
    same workload, or on the sequences `seqs` of it; best-of, the inputs
    already converted to float64, BLAS on `threads` threads (default: every
    core this process may use). Returns seconds per call, a description and
    the thread count."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    q = inp.q.double().numpy()
    k = inp.k_pool.double().numpy()
    v = inp.v_pool.double().numpy()
    bt = inp.block_table.numpy().astype(np.int64)
    lens = inp.context_lens.numpy().astype(np.int64)
    qs = inp.q_start.numpy().astype(np.int64)
    if seqs is not None:
        rows = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in seqs])
        n_q = np.array([qs[s + 1] - qs[s] for s in seqs])
        q = q[rows]
        bt = bt[list(seqs)]
        lens = lens[list(seqs)]
        qs = np.concatenate([[0], np.cumsum(n_q)])
    if threads is None:
        threads = host_cores()[0]
    with threadpool_limits(limits=threads):
        times = time_runs(lambda: oracle.paged_attention(
            q, k, v, bt, lens, q_start=qs if prefill else None, scale=inp.scale), seconds)
    st = run_stats(times)
    what = "full workload" if seqs is None else f"sequences {list(seqs)} of the workload"
    desc = (f"{what}, float64 numpy, {threads} BLAS thread{'s' if threads > 1 else ''}, "
            f"best of {st['runs']} runs (median {st['median'] * 1e3:.2f} ms) in "
            f"{sum(times):.1f} s")
    return st["best"], desc, threads


def cpu_record(value, unit, desc, threads, **extra):
    """The cpu_baseline object: `cores` is the BLAS thread count used."""
    avail, total = host_cores()
    rec = {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "sample": desc,
           "cores_available": avail, "cpu_count": total}
    rec.update(extra)
    return rec


_FLUSH = {}


def cache_flush() -> None:
    """Read 512 MiB of an unrelated buffer (twice the Infinity Cache, far more
    than the L2s), so nothing a timed replay reads is still cached."""
    import torch

    from paged_kv_cache_178_amd import binding

    dev = torch.cuda.current_device()
    if dev not in _FLUSH:
        _FLUSH[dev] = (torch.ones(512 << 20, dtype=torch.uint8, device=dev),
                       torch.empty(2048 * 256, dtype=torch.int32, device=dev))
    src, sink = _FLUSH[dev]
    binding.np_probe_stream_read(src, 2048, sink)


def graph_us(fn, n: int) -> float:
    """Average device time per call of n calls captured in one HIP graph: one
    untimed replay, a 512 MiB cache flush, then the timed replay.

    The timed replay is enqueued while the flush still runs, so its first
    kernel starts as soon as the flush ends: the host's submission of the
    graph (tens of microseconds, paid once per replay however many steps it
    holds) is not inside the interval, and the time per step does not depend
    on n."""
    import torch

    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    cache_flush()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    b.record()
    torch.cuda.synchronize()
    return per_step_us(a.elapsed_time(b), n)

def event_us(fn, n: int):
    """Mean of per-call event intervals around n eager calls."""
    import numpy as np
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for i in range(n):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    t = np.array([x.elapsed_time(y) * 1e3 for x, y in evs])
    return float(t.mean()), t


def causal_flops(inp) -> int:
    """QK^T and PV multiply-adds of causal attention, 2 flops each."""
    lens = inp.context_lens.tolist()
    qs = inp.q_start.tolist()
    total = 0
    for s, length in enumerate(lens):
        n_q = qs[s + 1] - qs[s]
        past = length - n_q
        keys = n_q * (past + 1) + n_q * (n_q - 1) // 2
        total += 4 * inp.head_dim * keys * inp.num_q_heads
    return total


def main(argv=None) -> int:
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU leg "
              "(decode shards by sequence or KV head with no exchange inside the path); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_kv_cache_178_amd import binding
    from paged_kv_cache_178_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    if args.workload == "prefill":
        return run_prefill(args, dev, props)
    if args.workload == "append":
        return run_append(args, dev, props)
    if args.workload == "splitkv":
        return run_splitkv(args, dev, props)
    if args.workload == "fused-prefill":
        return run_fused_prefill(args, dev, props)
    if args.workload == "read-ceiling":
        return run_read_ceiling(args, dev, props)
    decode = args.workload == "decode"
    inp = {"decode": lambda: wl.llama_decode(args.history),
           "batching": wl.continuous_batching, "tiny": wl.tiny_fp32,
           "awkward": wl.awkward_fp16}[args.workload]()
    kv_bytes = inp.kv_bytes()
    log(f"[bench] workload {inp.name}: {kv_bytes} KV bytes, pool {tuple(inp.k_pool.shape)}")

    q = inp.q.to(dev)
    bt = inp.block_table.to(dev)
    lens = inp.context_lens.to(dev)
    pool_bytes = 2 * inp.k_pool.numel() * inp.k_pool.element_size()
    copies = 1 if args.warm else max(1, math.ceil(args.pool_bytes / pool_bytes))
    kbig = inp.k_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
    vbig = inp.v_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
    out = torch.empty_like(q)
    log(f"[bench] {copies} pool copies ({copies * pool_bytes / 2**20:.0f} MiB)")

    opts = binding.PlanOpts(combine_mode=args.combine_mode,
                            force_blocks_per_split=args.blocks_per_split,
                            wgs_per_cu=args.wgs_per_cu, num_cus=props.multi_processor_count,
                            schedule=args.schedule, segment_cost=args.segment_cost)
    desc = binding.make_desc(q, kbig[0], bt, out=out, scale=inp.scale)
    lens_h = inp.context_lens.numpy()
    bt_h = inp.block_table.numpy()
    st = binding.np_check_paged_inputs(desc, q, kbig[0], vbig[0], bt, lens, out, bt_h, lens_h)
    if st:
        raise binding.NPError(st, "np_check_paged_inputs")
    plan = binding.np_plan(desc, lens_h, None, opts)
    ws = binding.workspace_for(plan, dev)
    grid, wg, comb = plan.launch_shape()
    log(f"[bench] plan: schedule {plan.schedule}, blocks/split (stream-K: units per "
        f"workgroup) {plan.blocks_per_split}, splits {plan.max_splits}, "
        f"grid {grid}, combine wgs {comb}, workspace {plan.workspace_bytes} B")

    def step(i: int) -> None:
        c = i % copies
        binding.np_paged_attention_decode(desc, plan, q, kbig[c], vbig[c], bt, lens, out, ws)

    if args.pmc_probe:
        for i in range(10):
            step(i)
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] pmc probe done ({inp.name}): 10 decode steps, 3 copies of 268435456 bytes")
        return 0

    # ---- parity gate (on copy 0) before any timing
    import oracle

    log("[bench] parity gate against the oracle")
    step(0)
    torch.cuda.synchronize()
    ref = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                 inp.context_lens, scale=inp.scale)
    got = out.to("cpu", torch.float64).numpy()
    err = np.abs(got - ref)
    tol = 1e-5 if inp.dtype == "f32" else 1e-2
    if not (err <= tol + tol * np.abs(ref)).all():
        print(f"bench.py: parity gate failed, max abs err {err.max():.3e}", file=sys.stderr)
        return 1
    log(f"[bench] parity gate passed: max abs err {err.max():.3e}")

    # ---- warmup
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: one graph of K steps, each on its own pool copy
    K = args.steps
    us_per_step = graph_us(step, K)
    log(f"[bench] graph: {K} steps -> {us_per_step:.3f} us/step")

    # ---- the decode kernel alone: events around each eager launch
    kernel_us, launch_us = event_us(step, K)
    log(f"[bench] per-launch events: mean {kernel_us:.3f} us, median "
        f"{float(np.median(launch_us)):.3f} us, min {float(launch_us.min()):.3f} us")
    if not decode:
        return report_batching(args, inp, plan, grid, us_per_step, err, props, K, copies)

    # ---- reference kernels: the empty-kernel floor and a plain read of the
    # same number of bytes (cold, rotating over the same pool copies)
    sink = torch.empty(grid[0] * 256, dtype=torch.int32, device=dev)
    kflat = kbig.view(copies, -1)
    read_bytes = kv_bytes // 2 * 2                      # == K half + V half
    src_elems = read_bytes // kbig.element_size()

    def probe_read(i):
        binding.np_probe_stream_read(kflat[i % copies, :src_elems], grid[0], sink)

    def probe_empty(i):
        binding.np_probe_empty()

    empty_us = graph_us(probe_empty, K)
    read_us = graph_us(probe_read, K)
    read_ev_us, _ = event_us(probe_read, K)
    log(f"[bench] probes (graph): empty kernel {empty_us:.3f} us, stream read of {read_bytes} B "
        f"{read_us:.3f} us ({read_bytes / read_us / 1e3:.1f} GB/s)")

    # ---- eager steps with host validation and planning each step
    t_host = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        th = time.perf_counter()
        c = i % copies
        st = binding.np_check_paged_inputs(desc, q, kbig[c], vbig[c], bt, lens, out,
                                           None, lens_h)
        p2 = binding.np_plan(desc, lens_h, None, opts)
        t_host.append(time.perf_counter() - th)
        binding.np_paged_attention_decode(desc, p2, q, kbig[c], vbig[c], bt, lens, out, ws)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / K
    host_us = float(np.median(t_host)) * 1e6
    log(f"[bench] eager with per-step check+plan: {eager_us:.2f} us/step "
        f"(host check+plan via ctypes {host_us:.2f} us)")

    gbs = kv_bytes / (us_per_step * 1e-6) / 1e9
    # The timed region is K back-to-back launches of the decode kernel (one
    # kernel per step), so its average launch duration is the graph time / K.
    achieved = gbs
    # The committed counter summary covers the default plan at 4096 tokens only.
    default_plan = (args.history == 4096 and args.blocks_per_split == 0 and
                    args.combine_mode == 0 and args.schedule == 0 and args.wgs_per_cu == 0)
    traffic = stored_traffic() if default_plan and not args.warm else None
    rec = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"paged decode, Llama-3.2-1B head shape, {args.history}-token history, "
                        "1 layer, batch 1",
            "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 64, "block_size": 16,
            "batch": 1, "history": args.history, "kv_bytes_per_step": kv_bytes,
            "accumulate": "fp32",
            "cache": "MALL-warm (one pool)" if args.warm else
                     f"cold: step i reads pool copy i mod {copies} ({copies * pool_bytes >> 20} "
                     "MiB of copies); 512 MiB flush read before the timed replay",
            "blocks_per_split": plan.blocks_per_split, "splits": plan.max_splits,
            "grid": list(grid), "combine": "separate kernel" if comb else "in-launch",
        },
        "us_per_step": round(us_per_step, 3),
        "hbm_peak_frac": round(gbs / PEAK_HBM_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": (None if traffic is None else traffic["traffic_bytes_per_launch"]),
            "kernel": "paged_decode_kernel (bf16, d_pad 64, group 4, block 16, in-launch merge)",
            "kernel_us": round(us_per_step, 3),
            "kernel_us_event_brackets": round(kernel_us, 3),
        },
        "eager_us_per_step_with_host_plan": round(eager_us, 3),
        "host_check_plan_us": round(host_us, 3),
        "probes": {
            "empty_kernel_us_graph": round(empty_us, 3),
            "stream_read_bytes": read_bytes,
            "stream_read_us_graph": round(read_us, 3),
            "stream_read_gbs_graph": round(read_bytes / read_us / 1e3, 2),
            "stream_read_us_events": round(read_ev_us, 3),
            "note": "same grid size as the decode, cold rotating copies",
        },
        "parity_max_abs_err": float(err.max()),
        "device": props.name,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on the host for ~{args.cpu_seconds:.0f} s")
        best, sample, threads = cpu_baseline(inp, args.cpu_seconds)
        best1, _, _ = cpu_baseline(inp, min(3.0, args.cpu_seconds), threads=1)
        rec["cpu_baseline"] = cpu_record(round(rate(kv_bytes, best * 1e6), 4), "GB/s", sample,
                                         threads, ms_per_step=round(best * 1e3, 3),
                                         one_thread_gbs=round(rate(kv_bytes, best1 * 1e6), 4))
    else:
        rec["cpu_baseline"] = None
    if args.history == 4096 and not args.warm and not args.no_secondary:
        rec["secondary"] = secondary_runs()
    print(json.dumps(rec), flush=True)
    return 0


def secondary_runs(workloads=("batching", "prefill")) -> dict:
    """The continuous-batching decode and the chunked prefill, each measured by a
    child run of this script (default plan, parity gate, graph timing, no CPU
    leg, default steps and warmup, so the per-replay graph overhead is spread
    as in their own runs). A child that fails is recorded with its exit
    status; the headline line is printed either way."""
    out = {}
    for w in workloads:
        log(f"[bench] secondary workload {w}: child run")
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", w, "--no-cpu-baseline"]
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        except subprocess.TimeoutExpired:
            out[w] = {"error": "child run timed out after 600 s"}
            continue
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            out[w] = {"error": f"child run exited with status {r.returncode}",
                      "stderr_tail": r.stderr[-400:]}
            continue
        child = json.loads(lines[-1])
        out[w] = {
            "metric": child["metric"], "value": child["value"], "unit": child["unit"],
            "us_per_step": child["us_per_step"], "steps": child["steps"],
            "roofline_frac": child["roofline"]["frac"], "roofline_bound": child["roofline"]["bound"],
            "traffic": child["roofline"]["traffic"],
            "parity_max_abs_err": child["parity_max_abs_err"],
            "workload": child["config"]["workload"],
        }
        log(f"[bench] secondary {w}: {child['us_per_step']} us/step, "
            f"{child['value']} {child['unit']}")
    return out


SMALL_DECODE = {
    "tiny": ("paged-decode µs/step and KV GB/s, tiny fp32 decode",
             "paged decode, 1 sequence of 64 tokens, Hq = 4, Hkv = 2, d = 64, fp32, 16-block "
             "pool with a permuted table"),
    "awkward": ("paged-decode µs/step and KV GB/s, awkward-shape fp16 decode",
                "paged decode, 3 sequences of 13, 100 and 1037 tokens, Hq = 12, Hkv = 4, "
                "d = 48 padded to 64, fp16, K x4 on 1% of tokens"),
}


def report_batching(args, inp, plan, grid, us_per_step, err, props, K, copies) -> int:
    kv_bytes = inp.kv_bytes()
    if args.workload in SMALL_DECODE:
        return report_small(args, inp, plan, grid, us_per_step, err, props, K, copies)
    # The committed counter summary covers the default stream-K plan only.
    default_plan = (plan.schedule == 2 and args.segment_cost == 0 and args.wgs_per_cu == 0)
    traffic = stored_traffic(PMC_SUMMARY_BATCHING) if default_plan else None
    gbs = kv_bytes / (us_per_step * 1e-6) / 1e9
    rec = {
        "metric": "paged-decode KV GB/s (% HBM peak), continuous batching",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(us_per_step / 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "paged decode, continuous batching: 64 sequences, lengths uniform on "
                        "[128, 8192], Llama-3.2-1B head shape, 40000-block pool, 1 layer",
            "num_seqs": inp.num_seqs, "total_tokens": int(inp.context_lens.sum()),
            "kv_bytes_per_step": kv_bytes,
            "schedule": "stream-K" if plan.schedule == 2 else "uniform splits",
            "blocks_per_split" if plan.schedule == 1 else "units_per_workgroup":
                plan.blocks_per_split,
            "max_splits" if plan.schedule == 1 else "max_pieces_per_segment": plan.max_splits,
            "grid": list(grid),
            "cache": f"{copies} pool copy of {2 * inp.k_pool.numel() * 2 >> 20} MiB (> MALL)",
        },
        "us_per_step": round(us_per_step, 3),
        "hbm_peak_frac": round(gbs / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": (None if traffic is None else traffic["traffic_bytes_per_launch"]),
                     "kernel": ("paged_decode_sk_kernel" if plan.schedule == 2 else
                                "paged_decode_kernel") + " (bf16, d_pad 64, group 4, block 16)"},
        "parity_max_abs_err": float(err.max()),
        "device": props.name,
    }
    if not args.no_cpu_baseline:
        seqs = [0, 1, 2, 3]
        best, sample, threads = cpu_baseline(inp, args.cpu_seconds, seqs=seqs)
        sub_bytes = 2 * inp.num_kv_heads * inp.head_dim * 2 * int(inp.context_lens[seqs].sum())
        rec["cpu_baseline"] = cpu_record(round(rate(sub_bytes, best * 1e6), 4), "GB/s", sample,
                                         threads)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def report_small(args, inp, plan, grid, us_per_step, err, props, K, copies) -> int:
    """The two small decode configurations: latency-bound (a few KiB to a few
    MiB of K/V), reported as µs per step with the GB/s for reference."""
    metric, workload = SMALL_DECODE[args.workload]
    kv_bytes = inp.kv_bytes()
    gbs = kv_bytes / (us_per_step * 1e-6) / 1e9
    rec = {
        "metric": metric, "value": round(us_per_step, 3), "unit": "us/step", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(us_per_step / 1e3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": inp.dtype, "data": "synthetic",
        "config": {"workload": workload, "kv_bytes_per_step": kv_bytes,
                   "schedule": "stream-K" if plan.schedule == 2 else "uniform splits",
                   "grid": list(grid), "cache": f"{copies} rotating pool copies"},
        "us_per_step": round(us_per_step, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 6), "traffic": None,
                     "kernel": ("paged_decode_sk_kernel" if plan.schedule == 2 else
                                "paged_decode_kernel")},
        "parity_max_abs_err": float(err.max()),
        "device": props.name,
    }
    if not args.no_cpu_baseline:
        best, sample, threads = cpu_baseline(inp, args.cpu_seconds)
        rec["cpu_baseline"] = cpu_record(round(best * 1e6, 2), "us/step", sample, threads)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def run_prefill(args, dev, props) -> int:
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_178_amd import binding
    from paged_kv_cache_178_amd import workloads as wl

    inp = wl.chunked_prefill()
    flops = causal_flops(inp)
    log(f"[bench] workload {inp.name}: {flops} causal flops per step")
    q = inp.q.to(dev)
    bt = inp.block_table.to(dev)
    lens = inp.context_lens.to(dev)
    qst = inp.q_start.to(dev)
    pool_bytes = 2 * inp.k_pool.numel() * inp.k_pool.element_size()
    copies = 1 if args.warm else max(1, math.ceil(args.pool_bytes / pool_bytes))
    kbig = inp.k_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
    vbig = inp.v_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
    out = torch.empty_like(q)
    desc = binding.make_desc(q, kbig[0], bt, out=out, scale=inp.scale)
    st = binding.np_check_paged_inputs(desc, q, kbig[0], vbig[0], bt, lens, out,
                                       inp.block_table.numpy(), inp.context_lens.numpy(),
                                       inp.q_start.numpy())
    if st:
        raise binding.NPError(st, "np_check_paged_inputs")
    plan = binding.np_plan(desc, inp.context_lens.numpy(), inp.q_start.numpy())
    grid, wg, _ = plan.launch_shape()
    log(f"[bench] {copies} pool copies; grid {grid}")

    def step(i: int) -> None:
        c = i % copies
        binding.np_paged_attention_prefill(desc, plan, q, kbig[c], vbig[c], bt, lens, qst, out)

    if args.pmc_probe:
        for i in range(5):
            step(i)
        torch.cuda.synchronize()
        return 0
    step(0)
    torch.cuda.synchronize()
    ref = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                 inp.context_lens, q_start=inp.q_start, scale=inp.scale)
    err = np.abs(out.to("cpu", torch.float64).numpy() - ref)
    if not (err <= 1e-2 + 1e-2 * np.abs(ref)).all():
        print(f"bench.py: parity gate failed, max abs err {err.max():.3e}", file=sys.stderr)
        return 1
    log(f"[bench] parity gate passed: max abs err {err.max():.3e}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    us = graph_us(step, K)
    tfs = flops / (us * 1e-6) / 1e12
    log(f"[bench] graph: {K} steps -> {us:.3f} us/step, {tfs:.1f} TFLOP/s")
    rec = {
        "metric": "paged chunked-prefill TFLOP/s (% of dense bf16 MFMA peak)",
        "value": round(tfs, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": "chunked prefill over a paged cache: 4 sequences x (2048 cached + "
                        "512 new rows), causal, Llama-3.2-1B head shape, 1 layer",
            "causal_flops_per_step": flops, "grid": list(grid),
            "cache": f"{copies} rotating pool copies",
        },
        "us_per_step": round(us, 3),
        "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tfs / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "paged_prefill_kernel (bf16, d 64, block 16)"},
        "parity_max_abs_err": float(err.max()),
        "device": props.name,
    }
    busy = stored_mfma_busy()
    rec["mfma_busy"] = None if busy is None else {
        "frac": busy, "counters": "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCC x SIMDs)",
        "from": os.path.relpath(PREFILL_COUNTERS, ROOT)}
    if not args.no_cpu_baseline:
        best, sample, threads = cpu_baseline(inp, args.cpu_seconds, seqs=[0], prefill=True)
        sub = wl.PagedInputs(**{**inp.__dict__, "context_lens": inp.context_lens[:1],
                                "q_start": inp.q_start[:2]})
        rec["cpu_baseline"] = cpu_record(round(rate(causal_flops(sub), best * 1e6, 1e12), 6),
                                         "TFLOP/s", sample, threads)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def run_splitkv(args, dev, props) -> int:
    """Split-KV decode over contiguous caches (NULL block table): the
    num_splits sweep of the contiguous-cache benchmark (B = 4, H = 16, D = 64,
    fp16, N from 1K to 16K, num_splits 1 .. 128 as page-aligned blocks per
    split), next to the planner's default plan."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_178_amd import binding
    from paged_kv_cache_178_amd import workloads as wl

    K = args.steps
    sweep, default, errs = [], {}, []
    cpu_inp = None
    for n_ctx in wl.SPLITKV_CONTEXTS:
        inp = wl.splitkv_decode(n_ctx)
        if cpu_inp is None:
            cpu_inp = inp
        ns = inp.num_seqs
        q = inp.q.to(dev)
        lens = inp.context_lens.to(dev)
        lens_h = inp.context_lens.numpy()
        cache_bytes = 2 * inp.k_pool.numel() * inp.k_pool.element_size()
        copies = max(1, math.ceil(args.pool_bytes / cache_bytes))
        kbig = inp.k_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
        vbig = inp.v_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
        kd = [wl.dense_view(kbig[c], ns) for c in range(copies)]
        vd = [wl.dense_view(vbig[c], ns) for c in range(copies)]
        out = torch.empty_like(q)
        desc = binding.make_desc_contiguous(q, kd[0], out=out, scale=inp.scale)
        st = binding.np_check_paged_inputs(desc, q, kd[0], vd[0], None, lens, out, None, lens_h)
        if st:
            raise binding.NPError(st, "np_check_paged_inputs")
        nb = n_ctx // 16
        plans = [("default", binding.np_plan(desc, lens_h, None,
                                             binding.PlanOpts(num_cus=props.multi_processor_count)))]
        for sp in wl.SPLITKV_SPLITS:
            bps = max(1, -(-nb // sp))
            plans.append((sp, binding.np_plan(desc, lens_h, None,
                                              binding.PlanOpts(force_blocks_per_split=bps))))
        ref = oracle.paged_attention(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                     inp.context_lens, scale=inp.scale)
        for name, plan in plans:
            ws = binding.workspace_for(plan, dev)

            def step(i, plan=plan, ws=ws):
                c = i % copies
                binding.np_paged_attention_decode(desc, plan, q, kd[c], vd[c], None, lens, out,
                                                  ws)

            step(0)
            torch.cuda.synchronize()
            err = np.abs(out.to("cpu", torch.float64).numpy() - ref)
            if not (err <= 1e-2 + 1e-2 * np.abs(ref)).all():
                print(f"bench.py: parity gate failed at N={n_ctx}, plan {name}: max abs err "
                      f"{err.max():.3e}", file=sys.stderr)
                return 1
            errs.append(float(err.max()))
            for i in range(args.warmup):
                step(i)
            us = graph_us(step, K)
            gbs = inp.kv_bytes() / (us * 1e-6) / 1e9
            entry = {"n_ctx": n_ctx, "num_splits": plan.max_splits, "us": round(us, 3),
                     "gbs": round(gbs, 1), "schedule": "stream-K" if plan.schedule == 2
                     else "uniform splits"}
            if name == "default":
                default[n_ctx] = entry
            else:
                entry["requested_splits"] = name
                entry["blocks_per_split"] = plan.blocks_per_split
                sweep.append(entry)
            log(f"[bench] N={n_ctx} plan {name}: {us:.2f} us, {gbs:.0f} GB/s "
                f"({entry['num_splits']} splits)")
        del kbig, vbig, kd, vd
    best = {}
    for e in sweep:
        b = best.get(e["n_ctx"])
        if b is None or e["us"] < b["us"]:
            best[e["n_ctx"]] = e
    top = default[wl.SPLITKV_CONTEXTS[-1]]
    rec = {
        "metric": "contiguous split-KV decode KV GB/s (% HBM peak), B=4 H=16 D=64 fp16, N=16384",
        "value": top["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(top["us"] / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "split-KV decode over contiguous caches (NULL block table): "
                               "4 sequences, Hq = Hkv = 16, d = 64, fp16, one query row",
                   "n_ctx": list(wl.SPLITKV_CONTEXTS), "num_splits": list(wl.SPLITKV_SPLITS),
                   "cache": f"rotating copies, >= {args.pool_bytes / 2**20:.0f} MiB per N"},
        "roofline": {"bound": "hbm", "achieved": top["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(top["gbs"] / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "paged_decode_sk_kernel (f16, d_pad 64, group 1, block 16)"},
        "default_plan": [default[n] for n in wl.SPLITKV_CONTEXTS],
        "best_forced_split": [best[n] for n in wl.SPLITKV_CONTEXTS],
        "sweep": sweep,
        "parity_max_abs_err": max(errs),
        "device": props.name,
    }
    if not args.no_cpu_baseline:
        bst, sample, threads = cpu_baseline(cpu_inp, args.cpu_seconds)
        rec["cpu_baseline"] = cpu_record(round(rate(cpu_inp.kv_bytes(), bst * 1e6), 4), "GB/s",
                                         f"N={cpu_inp.context_lens[0].item()}: {sample}",
                                         threads)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def run_fused_prefill(args, dev, props) -> int:
    """Whole-prompt causal prefill over contiguous caches (past = 0): time and
    peak device memory per N, next to the bytes a prefill that materialises
    the [B, H, N, N] scores and probabilities in fp16 would need (derived,
    not run)."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_178_amd import binding
    from paged_kv_cache_178_amd import workloads as wl

    K = max(1, min(args.steps, 20))
    rows, errs = [], []
    for n_ctx in wl.SPLITKV_CONTEXTS:
        inp = wl.fused_prefill(n_ctx)
        ns, hq, d = inp.num_seqs, inp.num_q_heads, inp.head_dim
        flops = causal_flops(inp)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        q = inp.q.to(dev)
        k = wl.dense_view(inp.k_pool.to(dev), ns)
        v = wl.dense_view(inp.v_pool.to(dev), ns)
        lens = inp.context_lens.to(dev)
        qst = inp.q_start.to(dev)
        torch.cuda.synchronize()
        in_bytes = sum(t.numel() * t.element_size() for t in (q, k, v))
        torch.cuda.reset_peak_memory_stats(dev)
        before = torch.cuda.memory_allocated(dev)
        out = torch.empty_like(q)
        desc = binding.make_desc_contiguous(q, k, out=out, scale=inp.scale)
        plan = binding.np_plan(desc, inp.context_lens.numpy(), inp.q_start.numpy())
        ws = binding.workspace_for(plan, dev)
        binding.np_paged_attention_prefill(desc, plan, q, k, v, None, lens, qst, out, ws)
        torch.cuda.synchronize()
        peak_extra = torch.cuda.max_memory_allocated(dev) - before
        out_bytes = out.numel() * out.element_size()
        # Sampled rows against the oracle: row t of sequence s is the decode of
        # query t over keys 0..t of the same cache.
        rng = np.random.default_rng(n_ctx)
        got = out.to("cpu", torch.float64).numpy()
        worst = 0.0
        for s in range(ns):
            for t in sorted({0, n_ctx // 2, n_ctx - 1, int(rng.integers(n_ctx))}):
                r = s * n_ctx + t
                # Only the blocks row t sees, as a pool of their own.
                nb_t = t // 16 + 1
                b0 = int(inp.block_table[s, 0])
                ref = oracle.paged_attention(inp.q[r:r + 1], inp.k_pool[b0:b0 + nb_t],
                                             inp.v_pool[b0:b0 + nb_t],
                                             torch.arange(nb_t, dtype=torch.int32)[None],
                                             torch.tensor([t + 1], dtype=torch.int32),
                                             scale=inp.scale)
                err = np.abs(got[r:r + 1] - ref)
                if not (err <= 1e-2 + 1e-2 * np.abs(ref)).all():
                    print(f"bench.py: parity gate failed at N={n_ctx}, row {r}: max abs err "
                          f"{err.max():.3e}", file=sys.stderr)
                    return 1
                worst = max(worst, float(err.max()))
        errs.append(worst)

        def step(i):
            binding.np_paged_attention_prefill(desc, plan, q, k, v, None, lens, qst, out, ws)

        for i in range(min(args.warmup, 3)):
            step(i)
        us = graph_us(step, K)
        tfs = flops / (us * 1e-6) / 1e12
        naive = 2 * ns * hq * n_ctx * n_ctx * 2
        rows.append({"n_ctx": n_ctx, "us": round(us, 2), "tflops": round(tfs, 1),
                     "inputs_bytes": in_bytes, "output_bytes": out_bytes,
                     "workspace_bytes": plan.workspace_bytes,
                     "peak_bytes_during_call": peak_extra,
                     "peak_total_bytes": in_bytes + peak_extra,
                     "naive_scores_and_probs_bytes": naive,
                     "naive_peak_bytes": in_bytes + out_bytes + naive})
        log(f"[bench] N={n_ctx}: {us:.1f} us, {tfs:.0f} TFLOP/s; peak {in_bytes + peak_extra} B "
            f"(inputs {in_bytes}, during the call {peak_extra}); naive would hold "
            f"{in_bytes + out_bytes + naive} B")
        del q, k, v, out, ws
    at = next(r for r in rows if r["n_ctx"] == 4096)
    rec = {
        "metric": "fused causal prefill over contiguous caches TFLOP/s, B=4 H=16 D=64 fp16, "
                  "N=4096 (peak memory per N in 'memory')",
        "value": at["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": min(args.warmup, 3), "ms_per_step": round(at["us"] / 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "whole-prompt causal prefill (past = 0), 4 sequences, Hq = Hkv "
                               "= 16, d = 64, fp16, NULL block table",
                   "n_ctx": list(wl.SPLITKV_CONTEXTS)},
        "roofline": {"bound": "mfma", "achieved": at["tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(at["tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "paged_prefill_kernel (f16, d 64, block 16)"},
        "memory": rows,
        "parity": "4 sampled rows per sequence per N against the oracle",
        "parity_max_abs_err": max(errs),
        "device": props.name,
    }
    if not args.no_cpu_baseline:
        small = wl.fused_prefill(1024)
        best, sample, threads = cpu_baseline(small, args.cpu_seconds, seqs=[0], prefill=True)
        sub = wl.PagedInputs(**{**small.__dict__, "context_lens": small.context_lens[:1],
                                "q_start": small.q_start[:2]})
        rec["cpu_baseline"] = cpu_record(round(rate(causal_flops(sub), best * 1e6, 1e12), 6),
                                         "TFLOP/s", f"one 1024-token prompt: {sample}", threads)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


READ_CEILING_SHAPES = ([(w, 256, u) for w in (256, 512, 1024, 2048) for u in (1, 2, 4, 8, 16)] +
                       [(256, t, u) for t in (512, 1024) for u in (1, 2, 4, 8, 16)])


def run_read_ceiling(args, dev, props) -> int:
    """Best single-launch time of a plain read of 8 MiB (the headline's K/V
    bytes) over grid shapes and loads in flight, cold: step i reads copy
    i mod 128 of 1 GiB, with the 512 MiB flush before the timed replay."""
    import torch

    from paged_kv_cache_178_amd import binding

    nbytes = 8 << 20
    copies = 128
    buf = torch.ones((copies, nbytes), dtype=torch.uint8, device=dev)
    sink = torch.empty(2048 * 1024, dtype=torch.int32, device=dev)
    K = args.steps
    empty_us = graph_us(lambda i: binding.np_probe_empty(), K)
    log(f"[bench] empty kernel: {empty_us:.3f} us per graph step")
    rows = []
    for wgs, wg, u in READ_CEILING_SHAPES:
        def step(i, wgs=wgs, wg=wg, u=u):
            binding.np_probe_stream_read_ex(buf[i % copies], wgs, wg, u, sink)
        us = graph_us(step, K)
        per_thread = nbytes // 16 / (wgs * wg)
        rows.append({"workgroups": wgs, "threads": wg, "loads_in_flight": u,
                     "chunks_per_thread": per_thread, "us": round(us, 3),
                     "gbs": round(rate(nbytes, us), 1)})
        log(f"[bench] read {nbytes} B: {wgs} x {wg} threads, {u} loads in flight "
            f"({per_thread:g} chunks per thread): {us:.3f} us, {rate(nbytes, us):.0f} GB/s")
    best = min(rows, key=lambda r: r["us"])
    by_grid = {}
    for r in rows:
        key = (r["workgroups"], r["threads"])
        if key not in by_grid or r["us"] < by_grid[key]["us"]:
            by_grid[key] = r
    rec = {
        "metric": "single-launch plain read of 8 MiB, GB/s (the decode step's read ceiling)",
        "value": best["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": 0,
        "ms_per_step": round(best["us"] / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": "np_probe_stream_read_ex over 8 MiB, graph-timed, cold copies",
                   "bytes": nbytes, "copies": copies},
        "empty_kernel_us_graph": round(empty_us, 3),
        "best": best,
        "best_per_grid": list(by_grid.values()),
        "sweep": rows,
        "roofline": {"bound": "hbm", "achieved": best["gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(best["gbs"] / PEAK_HBM_GBS, 4),
                     "traffic": None, "kernel": "probe_stream_read_kernel"},
        "cpu_baseline": None,
        "device": props.name,
    }
    print(json.dumps(rec), flush=True)
    return 0


def run_append(args, dev, props) -> int:
    """Cache write of the chunked-prefill step: 4 sequences of 2048 cached
    tokens each grow by a 512-token chunk (Llama-3.2-1B head shape, bf16); the
    host allocator grows the tables, the kernel scatters the new K/V rows.
    Bound by HBM: every row is read once and written once."""
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_178_amd import binding

    num_seqs, cached, chunk, hkv, hq, d, bs = 4, 2048, 512, 8, 32, 64, 16
    n_blocks = 2 * num_seqs * (cached + chunk) // bs
    rng = np.random.default_rng(6)
    alloc = binding.BlockAllocator(n_blocks, bs, num_seqs, (cached + chunk) // bs,
                                   rng.permutation(n_blocks))
    for s in range(num_seqs):
        alloc.extend(s, cached + chunk)
    table = alloc.block_table()
    lens = alloc.context_lens()
    new_start = np.arange(num_seqs + 1, dtype=np.int32) * chunk
    n = num_seqs * chunk
    g = torch.Generator().manual_seed(6)
    k_pool = torch.randn((n_blocks, bs, hkv, d), generator=g).to(torch.bfloat16)
    v_pool = torch.randn((n_blocks, bs, hkv, d), generator=g).to(torch.bfloat16)
    k_new = torch.randn((n, hkv, d), generator=g).to(torch.bfloat16)
    v_new = torch.randn((n, hkv, d), generator=g).to(torch.bfloat16)
    row_bytes = 2 * n * hkv * d * 2          # K and V rows of the chunk
    traffic_alg = 2 * row_bytes              # each read once, written once
    per_copy = 2 * k_pool.numel() * 2 + row_bytes
    copies = 1 if args.warm else max(1, math.ceil(args.pool_bytes / per_copy))
    kp = k_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
    vp = v_pool.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1, 1)
    kn = k_new.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1)
    vn = v_new.to(dev).unsqueeze(0).repeat(copies, 1, 1, 1)
    bt = torch.from_numpy(table).to(dev)
    ln = torch.from_numpy(lens).to(dev)
    ns = torch.from_numpy(new_start).to(dev)
    q_dummy = torch.empty((n, hq, d), dtype=torch.bfloat16, device=dev)
    desc = binding.make_desc(q_dummy, kp[0], bt, n_q_total=n)
    plan = binding.np_plan(desc, lens, new_start)
    grid, _, _ = plan.launch_shape()

    def step(i: int) -> None:
        c = i % copies
        binding.np_paged_kv_append(desc, plan, kn[c], vn[c], bt, ln, ns, kp[c], vp[c])

    log(f"[bench] append: {n} rows, {copies} rotating copies")
    step(0)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.append_kv(k_pool, v_pool, table, lens, new_start, k_new, v_new)
    ok = (np.array_equal(oracle.paged._raw_bits(kp[0].cpu()), k_ref) and
          np.array_equal(oracle.paged._raw_bits(vp[0].cpu()), v_ref))
    if not ok:
        print("bench.py: parity gate failed: pools differ from the oracle", file=sys.stderr)
        return 1
    log("[bench] parity gate passed: pools bit-exact")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    us = graph_us(step, K)
    gbs = traffic_alg / (us * 1e-6) / 1e9
    log(f"[bench] graph: {K} steps -> {us:.3f} us/step, {gbs:.1f} GB/s")
    rec = {
        "metric": "paged KV append GB/s (rows read + written, % HBM peak)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": "KV cache write of a chunked-prefill step: 4 sequences x 512 new "
                        "tokens after 2048 cached, Llama-3.2-1B head shape, 1 layer",
            "rows": n, "bytes_read_plus_written": traffic_alg, "grid": list(grid),
            "cache": f"{copies} rotating copies of pools and new rows",
        },
        "us_per_step": round(us, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "paged_append_kernel"},
        "device": props.name,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        times = time_runs(lambda: oracle.append_kv(k_pool, v_pool, table, lens, new_start,
                                                   k_new, v_new), args.cpu_seconds)
        st = run_stats(times)
        rec["cpu_baseline"] = cpu_record(
            round(rate(traffic_alg, st["best"] * 1e6), 4), "GB/s",
            f"full workload (numpy copies, one thread), best of {st['runs']} runs", 1)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
