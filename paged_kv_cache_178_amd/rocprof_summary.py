"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

stats:    kernel-trace statistics (calls, average/min/max duration per kernel).
counters: median per-dispatch value of every counter collected for one kernel
       (with --simds and --xccs, also the fraction of SIMD cycles the matrix
       cores were busy; with --sha, stamped for the benchmark to read).
pmc:      HBM traffic per launch of one kernel from two counter runs
       (FETCH_SIZE and WRITE_SIZE, KiB per dispatch), each scaled by what the
       same counter reads for a plain copy of known size in the same run.

Usage:
  python -m paged_kv_cache_178_amd.rocprof_summary stats STATS_CSV --out FILE --cmd "..."
  python -m paged_kv_cache_178_amd.rocprof_summary counters CSV [CSV ...] --kernel SUBSTR \
      --out FILE --cmd "..." [--simds N --xccs N --sha SHA]
  python -m paged_kv_cache_178_amd.rocprof_summary pmc --fetch CSV --write CSV \
      --kernel SUBSTR --copy-kernel SUBSTR --copy-bytes N --kv-bytes N --sha SHA \
      --out FILE --cmd "..."
"""

from __future__ import annotations

import argparse
import csv
import json
import statistics


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats(args) -> None:
    rows = _rows(args.csv)
    lines = [f"# Kernel trace: {args.title}", "", "Command:", "", "```", args.cmd, "```", "",
             "| kernel | calls | average (ns) | min (ns) | max (ns) |", "|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} |")
    open(args.out, "w").write("\n".join(lines) + "\n")


def counters(args) -> None:
    vals = {}
    for path in args.csv:
        for r in _rows(path):
            if args.kernel in r.get("Kernel_Name", ""):
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no dispatches of the kernel in the counter files")
    lines = [f"# Hardware counters: {args.title}", "", "Commands (one run per counter set):", "",
             "```", args.cmd, "```", "", "| counter | dispatches | median per dispatch |",
             "|---|---|---|"]
    for name in sorted(vals):
        lines.append(f"| `{name}` | {len(vals[name])} | {statistics.median(vals[name]):.0f} |")
    busy = mfma_busy_frac(vals, args.simds, args.xccs)
    if busy is not None:
        lines += ["", f"- MFMA busy: {100 * busy:.1f}% of the SIMD cycles while the GPU was active "
                      f"(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {args.xccs} XCCs x "
                      f"{args.simds} SIMDs), medians per dispatch)"]
        if args.sha:
            lines.append("counters-json: " + json.dumps({"kernel_sha": args.sha,
                                                         "mfma_busy_frac": round(busy, 4)}))
    open(args.out, "w").write("\n".join(lines) + "\n")


def mfma_busy_frac(vals, simds, xccs):
    """Fraction of SIMD cycles the matrix cores were busy: the busy cycles
    summed over all SIMDs, over the GPU-active cycles of one XCC (the
    per-dispatch value sums the XCCs) times the SIMD count. None without the
    two counters or the device sizes."""
    if not simds or not xccs:
        return None
    if "SQ_VALU_MFMA_BUSY_CYCLES" not in vals or "GRBM_GUI_ACTIVE" not in vals:
        return None
    busy = statistics.median(vals["SQ_VALU_MFMA_BUSY_CYCLES"])
    active = statistics.median(vals["GRBM_GUI_ACTIVE"]) / xccs
    return busy / (active * simds) if active > 0 else None


def _per_dispatch(path, counter, substr):
    """Counter values of the matching kernel's dispatches, in dispatch order."""
    vals = []
    for r in _rows(path):
        if r.get("Counter_Name") != counter:
            continue
        if substr in r.get("Kernel_Name", ""):
            vals.append((int(r.get("Dispatch_Id", 0)), float(r["Counter_Value"])))
    return [v for _, v in sorted(vals)]


def pmc(args) -> None:
    fk = _per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    wk = _per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    # The copy kernel also serves the set-up copies (host to device uploads,
    # some larger): the probe's copies of known size are its last n_copies
    # dispatches.
    fc = _per_dispatch(args.fetch, "FETCH_SIZE", args.copy_kernel)[-args.n_copies:]
    wc = _per_dispatch(args.write, "WRITE_SIZE", args.copy_kernel)[-args.n_copies:]
    if not (fk and wk and fc and wc):
        raise SystemExit("missing dispatches for the kernel or the copy in the counter files")
    # The copy reads and writes copy_bytes each: counter KiB -> bytes factors.
    f_scale = args.copy_bytes / statistics.median(fc)
    w_scale = args.copy_bytes / statistics.median(wc)
    fetch_b = statistics.median(fk) * f_scale
    write_b = statistics.median(wk) * w_scale
    rec = {
        "kernel_sha": args.sha,
        "fetch_kib_per_dispatch": statistics.median(fk),
        "write_kib_per_dispatch": statistics.median(wk),
        "copy_fetch_kib": statistics.median(fc),
        "copy_write_kib": statistics.median(wc),
        "fetch_bytes_per_kib": f_scale,
        "write_bytes_per_kib": w_scale,
        "traffic_bytes_per_launch": round(fetch_b + write_b),
        "kv_bytes_per_launch": args.kv_bytes,
    }
    lines = [
        f"# HBM traffic: {args.title}", "",
        "Commands (one counter per run):", "", "```", args.cmd, "```", "",
        f"- decode kernel dispatches: {len(fk)} (FETCH_SIZE), {len(wk)} (WRITE_SIZE)",
        f"- FETCH_SIZE median {rec['fetch_kib_per_dispatch']:.1f} KiB, WRITE_SIZE median "
        f"{rec['write_kib_per_dispatch']:.1f} KiB per dispatch",
        f"- plain copy of {args.copy_bytes} bytes: FETCH_SIZE {rec['copy_fetch_kib']:.1f} KiB, "
        f"WRITE_SIZE {rec['copy_write_kib']:.1f} KiB -> {f_scale:.2f} and {w_scale:.2f} bytes "
        "per counted KiB",
        f"- scaled: {fetch_b:.0f} bytes fetched + {write_b:.0f} bytes written = "
        f"{rec['traffic_bytes_per_launch']} bytes per launch; algorithmic K+V bytes "
        f"{args.kv_bytes} (ratio {rec['traffic_bytes_per_launch'] / args.kv_bytes:.3f})",
        "", f"traffic-json: {json.dumps(rec)}", ""]
    open(args.out, "w").write("\n".join(lines))


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--out", required=True)
    a.add_argument("--cmd", required=True)
    a.add_argument("--title", default="")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--sha", default="")
    c.add_argument("--simds", type=int, default=0)
    c.add_argument("--xccs", type=int, default=0)
    b = sub.add_parser("pmc")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True)
    b.add_argument("--copy-kernel", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--n-copies", type=int, default=3)
    b.add_argument("--kv-bytes", type=int, required=True)
    b.add_argument("--sha", required=True)
    b.add_argument("--out", required=True)
    b.add_argument("--cmd", required=True)
    b.add_argument("--title", default="")
    args = ap.parse_args(argv)
    {"stats": stats, "counters": counters, "pmc": pmc}[args.mode](args)


if __name__ == "__main__":
    main()
