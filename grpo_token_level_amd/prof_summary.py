"""Turns rocprofv3 CSV output into the short text summaries kept under
``profiles/``.

    python -m grpo_token_level_amd.prof_summary stats KERNEL_STATS_CSV OUT.txt --cmd "..."
    python -m grpo_token_level_amd.prof_summary pmc FETCH_CSV WRITE_CSV OUT.txt --cmd "..." \
        [--kernel tok_reg_kernel<1, 1, 1024, 19, true>]

``pmc`` calibrates the two TCC byte counters with the plain copy the bench
runs under ``--copy-calibration`` (a 1 GiB int32 bitwise-not: 1 GiB read,
1 GiB written, one dispatch): factor = counter / known bytes.  The traffic of
the named kernel per launch is then fetch/f_fetch + write/f_write.  The
summary records a hash of the kernel source so that a stale figure is never
reported for a changed kernel.
"""

import argparse
import csv
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(PKG, "csrc", "loss_kernels.hip")
CALIB_KERNEL = "bitwise_not_kernel"
CALIB_BYTES = 1 << 30


def kernel_source_hash(path=KERNEL_SOURCE):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def stats(args):
    rows = _rows(args.csv)
    lines = [f"# rocprofv3 kernel trace summary: {args.title}", "", "command:", f"  {args.cmd}", "",
             f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}"]
    for r in rows[: args.top]:
        lines.append(f"{r['Name'][:72]:<72} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>8.2f}")
    if args.bench_log:
        with open(args.bench_log) as f:
            for line in f:
                if line.startswith("{") and '"roofline"' in line:
                    rec = json.loads(line)
                    rf = rec["roofline"]
                    lines += ["", "the profiled bench run's own line (HIP events around each fused-loss call):",
                              f"  avg_launch_ms {rf['avg_launch_ms']}  achieved {rf['achieved']} {rf['unit']}  "
                              f"ms_per_step {rec['ms_per_step']}  value {rec['value']} {rec['unit']}"]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_kernel(rows, needle):
    vals = [float(r["Counter_Value"]) for r in rows if needle in r["Kernel_Name"]]
    return vals


def pmc(args):
    fr, wr = _rows(args.fetch), _rows(args.write)
    kf, kw = _per_kernel(fr, args.kernel), _per_kernel(wr, args.kernel)
    cf, cw = _per_kernel(fr, CALIB_KERNEL), _per_kernel(wr, CALIB_KERNEL)
    if not kf or not kw or not cf or not cw:
        raise SystemExit("kernel or calibration copy not found in the counter CSVs")
    f_fetch = (sum(cf) / len(cf)) * 1024 / CALIB_BYTES
    f_write = (sum(cw) / len(cw)) * 1024 / CALIB_BYTES
    fetch = sum(kf) / len(kf)
    write = sum(kw) / len(kw)
    traffic = (fetch / f_fetch + write / f_write) * 1024
    rec = {"kernel": args.kernel, "workload": args.workload, "launches": len(kf),
           "fetch_kib_per_launch": round(fetch, 1), "write_kib_per_launch": round(write, 1),
           "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4),
           "traffic_bytes_per_launch": int(traffic), "kernel_source_sha256": kernel_source_hash()}
    lines = [f"# rocprofv3 HBM byte counters: {args.kernel} on the {args.workload} workload", "",
             "commands:", f"  {args.cmd}", "",
             f"calibration copy ({CALIB_KERNEL}, 1 GiB read + 1 GiB written, {len(cf)} dispatches):",
             f"  FETCH_SIZE {sum(cf) / len(cf):.1f} KiB -> factor {f_fetch:.4f}",
             f"  WRITE_SIZE {sum(cw) / len(cw):.1f} KiB -> factor {f_write:.4f}", "",
             f"{args.kernel}, {len(kf)} launches:",
             f"  FETCH_SIZE {fetch:.1f} KiB/launch -> {fetch / f_fetch * 1024 / 1e9:.4f} GB read",
             f"  WRITE_SIZE {write:.1f} KiB/launch -> {write / f_write * 1024 / 1e9:.4f} GB written",
             f"  traffic {traffic / 1e9:.4f} GB/launch", "",
             "TRAFFIC_JSON " + json.dumps(rec)]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def load_traffic(path, kernel_source=KERNEL_SOURCE):
    """The TRAFFIC_JSON record of a pmc summary, or None when it is missing or
    was taken on a different kernel source."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("TRAFFIC_JSON "):
                    rec = json.loads(line[len("TRAFFIC_JSON "):])
                    if rec.get("kernel_source_sha256") == kernel_source_hash(kernel_source):
                        return rec
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--bench-log", default=None, help="stdout of the profiled bench.py run")
    p = sub.add_parser("pmc")
    p.add_argument("fetch")
    p.add_argument("write")
    p.add_argument("out")
    p.add_argument("--cmd", required=True)
    p.add_argument("--kernel", default="tok_reg_kernel<1, 1, 1024, 19, true>")
    p.add_argument("--workload", default="qwen")
    a = ap.parse_args()
    stats(a) if a.mode == "stats" else pmc(a)


if __name__ == "__main__":
    main()
