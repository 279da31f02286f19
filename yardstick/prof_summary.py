"""Turns rocprofv3 CSV output into the short text summaries kept under
``profiles/``.

    python -m yardstick.prof_summary stats KERNEL_STATS_CSV OUT.txt --cmd "..."
    python -m yardstick.prof_summary pmc FETCH_CSV WRITE_CSV OUT.txt --cmd "..." \
        [--kernel "tok_reg_kernel<1, 1, 1024, 19, true, 0, 0>"]

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

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCE = os.path.join(ROOT, "grpo_token_level_amd", "csrc", "loss_kernels.hip")
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
             f"  traffic {traffic / 1e9:.4f} GB/launch", ""]
    algo = _bench_algorithmic_bytes(args.bench_log) if args.bench_log else None
    if algo:
        rec["algorithmic_bytes_per_launch"] = algo
        lines += [f"algorithmic bytes per launch (the profiled bench run's own line): {algo / 1e9:.4f} GB",
                  f"  traffic / algorithmic = {traffic / algo:.4f}", ""]
    lines.append("TRAFFIC_JSON " + json.dumps(rec))
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _bench_algorithmic_bytes(path):
    with open(path) as f:
        for line in f:
            if line.startswith("{") and '"roofline"' in line:
                return json.loads(line)["roofline"].get("algorithmic_bytes_per_launch")
    return None


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


def mfma(args):
    """MFMA busy share and bf16 MFMA work per kernel from one --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16 and GRBM_GUI_ACTIVE.
    The CSV holds each counter summed over the XCD instances, so the GPU-busy
    cycles of a dispatch are GRBM_GUI_ACTIVE / n_xcd; busy share =
    sum(MFMA busy cycles) / (GPU-busy cycles * SIMDs); bf16 MFMA flops =
    MOPS * 512."""
    per = {}
    for r in _rows(args.csv):
        name = r["Kernel_Name"]
        if args.needle not in name:
            continue
        key = name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]
        d = per.setdefault(key, {})
        disp = d.setdefault(r["Dispatch_Id"], {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        disp[r["Counter_Name"]] = float(r["Counter_Value"])
    lines = [f"# rocprofv3 MFMA counters: {args.title}", "", "command:", f"  {args.cmd}", "",
             f"busy share = sum(SQ_VALU_MFMA_BUSY_CYCLES) / ((GRBM_GUI_ACTIVE / {args.n_xcd}) * {args.simds} SIMDs); "
             "bf16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512", "",
             f"{'kernel':40s} {'dispatches':>10s} {'avg_us':>9s} {'MFMA busy %':>12s} {'MFMA TFLOP':>11s} "
             f"{'TFLOP/s':>9s}"]
    tot_busy = tot_active = tot_flop = tot_ns = 0.0
    for key, d in sorted(per.items()):
        busy = sum(x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in d.values())
        active = sum(x.get("GRBM_GUI_ACTIVE", 0.0) for x in d.values()) / args.n_xcd
        flop = sum(x.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for x in d.values()) * 512
        ns = sum(x["ns"] for x in d.values())
        tot_busy += busy
        tot_active += active
        tot_flop += flop
        tot_ns += ns
        lines.append(f"{key[:40]:40s} {len(d):10d} {ns / len(d) / 1e3:9.1f} {100 * busy / (active * args.simds):12.1f} "
                     f"{flop / 1e12:11.2f} {flop / (ns * 1e-9) / 1e12:9.1f}")
    if per:
        lines.append(f"{'all of the above':40s} {'':10s} {'':9s} {100 * tot_busy / (tot_active * args.simds):12.1f} "
                     f"{tot_flop / 1e12:11.2f} {tot_flop / (tot_ns * 1e-9) / 1e12:9.1f}")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


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
    p.add_argument("--kernel", default="tok_reg_kernel<1, 1, 1024, 19, true, 0, 0, false>")
    p.add_argument("--workload", default="qwen")
    p.add_argument("--bench-log", default=None, help="stdout of one of the profiled bench.py runs")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("out")
    m.add_argument("--cmd", required=True)
    m.add_argument("--title", default="")
    m.add_argument("--needle", default="gemm_nt_kernel", help="keep kernels whose name contains this")
    m.add_argument("--n-xcd", type=int, default=8)
    m.add_argument("--simds", type=int, default=1024, help="SIMDs on the chip (256 CUs x 4)")
    a = ap.parse_args()
    {"stats": stats, "pmc": pmc, "mfma": mfma}[a.mode](a)


if __name__ == "__main__":
    main()
