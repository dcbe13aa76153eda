"""Short text summaries of rocprofv3 CSV output, for committing beside the code.

Two modes:

  stats    from a `rocprofv3 --kernel-trace --stats -f csv` run: per-kernel calls and
           durations, largest total first.
  traffic  from two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a workload and
           the same two counters read on bd_hbm_copy of a known size (the calibration): HBM
           bytes per call of an entry point, as the mean per-dispatch counter of every kernel
           the entry point launches, summed, times the copy's bytes-per-counter-unit.

Usage:
  python -m block_diffusion_lm_router_amd.profsum stats --csv X_kernel_stats.csv \
      --command "..." --out profiles/NAME.txt
  python -m block_diffusion_lm_router_amd.profsum traffic --fetch A_counter_collection.csv \
      --write B_counter_collection.csv --copy-fetch C.csv --copy-write D.csv \
      --copy-bytes 1073741824 --kernel REGEX [--kernel REGEX ...] --entry NAME \
      --command "..." --out profiles/NAME.json
"""

import argparse
import csv
import hashlib
import json
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash():
    """Short hash of the grouped GEMM's source, stamped on traffic summaries so that a
    summary taken on another version of the kernel is recognised as stale."""
    h = hashlib.sha256()
    with open(os.path.join(_HERE, "csrc", "moe_w4a16.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats(args):
    rows = _rows(args.csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"command: {args.command}", "",
           f"{'calls':>7} {'total_us':>11} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}  kernel"]
    for r in rows[:args.top]:
        out.append(f"{int(r['Calls']):>7} {float(r['TotalDurationNs']) / 1e3:>11.1f} "
                   f"{float(r['AverageNs']) / 1e3:>9.2f} {float(r['MinNs']) / 1e3:>9.2f} "
                   f"{float(r['MaxNs']) / 1e3:>9.2f} {100 * float(r['TotalDurationNs']) / total:>6.2f}"
                   f"  {r['Name']}")
    out.append(f"\nall kernels: {total / 1e3:.1f} us over {sum(int(r['Calls']) for r in rows)} calls")
    text = "\n".join(out) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


def _per_dispatch(path, counter, patterns):
    """Mean counter value per dispatch for each kernel whose name matches a pattern."""
    vals = {}
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        for p in patterns:
            if re.search(p, name):
                vals.setdefault(p, {}).setdefault(r["Dispatch_Id"], 0.0)
                vals[p][r["Dispatch_Id"]] += float(r["Counter_Value"])
                break
    return {p: (sum(d.values()) / len(d), len(d)) for p, d in vals.items()}


def traffic(args):
    copy_f = _per_dispatch(args.copy_fetch, "FETCH_SIZE", ["copy"])
    copy_w = _per_dispatch(args.copy_write, "WRITE_SIZE", ["copy"])
    f_kib, _ = copy_f["copy"]
    w_kib, _ = copy_w["copy"]
    f_scale = args.copy_bytes / (f_kib * 1024.0)   # bytes per counted byte
    w_scale = args.copy_bytes / (w_kib * 1024.0)
    fetch = _per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    write = _per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    kernels = {}
    total = 0.0
    for p in args.kernel:
        fk, nf = fetch.get(p, (0.0, 0))
        wk, nw = write.get(p, (0.0, 0))
        b = fk * 1024.0 * f_scale + wk * 1024.0 * w_scale
        kernels[p] = {"fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
                      "dispatches": [nf, nw], "hbm_bytes": int(b)}
        total += b
    rec = {"entry_point": args.entry, "command": args.command,
           "kernel_source_sha256_16": kernel_source_hash(),
           "calibration": {"copy_bytes": args.copy_bytes, "copy_fetch_kib_raw": round(f_kib, 1),
                           "copy_write_kib_raw": round(w_kib, 1),
                           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "kernels": kernels, "hbm_bytes_per_launch": int(total)}
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--top", type=int, default=20)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "command", "out", "entry"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", action="append", required=True)
    args = ap.parse_args()
    (stats if args.mode == "stats" else traffic)(args)


if __name__ == "__main__":
    main()
