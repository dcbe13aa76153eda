"""Short text summaries of rocprofv3 CSV output, for committing beside the code.

Two modes:

  stats    from a `rocprofv3 --kernel-trace --stats -f csv` run: per-kernel calls and
           durations, largest total first.
  traffic  HBM bytes per call of an entry point, from `rocprofv3 --pmc` runs of a workload and
           of bd_hbm_copy over a known number of bytes (the calibration):
             * FETCH_SIZE and WRITE_SIZE (one run each), each scaled by the bytes the copy moved
               per unit the same counter read on it;
             * optionally the raw request counters TCC_EA0_RDREQ_{32B,64B,128B}_sum and
               TCC_EA0_WRREQ_64B_sum (32/64/128-byte reads, 64-byte writes), checked the same
               way on the copy.
           The per-dispatch mean of every kernel the entry point launches is summed.

  counters per-kernel means of any counters (raw or derived, e.g. MfmaUtil, VALUBusy) from a
           `rocprofv3 --pmc ...` run, one line per kernel pattern.

Usage:
  python -m block_diffusion_lm_router_amd.profsum counters --csv X_counter_collection.csv \
      --kernel NAME=REGEX [--kernel NAME=REGEX ...] --command "..." --out profiles/NAME.txt
  python -m block_diffusion_lm_router_amd.profsum stats --csv X_kernel_stats.csv \
      --command "..." --out profiles/NAME.txt
  python -m block_diffusion_lm_router_amd.profsum traffic --fetch A.csv --write B.csv \
      --copy-fetch C.csv --copy-write D.csv [--req E.csv --copy-req F.csv] \
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
    """Short hash of the sources behind the gate/up launch (the grouped GEMM, and the routing
    that builds its work list), stamped on traffic summaries so that a summary taken on
    another version of them is recognised as stale."""
    h = hashlib.sha256()
    for name in ("moe_w4a16.hip", "moe_route.hip"):
        with open(os.path.join(_HERE, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name, width=110):
    """Kernel name without namespaces noise, cut to a readable width."""
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"rocprim::ROCPRIM_\w+::(detail::)?", "rocprim::", name)
    return name if len(name) <= width else name[:width - 3] + "..."


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
                   f"  {_short(r['Name'])}")
    out.append(f"\nall kernels: {total / 1e3:.1f} us over {sum(int(r['Calls']) for r in rows)} calls")
    text = "\n".join(out) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


def counters(args):
    """Mean of every counter per kernel pattern (the first pattern that matches a kernel name)."""
    pats = [kv.split("=", 1) for kv in args.kernel]
    vals = {}
    for r in _rows(args.csv):
        for name, rx in pats:
            if re.search(rx, r["Kernel_Name"]):
                d = vals.setdefault(name, {}).setdefault(r["Counter_Name"], {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
                break
    names = sorted({c for per in vals.values() for c in per})
    out = [f"command: {args.command}", "",
           f"{'kernel':<16} {'dispatches':>10} " + " ".join(f"{c:>14}" for c in names)]
    for name, _ in pats:
        per = vals.get(name, {})
        n = max((len(d) for d in per.values()), default=0)
        cells = []
        for c in names:
            d = per.get(c, {})
            cells.append(f"{sum(d.values()) / len(d):>14.2f}" if d else f"{'-':>14}")
        out.append(f"{name:<16} {n:>10} " + " ".join(cells))
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


_REQ = (("TCC_EA0_RDREQ_32B_sum", 32), ("TCC_EA0_RDREQ_64B_sum", 64),
        ("TCC_EA0_RDREQ_128B_sum", 128))


def _req_bytes(path, patterns):
    """Read and write bytes per dispatch from the raw request counters."""
    rd = {p: 0.0 for p in patterns}
    for counter, size in _REQ:
        for p, (v, _) in _per_dispatch(path, counter, patterns).items():
            rd[p] += v * size
    wr = {p: v * 64 for p, (v, _) in _per_dispatch(path, "TCC_EA0_WRREQ_64B_sum", patterns).items()}
    return rd, wr


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
    if args.req and args.copy_req:
        crd, cwr = _req_bytes(args.copy_req, ["copy"])
        rd, wr = _req_bytes(args.req, args.kernel)
        rec["request_counters"] = {
            "copy_read_bytes": int(crd["copy"]), "copy_write_bytes": int(cwr.get("copy", 0)),
            "per_kernel": {p: {"read_bytes": int(rd[p]), "write_bytes": int(wr.get(p, 0))}
                           for p in args.kernel},
            "bytes_per_launch": int(sum(rd.values()) + sum(wr.values()))}
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
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--kernel", action="append", required=True, help="NAME=REGEX")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "command", "out", "entry"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--req")
    t.add_argument("--copy-req")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", action="append", required=True)
    args = ap.parse_args()
    {"stats": stats, "traffic": traffic, "counters": counters}[args.mode](args)


if __name__ == "__main__":
    main()
