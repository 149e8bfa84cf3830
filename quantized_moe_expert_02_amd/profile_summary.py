"""Short text summaries of rocprofv3 output for the profiles/ folder.

  python -m quantized_moe_expert_02_amd.profile_summary stats DB_OR_DIR --title T --command C
      per-kernel calls and average / min / max duration from a --kernel-trace run
  python -m quantized_moe_expert_02_amd.profile_summary traffic FETCH_DIR WRITE_DIR --kernel K --copy-mb N
      --workload W --source FILE --command C
      HBM traffic per launch of kernel K from a FETCH_SIZE run and a WRITE_SIZE run (rocprofv3 --pmc,
      --output-format csv), each scaled by what the same counter reads for the plain copy kernel that
      `bench.py --calibrate-copy-mb N` runs first (N MB read and N MB written per launch)
  python -m quantized_moe_expert_02_amd.profile_summary requests PMC_DIR --kernel K [K ...] --copy-mb N
      --workload W --command C
      HBM read bytes per launch from the read-request counts by size (32/64/128 B), for the copy kernel
      and the kernels named, to check the scale factor of FETCH_SIZE
  python -m quantized_moe_expert_02_amd.profile_summary mfma PMC_DIR --kernel K --workload W --command C
      fp16 matrix-core work per launch of the kernels whose names contain K, from one rocprofv3 --pmc run of
      the derived metrics MfmaFlopsF16 (SQ_INSTS_VALU_MFMA_MOPS_F16 x 512) and MfmaUtil (matrix-core busy
      cycles over GRBM_GUI_ACTIVE x SIMDs)
  python -m quantized_moe_expert_02_amd.profile_summary counters PMC_DIR --kernel K --title T --command C
      mean value per dispatch of every counter of one rocprofv3 --pmc run, for the kernels whose names
      contain K
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_KERNEL = "neg"  # torch.neg(src, out=dst): one read and one write of the tensor


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0]


def _find(path: str, pattern: str) -> str:
    if os.path.isfile(path):
        return path
    hits = sorted(glob.glob(os.path.join(path, "**", pattern), recursive=True))
    if not hits:
        sys.exit(f"no {pattern} under {path}")
    return hits[0]


def stats(args) -> None:
    db = _find(args.path, "*results.db")
    con = sqlite3.connect(db)
    rows = list(con.execute("select name, count(*), avg(end-start), min(end-start), max(end-start), sum(end-start) "
                            "from kernels group by name order by sum(end-start) desc"))
    print(f"# {args.title}")
    print(f"# command: {args.command}")
    print("# kernel durations from rocprofv3 --kernel-trace, in us; this library's kernels (moe::) only")
    print(f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total_us':>11}  kernel")
    for n, c, a, mi, ma, s in rows:
        k = _short(n)
        if k.startswith("moe::"):
            print(f"{c:6d} {a / 1e3:9.2f} {mi / 1e3:9.2f} {ma / 1e3:9.2f} {s / 1e3:11.1f}  {k[:110]}")


def _counter(path: str, counter: str):
    """{short kernel name: [values per dispatch]} for one counter (KiB per dispatch as rocprofv3 reports)."""
    f = _find(path, "*counter_collection.csv")
    out = {}
    with open(f) as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(_short(row["Kernel_Name"]), []).append(float(row["Counter_Value"]))
    return out


def traffic(args) -> None:
    fetch = _counter(args.fetch_dir, "FETCH_SIZE")
    write = _counter(args.write_dir, "WRITE_SIZE")

    def pick(d, key):
        hits = [v for k, v in d.items() if key in k]
        if not hits:
            sys.exit(f"kernel matching {key!r} not found; kernels: {sorted(d)[:20]}")
        vals = [x for h in hits for x in h]
        return sum(vals) / len(vals), len(vals)

    copy_bytes = args.copy_mb * (1 << 20)
    cf, _ = pick(fetch, COPY_KERNEL)
    cw, _ = pick(write, COPY_KERNEL)
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    kf, nf = pick(fetch, args.kernel)
    kw, nw = pick(write, args.kernel)
    fetch_b = kf * 1024.0 * f_scale
    write_b = kw * 1024.0 * w_scale
    src = os.path.join(ROOT, args.source)
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    label = args.label or args.kernel
    print(f"# HBM traffic per launch of {label} ({args.workload}), rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE")
    print(f"# command: {args.command}")
    print(f"# copy calibration: torch.neg over {args.copy_mb} MB reads FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE "
          f"{cw:.0f} KiB per launch; scale factors fetch {f_scale:.4f}, write {w_scale:.4f}")
    print(f"kernel = {label}")
    print(f"kernel_match = {args.kernel}")
    print(f"workload = {args.workload}")
    print(f"dispatches = {nf} / {nw}")
    print(f"fetch_kib_per_dispatch = {kf:.1f}")
    print(f"write_kib_per_dispatch = {kw:.1f}")
    print(f"fetch_bytes_per_launch = {fetch_b:.0f}")
    print(f"write_bytes_per_launch = {write_b:.0f}")
    print(f"bytes_per_launch = {fetch_b + write_b:.0f}")
    print(f"source = {args.source}")
    print(f"source_sha256 = {sha}")


def requests(args) -> None:
    """HBM read bytes per launch from the L2's read-request counts by size
    (TCC_EA0_RDREQ_{32B,64B,128B}_sum), an independent check of the scaled
    FETCH_SIZE: bytes = 32 n32 + 64 n64 + 128 n128, for the copy kernel and
    for the named kernels."""
    cnt = {c: _counter(args.path, c) for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum",
                                               "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")}
    print(f"# HBM read requests by size per launch, rocprofv3 --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum "
          f"TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum ({args.workload})")
    print(f"# command: {args.command}")
    print(f"# bytes = 32 n32 + 64 n64 + 128 n128; copy kernel: torch.neg over {args.copy_mb} MB "
          f"({args.copy_mb * (1 << 20)} bytes read per launch)")
    print(f"{'requests':>12} {'n32':>10} {'n64':>12} {'n128':>12} {'bytes':>14}  kernel")
    for key in [COPY_KERNEL] + args.kernel:
        row = []
        for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"):
            hits = [x for k, v in cnt[c].items() if key in k for x in v]
            row.append(sum(hits) / len(hits) if hits else float("nan"))
        n, n32, n64, n128 = row
        print(f"{n:12.0f} {n32:10.0f} {n64:12.0f} {n128:12.0f} {32 * n32 + 64 * n64 + 128 * n128:14.0f}  {key}")


def mfma(args) -> None:
    flops = _counter(args.path, "MfmaFlopsF16")
    util = _counter(args.path, "MfmaUtil")
    names = sorted(k for k in flops if args.kernel in k)
    if not names:
        sys.exit(f"kernel matching {args.kernel!r} not found; kernels: {sorted(flops)[:20]}")
    print(f"# fp16 matrix-core work per launch, {args.workload}: rocprofv3 --pmc MfmaFlopsF16 MfmaUtil")
    print(f"# command: {args.command}")
    print("# executed flops count every issued v_mfma (the padding of partly filled 16-token groups included);")
    print("# MfmaUtil = matrix-core busy cycles / (GRBM_GUI_ACTIVE x SIMDs) over the dispatch, in %")
    print(f"{'dispatches':>10} {'gflop_per_launch':>17} {'mfma_util_pct':>14}  kernel")
    for k in names:
        f = flops[k]
        u = util.get(k, [])
        um = sum(u) / len(u) if u else float("nan")
        print(f"{len(f):10d} {sum(f) / len(f) / 1e9:17.2f} {um:14.2f}  {k[:110]}")


def counters(args) -> None:
    f = _find(args.path, "*counter_collection.csv")
    vals = {}
    with open(f) as fh:
        for row in csv.DictReader(fh):
            k = _short(row["Kernel_Name"])
            if args.kernel in k:
                vals.setdefault(k, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    if not vals:
        sys.exit(f"kernel matching {args.kernel!r} not found")
    print(f"# {args.title}")
    print(f"# command: {args.command}")
    print("# mean counter value per dispatch")
    for k in sorted(vals):
        print(k[:110])
        for c in sorted(vals[k]):
            v = vals[k][c]
            print(f"  {c:28s} {sum(v) / len(v):16.4g}   ({len(v)} dispatches)")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    a = sub.add_parser("stats")
    a.add_argument("path")
    a.add_argument("--title", required=True)
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--kernel", required=True, help="substring of the kernel name in the counter output")
    b.add_argument("--label", default="", help="kernel name for the record (default: --kernel)")
    b.add_argument("--copy-mb", type=int, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--source", required=True)
    b.add_argument("--command", required=True)
    c = sub.add_parser("mfma")
    c.add_argument("path")
    c.add_argument("--kernel", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--command", required=True)
    r = sub.add_parser("requests")
    r.add_argument("path")
    r.add_argument("--kernel", nargs="+", required=True)
    r.add_argument("--copy-mb", type=int, required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--command", required=True)
    e = sub.add_parser("counters")
    e.add_argument("path")
    e.add_argument("--kernel", required=True)
    e.add_argument("--title", required=True)
    e.add_argument("--command", required=True)
    args = ap.parse_args()
    {"stats": stats, "traffic": traffic, "requests": requests, "mfma": mfma, "counters": counters}[args.mode](args)


if __name__ == "__main__":
    main()
