"""Summaries of rocprofv3 result databases (SQLite) for the OSCAR kernels.

    python -m kv_cache_int2_amd.rocprof_summary trace DB --command CMD [--tail NAME:N[:M]]
        per-kernel dispatch statistics (count, average / min / max duration),
        as a short markdown table; --tail adds the same statistics over the
        last N dispatches of the kernel whose name contains NAME (the timed
        steps of a run, without its warm-up), after leaving out its last M
        (dispatches that follow the timed steps).

    python -m kv_cache_int2_amd.rocprof_summary sq DB --kernel NAME [--kernel NAME ...]
        [--tail N] [--skip-last M]  MFMA utilisation and VALU busy per kernel from one
        SQ counter pass (SQ_INSTS_VALU, SQ_INSTS_MFMA, SQ_ACTIVE_INST_VALU,
        SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE); --skip-last drops each kernel's
        last M dispatches before --tail takes its last N.

    python -m kv_cache_int2_amd.rocprof_summary pmc --fetch DB --write DB
        --kernel NAME --copy NAME --copy-bytes N --workload W --source FILE
        --algorithmic-bytes N --command CMD [--tail N]
        HBM traffic per launch of one kernel from a FETCH_SIZE pass and a
        WRITE_SIZE pass (KiB per dispatch), each scaled by what the same
        counter reads for a plain copy kernel that moves a known number of
        bytes in each direction (its largest dispatch: a workload's own page
        copies are far smaller than the calibration copy).  Prints JSON; the
        source hash ties the figure to the kernel source it was measured on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import sqlite3
import sys


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0][-60:]


def kernel_stats(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                       "from kernels group by name order by sum(duration) desc").fetchall()
    return [dict(name=_short(n), calls=c, avg_us=a / 1e3, min_us=lo / 1e3, max_us=hi / 1e3, total_ms=t / 1e6)
            for n, c, a, lo, hi, t in rows]


def counter_per_dispatch(db: str, counter: str, kernel: str, tail: int = 0):
    """Per-dispatch values of a counter for kernels whose name contains `kernel`
    (summed over the counter's hardware instances), in dispatch order; tail > 0
    keeps the last `tail` dispatches."""
    con = sqlite3.connect(db)
    q = ("select k.dispatch_id, sum(p.counter_value) from pmc_events p join kernels k "
         "on p.dispatch_id = k.dispatch_id where p.counter_name = ? and k.name like ? group by k.dispatch_id "
         "order by k.dispatch_id")
    vals = [v for _, v in con.execute(q, (counter, f"%{kernel}%")).fetchall()]
    return vals[-tail:] if tail > 0 else vals


def counter_agg_per_dispatch(db: str, counter: str, kernel: str, agg: str):
    """Per-dispatch values of a counter over its hardware instances (agg: sum or max)."""
    con = sqlite3.connect(db)
    q = (f"select k.dispatch_id, {agg}(p.counter_value) from pmc_events p join kernels k "
         "on p.dispatch_id = k.dispatch_id where p.counter_name = ? and k.name like ? group by k.dispatch_id")
    return {d: v for d, v in con.execute(q, (counter, f"%{kernel}%")).fetchall()}


SQ_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def sq_stats(db: str, kernel: str, cu_num: int, simd_num: int, tail: int = 0, skip_last: int = 0):
    """MFMA utilisation and VALU busy of one kernel, averaged over its
    dispatches, with the tool's own derived-metric formulas:
      MfmaUtil = 100 sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) SIMD_NUM)
      VALUBusy = 100 sum(SQ_ACTIVE_INST_VALU) / CU_NUM / max(GRBM_GUI_ACTIVE)"""
    v = {c: counter_agg_per_dispatch(db, c, kernel, "max" if c.startswith("GRBM") else "sum") for c in SQ_COUNTERS}
    ids = sorted(set.intersection(*(set(x) for x in v.values())))
    if skip_last > 0:
        ids = ids[:-skip_last]
    if tail > 0:
        ids = ids[-tail:]
    if not ids:
        sys.exit(f"no SQ counters for {kernel} in {db}")
    mfma = [100.0 * v["SQ_VALU_MFMA_BUSY_CYCLES"][d] / (v["GRBM_GUI_ACTIVE"][d] * simd_num) for d in ids]
    valu = [100.0 * v["SQ_ACTIVE_INST_VALU"][d] / cu_num / v["GRBM_GUI_ACTIVE"][d] for d in ids]
    mean = lambda xs: sum(xs) / len(xs)
    return dict(dispatches=len(ids), mfma_util_pct=mean(mfma), valu_busy_pct=mean(valu),
                valu_insts=mean([v["SQ_INSTS_VALU"][d] for d in ids]),
                mfma_insts=mean([v["SQ_INSTS_MFMA"][d] for d in ids]),
                gui_active_cycles=mean([v["GRBM_GUI_ACTIVE"][d] for d in ids]))


def cmd_sq(a):
    out = [f"| kernel | dispatches | MFMA util % | VALU busy % | VALU insts | MFMA insts | GUI active cycles |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for k in a.kernel:
        r = sq_stats(a.db, k, a.cu_num, a.simd_num, a.tail, a.skip_last)
        out.append(f"| {k} | {r['dispatches']} | {r['mfma_util_pct']:.1f} | {r['valu_busy_pct']:.1f} "
                   f"| {r['valu_insts']:.4g} | {r['mfma_insts']:.4g} | {r['gui_active_cycles']:.4g} |")
    print("\n".join(out))


def tail_stats(db: str, kernel: str, n: int, skip_last: int = 0):
    con = sqlite3.connect(db)
    d = [r[0] for r in con.execute("select duration from kernels where name like ? order by start desc "
                                   "limit ? offset ?", (f"%{kernel}%", n, skip_last)).fetchall()]
    if not d:
        sys.exit(f"no dispatches of {kernel} in {db}")
    return dict(calls=len(d), avg_us=sum(d) / len(d) / 1e3, min_us=min(d) / 1e3, max_us=max(d) / 1e3,
                total_ms=sum(d) / 1e6)


def cmd_trace(a):
    rows = kernel_stats(a.db)
    out = [f"# rocprofv3 kernel trace: {a.title}", "", "Command:", "", "```", a.command, "```", "",
           "| kernel | calls | avg us | min us | max us | total ms |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {r['name']} | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | {r['max_us']:.2f} "
                   f"| {r['total_ms']:.3f} |")
    for spec in a.tail or []:
        parts = spec.split(":")
        name, n = parts[0], int(parts[1])
        skip = int(parts[2]) if len(parts) > 2 else 0
        r = tail_stats(a.db, name, n, skip)
        before = f" before its last {skip}" if skip else ""
        out += ["", f"Last {r['calls']} dispatches of {name}{before}:", "",
                "| kernel | calls | avg us | min us | max us | total ms |", "|---|---:|---:|---:|---:|---:|",
                f"| {name} (last {r['calls']}) | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} "
                f"| {r['max_us']:.2f} | {r['total_ms']:.3f} |"]
    if a.notes:
        with open(a.notes) as f:
            out += ["", f.read().rstrip()]
    print("\n".join(out))


def cmd_pmc(a):
    res = {"kernel": a.kernel, "workload": a.workload, "command": a.command}
    with open(a.source, "rb") as f:
        res["kernel_source_sha256"] = hashlib.sha256(f.read()).hexdigest()
    total = 0.0
    for counter, db in (("FETCH_SIZE", a.fetch), ("WRITE_SIZE", a.write)):
        k = counter_per_dispatch(db, counter, a.kernel, a.tail)
        c = counter_per_dispatch(db, counter, a.copy)
        if not k or not c:
            sys.exit(f"no {counter} values for {a.kernel} or {a.copy} in {db}")
        copy_kib = max(c)
        factor = a.copy_bytes / (copy_kib * 1024.0)        # true bytes per counted byte
        kern_kib = sum(k) / len(k)
        bytes_ = kern_kib * 1024.0 * factor
        res[counter.lower()] = {"kernel_kib_per_dispatch": kern_kib, "dispatches": len(k),
                                "copy_kib_per_dispatch": copy_kib, "copy_true_bytes": a.copy_bytes,
                                "scale": factor, "bytes_per_launch": bytes_}
        total += bytes_
    res["hbm_bytes_per_launch"] = total
    res["algorithmic_bytes_per_launch"] = a.algorithmic_bytes
    res["traffic_over_algorithmic"] = total / a.algorithmic_bytes if a.algorithmic_bytes else None
    print(json.dumps(res, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="")
    t.add_argument("--tail", action="append", help="NAME:N[:M], statistics of the last N dispatches "
                   "after leaving out the last M")
    t.add_argument("--notes", help="text file appended to the summary")
    p = sub.add_parser("pmc")
    for k in ("fetch", "write", "kernel", "copy", "workload", "source", "command"):
        p.add_argument("--" + k, required=True)
    p.add_argument("--copy-bytes", type=int, required=True)
    p.add_argument("--algorithmic-bytes", type=int, default=0)
    p.add_argument("--tail", type=int, default=0, help="only the kernel's last N dispatches")
    q = sub.add_parser("sq")
    q.add_argument("db")
    q.add_argument("--kernel", action="append", required=True, help="kernel name substring (repeatable)")
    q.add_argument("--cu-num", type=int, default=256)
    q.add_argument("--simd-num", type=int, default=1024)
    q.add_argument("--tail", type=int, default=0, help="only each kernel's last N dispatches")
    q.add_argument("--skip-last", type=int, default=0, help="leave out each kernel's last M dispatches first")
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "pmc": cmd_pmc, "sq": cmd_sq}[a.cmd](a)


if __name__ == "__main__":
    main()
