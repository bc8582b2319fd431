"""Turn rocprofv3 result databases of a bench.py run into the short text
summaries kept under profiles/.

    python rocprof_summary.py stats --db KT.db --workload llama8b --cmd "..." [--out NAME.md]
    python rocprof_summary.py pmc --fetch-db F.db --write-db W.db --workload llama8b \
        --cmd-fetch "..." --cmd-write "..." [--bench-json B.json]
    python rocprof_summary.py sq --db S1.db --cmd "..." [--db S2.db --cmd "..."] --workload llama8b

`stats` summarises a `--kernel-trace --stats` run: every kernel's call count
and duration, and the split-K decode kernel's per-dispatch spread.  `pmc`
turns the FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch) into HBM bytes
per split-K launch, calibrated by the same counters on the copy probe of the
same run, which moves exactly 1 GiB each way per launch.  The record carries
the hash of the decode kernel's sources, so bench.py ignores it once the
kernel has changed.  `sq` records the split-K kernel's SQ counters per
dispatch (wave cycles, waits, VALU / LDS activity, LDS bank conflicts) and
their ratios.  Every summary names the rocprofv3 command and this script's
own invocation.
"""
import argparse
import collections
import json
import os
import shlex
import sqlite3
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
DECODE = "decode_partials_kernel"
COPY = "probe_copy_kernel"
COPY_BYTES = 1 << 30


def invocation():
    """This script's command line, as run from the repository root."""
    return "python rocprof_summary.py " + shlex.join(sys.argv[1:])


def short(name):
    """Kernel name without namespace, return type and argument list."""
    name = name.replace("ada::(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    if "(" in name:
        name = name[: name.index("(")]
    return name if len(name) < 80 else name[:77] + "..."


def per_kernel_durations(db):
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    agg = collections.defaultdict(list)
    for name, d in rows:
        agg[name].append(d)
    return agg


def per_kernel_counter(db, counter):
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, value from counters_collection where counter_name=?",
                       (counter,)).fetchall()
    per_dispatch = collections.defaultdict(lambda: collections.defaultdict(float))
    for name, did, v in rows:
        per_dispatch[name][did] += v      # a counter may arrive split over dimensions
    return {k: list(d.values()) for k, d in per_dispatch.items()}


def pick(agg, key):
    hits = [k for k in agg if key in k]
    if not hits:
        raise SystemExit(f"no kernel matching {key!r} in the database")
    return hits


def cmd_stats(a):
    agg = per_kernel_durations(a.db)
    total = sum(sum(v) for v in agg.values())
    lines = [f"# rocprofv3 kernel trace: {a.workload}", "", "Commands (from the repository root): the profiled",
             "run, then the summary of its database:", "",
             "```", a.cmd, invocation(), "```", "",
             "| kernel | calls | total ms | avg us | % |", "|---|---:|---:|---:|---:|"]
    for name, d in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{short(name)}` | {len(d)} | {sum(d) / 1e6:.3f} | {sum(d) / len(d) / 1e3:.2f} | "
                     f"{100 * sum(d) / total:.1f} |")
    focus = a.kernel or DECODE
    lines += ["", f"`{focus}`, per dispatch (us):", ""]
    for name in pick(agg, focus):
        d = agg[name]
        lines.append(f"- `{short(name)}`: n={len(d)} mean={statistics.mean(d) / 1e3:.2f} "
                     f"median={statistics.median(d) / 1e3:.2f} min={min(d) / 1e3:.2f} max={max(d) / 1e3:.2f}")
    out = os.path.join(PROFILES, a.out or f"ada_decode_partials_{a.workload}_kernel_stats.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def cmd_pmc(a):
    import bench
    fetch = per_kernel_counter(a.fetch_db, "FETCH_SIZE")
    write = per_kernel_counter(a.write_db, "WRITE_SIZE")
    cf = statistics.mean(fetch[pick(fetch, COPY)[0]])
    cw = statistics.mean(write[pick(write, COPY)[0]])
    f_scale = COPY_BYTES / (cf * 1024)
    w_scale = COPY_BYTES / (cw * 1024)
    kn = pick(fetch, DECODE)[0]
    fk = statistics.mean(fetch[kn])
    wk = statistics.mean(write[pick(write, DECODE)[0]])
    rec = {
        "kernel": short(kn),
        "workload": a.workload,
        "kernel_source_hash": bench.kernel_source_hash(),
        "fetch_kib_per_dispatch": fk,
        "write_kib_per_dispatch": wk,
        "dispatches": len(fetch[kn]),
        "copy_probe_fetch_kib": cf,
        "copy_probe_write_kib": cw,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_read_bytes_per_launch": fk * 1024 * f_scale,
        "hbm_write_bytes_per_launch": wk * 1024 * w_scale,
        "hbm_bytes_per_launch": (fk * 1024 * f_scale) + (wk * 1024 * w_scale),
        "cmd_fetch": a.cmd_fetch,
        "cmd_write": a.cmd_write,
        "summary_cmd": invocation(),
    }
    if a.bench_json:
        with open(a.bench_json) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        rec["algorithmic_bytes_per_launch"] = b["roofline"]["algorithmic_bytes"]
        rec["traffic_over_algorithmic"] = rec["hbm_bytes_per_launch"] / b["roofline"]["algorithmic_bytes"]
    out = os.path.join(PROFILES, f"ada_decode_partials_{a.workload}_pmc.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(out)
    print(json.dumps(rec, indent=1))


def cmd_traffic(a):
    """HBM bytes per dispatch of every kernel in one command's FETCH_SIZE and
    WRITE_SIZE passes, scaled by the copy probe's counters from the passes
    of a decode run on the same box."""
    cf = statistics.mean(per_kernel_counter(a.calib_fetch_db, "FETCH_SIZE")[
        pick(per_kernel_counter(a.calib_fetch_db, "FETCH_SIZE"), COPY)[0]])
    cw = statistics.mean(per_kernel_counter(a.calib_write_db, "WRITE_SIZE")[
        pick(per_kernel_counter(a.calib_write_db, "WRITE_SIZE"), COPY)[0]])
    f_scale, w_scale = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    fetch = per_kernel_counter(a.fetch_db, "FETCH_SIZE")
    write = per_kernel_counter(a.write_db, "WRITE_SIZE")
    lines = [f"# HBM traffic per dispatch: {a.title}", "", "Commands (from the repository root): the profiled",
             "runs, then the summary of their databases:", "",
             "```", a.cmd_fetch, a.cmd_write, a.cmd_calib, invocation(), "```", "",
             f"Counter scale from the copy probe of {COPY_BYTES / 2**30:.0f} GiB: FETCH_SIZE x {f_scale:.4f}, "
             f"WRITE_SIZE x {w_scale:.4f}.", "",
             "| kernel | dispatches | read MB | write MB |", "|---|---|---|---|"]
    rows = []
    for k in fetch:
        fm = statistics.mean(fetch[k]) * 1024 * f_scale / 1e6
        wm = statistics.mean(write.get(k, [0.0])) * 1024 * w_scale / 1e6
        rows.append((fm + wm, short(k), len(fetch[k]), fm, wm))
    for _, name, n, fm, wm in sorted(rows, reverse=True):
        lines.append(f"| `{name}` | {n} | {fm:.1f} | {wm:.1f} |")
    out = os.path.join(PROFILES, a.out)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)
    print("\n".join(lines))


def counter_names(db):
    con = sqlite3.connect(db)
    return [r[0] for r in con.execute("select distinct counter_name from counters_collection").fetchall()]


def cmd_sq(a):
    """SQ counters of the split-K kernel, per dispatch, from one or more
    passes (one database each), and the usual ratios."""
    import bench
    rec = {"workload": a.workload, "kernel_source_hash": bench.kernel_source_hash(), "per_dispatch": {}}
    kn = None
    for db in a.db:
        for c in counter_names(db):
            vals = per_kernel_counter(db, c)
            kn = pick(vals, DECODE)[0]
            rec["per_dispatch"][c] = statistics.mean(vals[kn])
            rec["dispatches"] = len(vals[kn])
    if kn is None:
        raise SystemExit("no counters in the databases")
    rec["kernel"] = short(kn)
    d = rec["per_dispatch"]
    cyc = d.get("SQ_WAVE_CYCLES")
    if cyc:
        for c, key in (("SQ_WAIT_ANY", "wait_any_over_wave_cycles"),
                       ("SQ_ACTIVE_INST_VALU", "valu_active_over_wave_cycles"),
                       ("SQ_ACTIVE_INST_LDS", "lds_active_over_wave_cycles")):
            if c in d:
                rec[key] = d[c] / cyc
    if d.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in d:
        rec["lds_bank_conflict_cycles_per_lds_inst"] = d["SQ_LDS_BANK_CONFLICT"] / d["SQ_INSTS_LDS"]
    if d.get("SQ_WAVES"):
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_MFMA"):
            if c in d:
                rec[c.lower().replace("sq_insts_", "insts_") + "_per_wave"] = d[c] / d["SQ_WAVES"]
    rec["cmds"] = a.cmd
    rec["summary_cmd"] = invocation()
    out = os.path.join(PROFILES, f"ada_decode_partials_{a.workload}_sq.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(out)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--db", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", help="summary file name under profiles/")
    s.add_argument("--kernel", help="kernel whose per-dispatch spread is listed (default: the split-K decode)")
    t = sub.add_parser("traffic")
    for k in ("fetch-db", "write-db", "calib-fetch-db", "calib-write-db", "cmd-fetch", "cmd-write", "cmd-calib",
              "title", "out"):
        t.add_argument("--" + k, required=True)
    p = sub.add_parser("pmc")
    p.add_argument("--fetch-db", required=True)
    p.add_argument("--write-db", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--cmd-fetch", required=True)
    p.add_argument("--cmd-write", required=True)
    p.add_argument("--bench-json")
    q = sub.add_parser("sq")
    q.add_argument("--db", required=True, action="append", help="one database per counter pass")
    q.add_argument("--workload", required=True)
    q.add_argument("--cmd", required=True, action="append", help="the profiled command of each pass")
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "pmc": cmd_pmc, "sq": cmd_sq}[a.mode](a)


if __name__ == "__main__":
    main()
