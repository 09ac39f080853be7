"""Text summaries of rocprofv3 output for the profiles/ folder.

  python rocprof_summary.py stats DIR --cmd CMD --title T --out FILE.md
      kernel time table from DIR/*_kernel_stats.csv (--kernel-trace --stats)
  python rocprof_summary.py traffic FETCH_DIR WRITE_DIR --workload W --cmd-fetch C
          --cmd-write C --out-md FILE.md --out-json FILE.json
      HBM bytes per launch from FETCH_SIZE / WRITE_SIZE passes (KiB per
      dispatch), each scaled by what the same counter reads for the 256 MiB
      device copy that `bench.py --copy-calibration` runs first
  python rocprof_summary.py counters DIR... --cmd C... --title T --out FILE.md
      SQ counter ratios per kernel (MFMA busy, VALU co-execution, LDS bank
      conflicts, transcendental share) from --pmc passes
  python rocprof_summary.py compare DIR... --label L... --cmd C... --title T --out FILE.md
      average kernel durations of several --kernel-trace --stats runs side by side
  python rocprof_summary.py pmc DIR... --label L... --cmd C... --title T --out FILE.md
      raw per-kernel --pmc averages (with the L2 hit rate and the share of
      atomics sent on to memory when those counters are present)

Only the attention kernels (names in namespace fa::) and the calibration copy
are reported.  The JSON written by `traffic` carries a hash of the kernel
sources and build flags; bench.py reports the stored traffic only while that
hash matches the sources it runs.
"""
import argparse
import collections
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 256 * 1024 * 1024   # bench.py --copy-calibration: 64 Mi floats
NUM_XCD = 8
NUM_SIMD = 256 * 4


def short_name(kernel):
    name = kernel.split("(")[0]
    return name[5:] if name.startswith("void ") else name


def wanted(kernel):
    return "fa::" in kernel or COPY_KERNEL in kernel


def one_csv(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits[0]


def counter_rows(d):
    """{(kernel, counter): [value per dispatch]} and {kernel: [duration ns]}."""
    vals = collections.defaultdict(list)
    durs = collections.defaultdict(dict)
    with open(one_csv(d, "_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if not wanted(r["Kernel_Name"]):
                continue
            k = short_name(r["Kernel_Name"])
            vals[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
            durs[k][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return vals, {k: list(v.values()) for k, v in durs.items()}


def mean(x):
    return sum(x) / len(x)


def cmd_stats(a):
    rows = []
    with open(one_csv(a.dir, "_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            if "fa::" in r["Name"]:
                rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                             float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                             float(r["TotalDurationNs"])))
    total = sum(r[5] for r in rows)
    out = [f"# {a.title}", "", "Command (from the repository root, on one MI355X):", "", "```",
           "export TMPDIR=/tmp", a.cmd, "```", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share of attention-kernel time |",
           "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, tot in sorted(rows, key=lambda r: -r[5]):
        out.append(f"| `{name}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {100 * tot / total:.1f}% |")
    if a.note:
        out += ["", a.note]
    write(a.out, out)


def cmd_compare(a):
    """Average kernel durations of several --kernel-trace --stats runs side by
    side (one column per labelled run)."""
    runs = []
    for d in a.dirs:
        avg = {}
        with open(one_csv(d, "_kernel_stats.csv")) as f:
            for r in csv.DictReader(f):
                if "fa::" in r["Name"]:
                    avg[short_name(r["Name"])] = float(r["AverageNs"]) / 1e3
        runs.append(avg)
    names = sorted(set().union(*runs), key=lambda k: -runs[0].get(k, 0))
    out = [f"# {a.title}", "", "Commands (from the repository root, on one MI355X):", "", "```",
           "export TMPDIR=/tmp"] + a.cmd + ["```", "",
           "| kernel | " + " | ".join(f"{l} average (us)" for l in a.label) +
           (f" | {a.label[1]} / {a.label[0]}" if len(runs) == 2 else "") + " |",
           "|---|" + "---|" * (len(runs) + (1 if len(runs) == 2 else 0))]
    for k in names:
        vals = [r.get(k) for r in runs]
        cells = " | ".join("-" if v is None else f"{v:.1f}" for v in vals)
        ratio = (f" | {vals[1] / vals[0]:.2f}x" if len(runs) == 2 and None not in vals else
                 (" | -" if len(runs) == 2 else ""))
        out.append(f"| `{k}` | {cells}{ratio} |")
    if a.note:
        out += ["", a.note]
    write(a.out, out)


def cmd_pmc(a):
    """Per-kernel averages of raw --pmc counters (one or more labelled runs),
    with the L2 hit rate when TCC_HIT_sum / TCC_MISS_sum are present and the
    share of L2 atomic requests sent on to memory when TCC_ATOMIC_sum /
    TCC_EA0_ATOMIC_sum are."""
    out = [f"# {a.title}", "", "Commands (from the repository root, on one MI355X):", "", "```",
           "export TMPDIR=/tmp"] + a.cmd + ["```", ""]
    for d, label in zip(a.dirs, a.label):
        vals, _ = counter_rows(d)
        per = collections.defaultdict(dict)
        for (k, c), v in vals.items():
            if k != COPY_KERNEL:
                per[k][c] = mean(v)
        counters = sorted({c for kv in per.values() for c in kv})
        extra = []
        if {"TCC_HIT_sum", "TCC_MISS_sum"} <= set(counters):
            extra.append(("L2 hit rate", lambda c: c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"]),
                          "{:.1%}"))
        if {"TCC_ATOMIC_sum", "TCC_EA0_ATOMIC_sum"} <= set(counters):
            extra.append(("atomics sent on to memory",
                          lambda c: c["TCC_EA0_ATOMIC_sum"] / c["TCC_ATOMIC_sum"] if c["TCC_ATOMIC_sum"] else 0.0,
                          "{:.1%}"))
        out += [f"## {label}", "", "| kernel | " + " | ".join(counters + [e[0] for e in extra]) + " |",
                "|---|" + "---|" * (len(counters) + len(extra))]
        for k in sorted(per):
            c = per[k]
            cells = [f"{c.get(n, float('nan')):.4g}" for n in counters]
            cells += [fmt.format(fn(c)) for _, fn, fmt in extra]
            out.append(f"| `{k}` | " + " | ".join(cells) + " |")
        out.append("")
    if a.note:
        out += [a.note]
    write(a.out, out)


def source_sha256():
    """Hash of the kernel sources and build flags the counters were taken
    with (bench.py's key for the stored traffic)."""
    sys.path.insert(0, ROOT)
    import bench
    return bench.source_sha256()


def dispatch_rows(d):
    """{(kernel, counter): [value per dispatch]} like counter_rows, with each
    backward preprocess dispatch (`bwd_pre_kernel`) named after the kernel
    dispatched right after it: the preprocess zeroes dQ only ahead of the
    atomic modes, so its bytes depend on the mode it serves."""
    rows = []
    with open(one_csv(d, "_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if wanted(r["Kernel_Name"]):
                rows.append((int(r["Dispatch_Id"]), short_name(r["Kernel_Name"]), r["Counter_Name"],
                             float(r["Counter_Value"])))
    rows.sort()
    order = []  # kernel name per dispatch, in dispatch order
    for disp, k, _, _ in rows:
        if not order or order[-1][0] != disp:
            order.append((disp, k))
    label = {}
    for i, (disp, k) in enumerate(order):
        nxt = order[i + 1][1] if i + 1 < len(order) else None
        label[disp] = f"{k} (before {nxt})" if "bwd_pre_kernel" in k and nxt else k
    vals = collections.defaultdict(list)
    for disp, _, c, v in rows:
        vals[(label[disp], c)].append(v)
    return vals


def cmd_traffic(a):
    fv = dispatch_rows(a.fetch_dir)
    wv = dispatch_rows(a.write_dir)
    f_copy = mean(fv[(COPY_KERNEL, "FETCH_SIZE")])
    w_copy = mean(wv[(COPY_KERNEL, "WRITE_SIZE")])
    ff = COPY_BYTES / (f_copy * 1024.0)
    wf = COPY_BYTES / (w_copy * 1024.0)
    kernels = sorted({k for k, c in fv if k != COPY_KERNEL and c == "FETCH_SIZE"})
    res = {}
    for k in kernels:
        fk, wk = fv.get((k, "FETCH_SIZE")), wv.get((k, "WRITE_SIZE"))
        if not fk or not wk:
            continue
        res[k] = {"read_bytes": mean(fk) * 1024 * ff, "write_bytes": mean(wk) * 1024 * wf,
                  "launches": min(len(fk), len(wk))}
    js = {"workload": a.workload, "source_sha256": source_sha256(),
          "calibration": {"kernel": COPY_KERNEL, "bytes_read_and_written": COPY_BYTES,
                          "fetch_size_kib": f_copy, "write_size_kib": w_copy,
                          "fetch_factor": ff, "write_factor": wf},
          "kernels": res}
    with open(a.out_json, "w") as f:
        json.dump(js, f, indent=1)
    mib = 1024.0 * 1024.0
    out = [f"# HBM traffic per launch, {a.workload}", "",
           "Counters in separate passes (one counter per run):", "", "```", "export TMPDIR=/tmp",
           a.cmd_fetch, a.cmd_write, "```", "",
           f"Calibration: the 256 MiB device-to-device copy (`{COPY_KERNEL}`) reads as FETCH_SIZE "
           f"{f_copy:.0f} KiB and WRITE_SIZE {w_copy:.0f} KiB, so bytes = FETCH_SIZE x {ff:.3f} KiB "
           f"and WRITE_SIZE x {wf:.3f} KiB.", "",
           "| kernel | launches | read (MiB) | written (MiB) |", "|---|---|---|---|"]
    for k, r in res.items():
        out.append(f"| `{k}` | {r['launches']} | {r['read_bytes'] / mib:.1f} | "
                   f"{r['write_bytes'] / mib:.1f} |")
    if a.note:
        out += ["", a.note]
    write(a.out_md, out)


DERIVED = [
    ("cycles per XCD", lambda c: c["GRBM_GUI_ACTIVE"] / NUM_XCD, "{:.0f}"),
    ("MFMA busy (share of SIMD cycles)",
     lambda c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / (NUM_SIMD * c["GRBM_GUI_ACTIVE"] / NUM_XCD), "{:.1%}"),
    ("VALU co-executing with MFMA (share of MFMA-busy cycles)",
     lambda c: c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"], "{:.1%}"),
    ("VALU instructions per MFMA", lambda c: (c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]) / c["SQ_INSTS_MFMA"],
     "{:.2f}"),
    ("transcendental share of VALU instructions",
     lambda c: c["SQ_INSTS_VALU_TRANS_F32"] / c["SQ_INSTS_VALU"], "{:.1%}"),
    ("LDS instructions per MFMA", lambda c: c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"], "{:.2f}"),
    ("LDS bank-conflict cycles / LDS active cycles",
     lambda c: c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"], "{:.2%}"),
    ("waves waiting on LDS data (share of wave cycles)",
     lambda c: c["SQ_WAIT_INST_LDS"] / c["SQ_WAVE_CYCLES"], "{:.1%}"),
    ("waves waiting on any dependency (share of wave cycles)",
     lambda c: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"], "{:.1%}"),
]


def cmd_counters(a):
    merged = collections.defaultdict(dict)
    durs = {}
    for d in a.dirs:
        vals, du = counter_rows(d)
        for (k, c), v in vals.items():
            if k != COPY_KERNEL:
                merged[k].setdefault(c, mean(v))
        for k, v in du.items():
            durs.setdefault(k, mean(v))
    out = [f"# {a.title}", "", "Counter passes (one pass per command, each within the per-block "
           "counter limits):", "", "```", "export TMPDIR=/tmp"] + a.cmd + ["```", ""]
    for k, c in sorted(merged.items()):
        out += [f"## `{k}`", "", f"Average duration under counter collection: "
                f"{durs.get(k, 0) / 1e3:.1f} us.", "", "| quantity | value |", "|---|---|"]
        for label, fn, fmt in DERIVED:
            try:
                out.append(f"| {label} | {fmt.format(fn(c))} |")
            except (KeyError, ZeroDivisionError):
                pass
        out += ["", "Raw per-dispatch averages: " + ", ".join(
            f"{n} {v:.4g}" for n, v in sorted(c.items())), ""]
    if a.note:
        out += [a.note]
    write(a.out, out)


def write(path, lines):
    with open(path, "w") as f:
        f.write("\n".join(lines).rstrip() + "\n")
    print("wrote", path)


def main():
    p = argparse.ArgumentParser()
    sp = p.add_subparsers(dest="mode", required=True)
    s = sp.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--out", required=True)
    t = sp.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--workload", required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--note", default="")
    t.add_argument("--out-md", required=True)
    t.add_argument("--out-json", required=True)
    c = sp.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    m = sp.add_parser("compare")
    m.add_argument("dirs", nargs="+")
    m.add_argument("--label", action="append", required=True)
    m.add_argument("--cmd", action="append", required=True)
    m.add_argument("--title", required=True)
    m.add_argument("--note", default="")
    m.add_argument("--out", required=True)
    q = sp.add_parser("pmc")
    q.add_argument("dirs", nargs="+")
    q.add_argument("--label", action="append", required=True)
    q.add_argument("--cmd", action="append", required=True)
    q.add_argument("--title", required=True)
    q.add_argument("--note", default="")
    q.add_argument("--out", required=True)
    a = p.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters, "compare": cmd_compare,
     "pmc": cmd_pmc}[a.mode](a)


if __name__ == "__main__":
    main()
