"""Turn rocprofv3 CSV output of the benchmark into the short summaries kept
under profiles/.

    # per-kernel durations (rocprofv3 --kernel-trace --stats --output-format csv)
    python -m speculative_decoding_verify_dspk_amd.profile_summary stats \\
        <kernel_stats.csv> <kernel_trace.csv> <out.md> --cmd "<profiled command>"

    # per-width launch durations of the verify rounds (rocprofv3 --kernel-trace)
    python -m speculative_decoding_verify_dspk_amd.profile_summary rounds \\
        <kernel_trace.csv> <out.md> --sweep 1,8,16 --cmd "<profiled command>"

    # t(M) per projection and decomposition (trace of bench.py --variant-curves)
    python -m speculative_decoding_verify_dspk_amd.profile_summary curves \\
        <kernel_trace.csv> <curves.json> <out.md> --cmd "<profiled command>"

    # per-launch SQ counters of one kernel (one or more --pmc passes)
    python -m speculative_decoding_verify_dspk_amd.profile_summary counters <out.md> \\
        --csv <pass1 counter_collection.csv> --cmd "<pass1>" [--csv ... --cmd ...] \\
        --kernel prefill_kernel --title "<title>"

    # HBM bytes of the head kernel (two --pmc passes: FETCH_SIZE, WRITE_SIZE),
    # scaled by what the same counters read for a plain 256 MiB device copy
    python -m speculative_decoding_verify_dspk_amd.profile_summary traffic \\
        <fetch counter_collection.csv> <write counter_collection.csv> <out.txt> --cmd "<...>"
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# sources of the head kernel (their concatenation is hashed)
KERNEL_SRCS = [os.path.join(PKG, "csrc", f) for f in ("qgemm.hip", "decode.h", "dspk_internal.h")]
COPY_BYTES = 256 << 20          # the calibration copy that bench.py --calibrate runs


def short(name: str) -> str:
    for k in ("qgemm_slab_lds_kernel", "qgemm_slab_kernel", "qgemm_kernel", "prefill_kernel"):
        if k + "<" in name:
            return k + "<" + name.split(k + "<", 1)[1].split(">", 1)[0] + ">"
    m = re.search(r"accept_\w+", name)
    if m:
        return m.group(0)
    return (name[:70] + "...") if len(name) > 73 else name


def stats(stats_csv: str, trace_csv: str, out: str, cmd: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# Kernel durations: benchmark verify rounds", "", "Command:", "", "    " + cmd, "",
             "| kernel | calls | average us | total % |", "|---|---|---|---|"]
    for r in rows[:12]:
        lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    # per-launch split of the projection kernels by grid (one line per launch shape)
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        if "qgemm" in r["Kernel_Name"] or "prefill_kernel" in r["Kernel_Name"]:
            per[(short(r["Kernel_Name"]), r["Grid_Size_X"], r.get("Grid_Size_Y", "1"),
                 r.get("Grid_Size_Z", "1"))].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "Projection launches by grid (threads in x, workgroups in y and z; the prefill kernel's z is "
              "its K split):", "",
              "| kernel | grid x | grid y | grid z | launches | median us |", "|---|---|---|---|---|---|"]
    for (k, gx, gy, gz), v in sorted(per.items()):
        v.sort()
        lines.append(f"| {k} | {gx} | {gy} | {gz} | {len(v)} | {v[len(v) // 2]:.1f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def _dspk_launches(trace_csv: str):
    rows = [r for r in csv.DictReader(open(trace_csv)) if "dspk::" in r["Kernel_Name"]
            and "qgemm" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return rows


def _us(r) -> float:
    return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3


def rounds(trace_csv: str, out: str, cmd: str, sweep: list, title: str) -> None:
    """Per-width launch durations of the benchmark's verify rounds: each round
    is its layer's four projection launches followed by the head launch; the
    timed rounds cycle through the sweep, so the last whole cycles of the trace
    are the rounds at each width in sweep order."""
    rows = _dspk_launches(trace_csv)
    rds, cur = [], []
    for r in rows:
        cur.append(r)
        if "qgemm_kernel<" in r["Kernel_Name"] and ", true>" in r["Kernel_Name"]:
            if len(cur) >= 5:
                rds.append(cur[-5:])
            cur = []
    n = len(rds) // len(sweep) * len(sweep)
    rds = rds[len(rds) - n:]
    names = ["qkv", "o", "gate/up", "down", "head"]
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    kern = collections.defaultdict(dict)
    for i, rd in enumerate(rds):
        m = sweep[i % len(sweep)]
        for nm, r in zip(names, rd):
            per[m][nm].append(_us(r))
            kern[m][nm] = short(r["Kernel_Name"])
    med = lambda v: sorted(v)[len(v) // 2]   # noqa: E731
    lines = [f"# {title}", "", "Command:", "", "    " + cmd, "",
             f"Median kernel durations (us) over {n // len(sweep)} rounds per width (rocprofv3 kernel trace):", "",
             "| rows | " + " | ".join(names) + " | layer (4 launches) |", "|---" * (len(names) + 2) + "|"]
    for m in sweep:
        v = [med(per[m][nm]) for nm in names]
        lines.append(f"| {m} | " + " | ".join(f"{x:.2f}" for x in v) + f" | {sum(v[:4]):.2f} |")
    lines += ["", "Kernels per launch:", ""]
    for m in sweep:
        lines.append(f"- {m} rows: " + ", ".join(f"{nm} `{kern[m][nm]}`" for nm in names))
    open(out, "w").write("\n".join(lines) + "\n")


def curves(trace_csv: str, curves_json: str, out: str, cmd: str) -> None:
    """t(M) per projection and forced decomposition from the kernel trace of
    `bench.py --variant-curves`: its JSON line lists the launches in order
    (projection, variant, rows, launches, the first `warmup` untimed)."""
    import json
    plan = json.loads(open(curves_json).read().strip().splitlines()[-1])
    rows = _dspk_launches(trace_csv)
    pos = 0
    table = collections.defaultdict(dict)
    kern = {}
    for pname, vname, m, count in plan["launch_plan"]:
        blk = rows[pos:pos + count]
        pos += count
        d = sorted(_us(r) for r in blk[count // 8:])        # the warm-up launches come first
        table[(pname, vname)][m] = d[len(d) // 2]
        kern[(pname, vname)] = short(blk[-1]["Kernel_Name"])
    if pos != len(rows):
        raise SystemExit(f"trace has {len(rows)} projection launches, the plan {pos}")
    widths = sorted({m for v in table.values() for m in v})
    lines = ["# Projection launch time t(M) by decomposition (Qwen3-4B shapes, 8-bit)", "", "Command:", "",
             "    " + cmd, "",
             "Median kernel duration (us, rocprofv3 kernel trace) of each launch shape at each width;",
             "`mfma_*` reduce K on the matrix cores (bf16 16x16x32, rows padded to 16), `dot_slab` on the",
             "vector ALUs (v_dot2_f32_bf16, at most 4 rows), with the same decomposition and data movement",
             "as `mfma_slab`.", "",
             "| projection | variant | kernel | " + " | ".join(f"M={m}" for m in widths) + " |",
             "|---|---|---|" + "---|" * len(widths)]
    for (pname, vname), c in table.items():
        lines.append(f"| {pname} | {vname} | `{kern[(pname, vname)]}` | " +
                     " | ".join(f"{c[m]:.2f}" if m in c else "" for m in widths) + " |")
    open(out, "w").write("\n".join(lines) + "\n")


def counter_means(path: str, counter: str) -> dict:
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def traffic(fetch_csv: str, write_csv: str, out: str, cmd_fetch: str, cmd_write: str) -> None:
    res = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        per = counter_means(path, counter)
        # the calibration copy is the largest copy dispatch of the run (the
        # others are the rounds' small device-to-host copies)
        copy = max((v for k, vs in per.items() if "copyBuffer" in k for v in vs), default=0.0)
        head = [v for k, vs in per.items() if "qgemm_kernel" in k and "true>" in k for v in vs]
        if copy <= 0 or not head:
            raise SystemExit(f"{path}: calibration copy or head kernel missing")
        # bytes per counted KiB, from the copy that reads and writes COPY_BYTES once
        factor = COPY_BYTES / copy
        res[counter] = (sum(head) / len(head), factor)
    sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SRCS)).hexdigest()
    f_kib, f_fac = res["FETCH_SIZE"]
    w_kib, w_fac = res["WRITE_SIZE"]
    lines = [
        "# HBM traffic of the vocabulary-head kernel (qgemm_kernel<8,MT,true>), per launch",
        "# Commands (one counter per run):",
        "#   " + cmd_fetch,
        "#   " + cmd_write,
        f"# FETCH_SIZE per head launch: {f_kib:.0f} KiB; a 256 MiB device copy reads as "
        f"{COPY_BYTES / f_fac:.0f} KiB -> scale {f_fac:.1f} bytes per counted KiB",
        f"# WRITE_SIZE per head launch: {w_kib:.0f} KiB; the same copy writes as "
        f"{COPY_BYTES / w_fac:.0f} KiB -> scale {w_fac:.1f} bytes per counted KiB",
        f"kernel_source_sha256={sha}",
        f"fetch_bytes_per_launch={f_kib * f_fac:.0f}",
        f"write_bytes_per_launch={w_kib * w_fac:.0f}",
    ]
    open(out, "w").write("\n".join(lines) + "\n")


def counters(csv_paths: list, out: str, cmds: list, kernel: str, title: str) -> None:
    """Per-launch means of SQ counters (rocprofv3 --pmc passes) of the
    launches of `kernel` with the largest grid, one row per counter."""
    vals = collections.defaultdict(list)
    for path in csv_paths:
        rows = [r for r in csv.DictReader(open(path)) if kernel in r["Kernel_Name"]]
        if not rows:
            raise SystemExit(f"{path}: no {kernel} launches")
        big = max(int(r["Grid_Size"]) for r in rows)
        for r in rows:
            if int(r["Grid_Size"]) == big:
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# {title}", "", "Commands (one --pmc pass each):", ""] + ["    " + c for c in cmds] + [
        "", f"Mean per launch of the largest-grid `{kernel}` launches (sums over the device):", "",
        "| counter | value |", "|---|---|"]
    for name in sorted(vals):
        v = vals[name]
        lines.append(f"| {name} | {sum(v) / len(v):.0f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("stats_csv")
    a.add_argument("trace_csv")
    a.add_argument("out")
    a.add_argument("--cmd", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("out")
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    c = sub.add_parser("rounds")
    c.add_argument("trace_csv")
    c.add_argument("out")
    c.add_argument("--cmd", required=True)
    c.add_argument("--sweep", required=True)
    c.add_argument("--title", default="Verify-round launch durations by width")
    d = sub.add_parser("curves")
    d.add_argument("trace_csv")
    d.add_argument("curves_json")
    d.add_argument("out")
    d.add_argument("--cmd", required=True)
    e = sub.add_parser("counters")
    e.add_argument("out")
    e.add_argument("--csv", action="append", required=True)
    e.add_argument("--cmd", action="append", required=True)
    e.add_argument("--kernel", required=True)
    e.add_argument("--title", required=True)
    args = ap.parse_args()
    if args.what == "counters":
        counters(args.csv, args.out, args.cmd, args.kernel, args.title)
    elif args.what == "stats":
        stats(args.stats_csv, args.trace_csv, args.out, args.cmd)
    elif args.what == "rounds":
        rounds(args.trace_csv, args.out, args.cmd, [int(x) for x in args.sweep.split(",")], args.title)
    elif args.what == "curves":
        curves(args.trace_csv, args.curves_json, args.out, args.cmd)
    else:
        traffic(args.fetch_csv, args.write_csv, args.out, args.cmd_fetch, args.cmd_write)


if __name__ == "__main__":
    main()
