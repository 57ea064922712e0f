"""Summaries of rocprofv3 CSV output for the profiles folder.

``trace``: the kernel statistics of a ``rocprofv3 --kernel-trace --stats``
run (``*_kernel_stats.csv``) as a Markdown table of this library's kernels.

``traffic``: per-dispatch HBM bytes of this library's kernels from two
``rocprofv3 --pmc`` runs of the same command, one with ``FETCH_SIZE`` and one
with ``WRITE_SIZE`` (KiB per dispatch).  Both counters are scaled by what they
read for a reference dispatch of known size: the largest elementwise multiply
of an fp32 buffer (``bench.py --copy-mb N`` runs one over N MiB, reading and
writing N MiB).  Writes a Markdown table and the JSON that ``bench.py`` reads
for ``roofline.traffic`` (only while the recorded kernel-source hash matches).

``counters``: one ``rocprofv3 --pmc`` run with several instruction
counters (``SQ_INSTS_VALU`` and the like, summed over the device per
dispatch) as a table of per-dispatch means, with the decode's vector-ALU
instructions per 2-bit code (lanes per wave times ``SQ_INSTS_VALU`` over the
codes one launch dequantizes, ``--codes``).

Usage (from the repository root)::

    python -m bit_kv_cache_decode_amd.rocprof_summary trace STATS_CSV \\
        --workload NAME --command CMD [--note TEXT] -o OUT.md
    python -m bit_kv_cache_decode_amd.rocprof_summary traffic FETCH_CSV WRITE_CSV \\
        --workload NAME --copy-mb N --fetch-command CMD --write-command CMD \\
        -o OUT.md --json OUT.json
    python -m bit_kv_cache_decode_amd.rocprof_summary counters CSV --workload NAME \
        --command CMD --codes N [--kernel NAME] -o OUT.md
"""

import argparse
import collections
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(HERE, "csrc", "kivi_kernels.hip")
DECODE = "decode_kernel<2, 32, false, 2, false, false>"
STEP = "decode_kernel<2, 32, true, 2, false, false>"


def kernel_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short_name(name):
    """Drop namespaces; turn a mangled name into its identifier."""
    m = re.match(r"_ZN4kivi12_GLOBAL__N_1(\d+)(\w+)", name)
    if m:
        n = int(m.group(1))
        return m.group(2)[:n]
    return name.replace("kivi::(anonymous namespace)::", "")


def ours(name):
    return "kivi" in name


def trace(args):
    rows = list(csv.DictReader(open(args.csv)))
    lines = [f"# Kernel durations, workload {args.workload}", "",
             "Command (repository root, one MI355X):", "", "```", args.command, "```", "",
             f"Kernel source sha256: `{kernel_hash()}`", "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        if ours(r["Name"]):
            lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                         f"{r['MinNs']} | {r['MaxNs']} |")
    if args.note:
        lines += ["", args.note]
    open(args.out, "w").write("\n".join(lines) + "\n")


def _per_kernel(path):
    """{kernel name: [counter value of each dispatch]} and the largest fp32
    elementwise multiply dispatch (grid size, value)."""
    agg = collections.defaultdict(list)
    ref = (0, None)
    for r in csv.DictReader(open(path)):
        name, val = r["Kernel_Name"], float(r["Counter_Value"])
        agg[name].append(val)
        if "MulFunctor<float>" in name and int(r["Grid_Size"]) > ref[0]:
            ref = (int(r["Grid_Size"]), val)
    if ref[1] is None:
        raise SystemExit(f"{path}: no fp32 multiply dispatch to scale by (run with --copy-mb)")
    return agg, ref[1]


def traffic(args):
    fetch, fref = _per_kernel(args.fetch_csv)
    write, wref = _per_kernel(args.write_csv)
    ref_bytes = args.copy_mb << 20
    fscale = ref_bytes / (fref * 1024)
    wscale = ref_bytes / (wref * 1024)
    lines = [f"# HBM traffic per dispatch, workload {args.workload}", "",
             "Commands (repository root, one MI355X, one pass per counter):", "", "```",
             args.fetch_command, args.write_command, "```", "",
             f"Kernel source sha256: `{kernel_hash()}`", "",
             f"Reference dispatch: the elementwise multiply of a {args.copy_mb} MiB fp32 buffer "
             f"({ref_bytes} bytes read, {ref_bytes} written).",
             f"FETCH_SIZE reads {fref:.1f} KiB for it (scale factor {fscale:.3f}); WRITE_SIZE reads "
             f"{wref:.1f} KiB (scale factor {wscale:.3f}).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
             "|---|---:|---:|---:|---:|---:|"]
    per = {}
    for name, vals in fetch.items():
        if not ours(name) or name not in write:
            continue
        f = sum(vals) / len(vals)
        w = sum(write[name]) / len(write[name])
        rd, wr = f * 1024 * fscale, w * 1024 * wscale
        per[short_name(name)] = (rd, wr, f, w)
        lines.append(f"| {short_name(name)} | {len(vals)} | {f:.1f} | {w:.1f} | {rd / 1e6:.3f} | "
                     f"{wr / 1e6:.3f} |")
    open(args.out, "w").write("\n".join(lines) + "\n")

    def find(key):
        for n, v in per.items():
            if key in n:
                return v
        return None

    dec, step = find(DECODE), find(STEP)
    if dec is None:
        raise SystemExit(f"no {DECODE} dispatch in the counter runs")
    out = {"kernel_source_sha256": kernel_hash(), "workload": args.workload,
           "bytes_per_launch": int(round(dec[0] + dec[1])),
           "read_bytes_per_launch": int(round(dec[0])), "write_bytes_per_launch": int(round(dec[1])),
           "fetch_size_kib": dec[2], "write_size_kib": dec[3],
           "fetch_scale": fscale, "write_scale": wscale,
           "commands": [args.fetch_command, args.write_command]}
    if step is not None:
        out.update({"step_bytes_per_launch": int(round(step[0] + step[1])),
                    "step_read_bytes_per_launch": int(round(step[0])),
                    "step_write_bytes_per_launch": int(round(step[1]))})
    with open(args.json, "w") as f:
        json.dump(out, f, indent=1)


def counters(args):
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    names = []
    rows = [r for r in csv.DictReader(open(args.csv)) if ours(r["Kernel_Name"])]
    grids = collections.defaultdict(set)
    for r in rows:
        grids[r["Kernel_Name"]].add(r["Grid_Size"])
    for r in rows:
        c = r["Counter_Name"]
        if c not in names:
            names.append(c)
        key = short_name(r["Kernel_Name"])
        if len(grids[r["Kernel_Name"]]) > 1:  # one row per launch shape
            key += f" [{int(r['Grid_Size']) // int(r['Workgroup_Size'])} workgroups]"
        per[key][c].append(float(r["Counter_Value"]))
    lines = [f"# Instruction counters per dispatch, workload {args.workload}", "",
             "Command (repository root, one MI355X):", "", "```", args.command, "```", "",
             f"Kernel source sha256: `{kernel_hash()}`", "",
             "| kernel | dispatches | " + " | ".join(names) + " |",
             "|---|---:|" + "---:|" * len(names)]
    for k, cs in per.items():
        n = len(next(iter(cs.values())))
        cells = [f"{sum(cs[c]) / len(cs[c]):.4g}" if cs.get(c) else "-" for c in names]
        lines.append(f"| {k} | {n} | " + " | ".join(cells) + " |")
    dec = next((cs for k, cs in per.items() if args.kernel in k), None)
    if dec is not None and "SQ_INSTS_VALU" in dec and args.codes:
        valu = sum(dec["SQ_INSTS_VALU"]) / len(dec["SQ_INSTS_VALU"])
        lines += ["", f"{args.kernel}: {valu:.4g} wave-level VALU instructions per dispatch, "
                      f"{64 * valu / args.codes:.3f} lane-level VALU instructions per code "
                      f"({args.codes} codes per launch)."]
        if "SQ_WAVES" in dec:
            w = sum(dec["SQ_WAVES"]) / len(dec["SQ_WAVES"])
            lines.append(f"{w:.0f} waves per dispatch, {valu / w:.0f} VALU instructions per wave.")
    if args.note:
        lines += ["", args.note]
    open(args.out, "w").write("\n".join(lines) + "\n")


def main():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = p.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--note", default="")
    t.add_argument("-o", "--out", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch_csv")
    c.add_argument("write_csv")
    c.add_argument("--workload", required=True)
    c.add_argument("--copy-mb", type=int, required=True)
    c.add_argument("--fetch-command", required=True)
    c.add_argument("--write-command", required=True)
    c.add_argument("-o", "--out", required=True)
    c.add_argument("--json", required=True)
    n = sub.add_parser("counters")
    n.add_argument("csv")
    n.add_argument("--workload", required=True)
    n.add_argument("--command", required=True)
    n.add_argument("--codes", type=int, default=0)
    n.add_argument("--kernel", default=DECODE,
                   help="kernel (name substring) the per-code figure is for")
    n.add_argument("--note", default="")
    n.add_argument("-o", "--out", required=True)
    a = p.parse_args()
    {"trace": trace, "traffic": traffic, "counters": counters}[a.mode](a)


if __name__ == "__main__":
    main()
