"""Turns rocprofv3 CSV output into the short text summaries kept with the code.

    python -m block_sparse_video_map_amd.profsum stats  DIR --title T --command C > out.md
    python -m block_sparse_video_map_amd.profsum traffic FETCH_DIR WRITE_DIR \
        --kernel attn_bf16_kernel --copy-mib 1024 --title T --command C > out.md

`stats` tabulates `run_kernel_stats.csv` (calls, average / min / max time per
kernel). `traffic` reads two `--pmc` runs (FETCH_SIZE, then WRITE_SIZE; both
in KiB per dispatch) of a program that ends with one plain device copy of
`--copy-mib` MiB, and scales each counter by what it reads for that copy
(copy bytes / counter value), so the figures are HBM bytes. The traffic
summary ends with one JSON comment line that bench.py reads; it carries a
hash of the kernel sources it was measured on, so a changed kernel reports
no traffic until it is measured again.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
# Sources whose text decides each attention kernel's memory traffic.
KERNEL_SOURCES = {
    "attn_bf16_kernel": ("csrc/attn_bf16.hip", "csrc/attn_pairs.h", "csrc/attn_common.h",
                         "csrc/device_common.h"),
    "attn_fp8_kernel": ("csrc/attn_fp8.hip", "csrc/attn_pairs.h", "csrc/attn_common.h",
                        "csrc/device_common.h", "csrc/fp8_layout.h"),
}


def source_hash(kernel: str = "attn_bf16_kernel") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(PKG, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    name = name.replace("vsa::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


def stats_table(d: str) -> list[str]:
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    out = ["| kernel | calls | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e6:.3f} | {float(r['MinNs']) / 1e6:.3f} | "
                   f"{float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}% |")
    return out


def _per_dispatch(d: str):
    rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
    acc: dict[int, list] = {}
    for r in rows:
        i = int(r["Dispatch_Id"])
        e = acc.setdefault(i, [r["Kernel_Name"], 0.0])
        e[1] += float(r["Counter_Value"])
    return [(i, acc[i][0], acc[i][1]) for i in sorted(acc)]


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_mib: int):
    f = _per_dispatch(fetch_dir)
    w = _per_dispatch(write_dir)
    copy_kib = copy_mib * 1024.0
    fc = [v for _, n, v in f if "copyBuffer" in n or "copy_kernel" in n]
    wc = [v for _, n, v in w if "copyBuffer" in n or "copy_kernel" in n]
    if not fc or not wc:
        raise SystemExit("no plain copy dispatch found in the counter runs")
    fetch_scale = copy_kib / fc[-1]
    write_scale = copy_kib / wc[-1]
    fk = [v for _, n, v in f if kernel in n]
    wk = [v for _, n, v in w if kernel in n]
    if not fk or not wk:
        raise SystemExit(f"kernel {kernel} not found in the counter runs")
    fetch_b = sum(fk) / len(fk) * fetch_scale * 1024
    write_b = sum(wk) / len(wk) * write_scale * 1024
    per_kernel = {}
    for (_, n, fv), (_, n2, wv) in zip(f, w):
        s = short_name(n)
        e = per_kernel.setdefault(s, [0, 0.0, 0.0])
        e[0] += 1
        e[1] += fv
        e[2] += wv
    return {"fetch_scale": fetch_scale, "write_scale": write_scale,
            "fetch_bytes": fetch_b, "write_bytes": write_b,
            "bytes_per_launch": fetch_b + write_b, "dispatches": len(fk),
            "per_kernel": per_kernel}


def counters(d: str, kernel: str):
    """Counter totals of the last dispatch of `kernel` in one --pmc run."""
    rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
    acc: dict = {}
    for r in rows:
        if kernel not in r["Kernel_Name"]:
            continue
        key = (int(r["Dispatch_Id"]), r["Counter_Name"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    if not acc:
        raise SystemExit(f"kernel {kernel} not found in {d}")
    last = max(k[0] for k in acc)
    return {c: v for (i, c), v in sorted(acc.items()) if i == last}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True, help="FETCH_SIZE command; WRITE_SIZE is the same")
    t.add_argument("--workload", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--note", default="")
    a = ap.parse_args(argv)
    lines = [f"# {a.title}", "", "Command (from the repository root on the GPU host):", "",
             "```", a.command, "```", ""]
    if a.cmd == "counters":
        if a.note:
            lines += [a.note, ""]
        lines += [f"Totals over one dispatch of `{a.kernel}` (all XCDs):", "",
                  "| counter | value |", "|---|---|"]
        for k, v in counters(a.dir, a.kernel).items():
            lines.append(f"| {k} | {v:.4g} |")
    elif a.cmd == "stats":
        if a.note:
            lines += [a.note, ""]
        lines += ["rocprofv3 `run_kernel_stats.csv`:", ""] + stats_table(a.dir)
    else:
        r = traffic(a.fetch_dir, a.write_dir, a.kernel, a.copy_mib)
        lines += [
            "The same command is run twice, with `--pmc FETCH_SIZE` and then `--pmc WRITE_SIZE`.",
            f"The program ends with one plain device copy of {a.copy_mib} MiB; each counter is",
            "scaled by (copy bytes / what it reads for that copy):", "",
            f"* FETCH_SIZE scale: {r['fetch_scale']:.4f}",
            f"* WRITE_SIZE scale: {r['write_scale']:.4f}", "",
            "Raw counters per kernel (KiB, summed over dispatches, unscaled):", "",
            "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|---|"]
        for n, (c, fv, wv) in r["per_kernel"].items():
            lines.append(f"| `{n}` | {c} | {fv:.1f} | {wv:.1f} |")
        lines += ["", f"`{a.kernel}`, per launch, scaled: fetch {r['fetch_bytes'] / 1e9:.3f} GB, "
                      f"write {r['write_bytes'] / 1e9:.3f} GB, total "
                      f"{r['bytes_per_launch'] / 1e9:.3f} GB.", ""]
        rec = {"kernel": a.kernel, "workload": a.workload,
               "bytes_per_launch": round(r["bytes_per_launch"]),
               "fetch_bytes": round(r["fetch_bytes"]), "write_bytes": round(r["write_bytes"]),
               "fetch_scale": round(r["fetch_scale"], 5), "write_scale": round(r["write_scale"], 5),
               "source_hash": source_hash(a.kernel)}
        lines.append(f"<!-- traffic: {json.dumps(rec)} -->")
    sys.stdout.write("\n".join(lines) + "\n")


def read_traffic(path: str, kernel: str, workload: str):
    """bytes per launch from a committed traffic summary, or None when the
    summary is missing, is for another kernel or workload, or was measured on
    different kernel sources."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"<!-- traffic: (\{.*\}) -->", text)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel") != kernel or rec.get("workload") != workload:
        return None
    if kernel not in KERNEL_SOURCES or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec


if __name__ == "__main__":
    main()
