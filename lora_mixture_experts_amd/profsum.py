"""Summaries of rocprofv3 output for the layer's kernels (profiling support).

Two modes, each writing one short markdown file:

  stats   from a `rocprofv3 --kernel-trace --stats --output-format csv` run:
          calls and average / min / max duration per kernel.
  counters  per-kernel averages of whatever counters one or more
          `rocprofv3 --pmc` runs collected (e.g. MFMA busy cycles, LDS bank
          conflicts, L2 hits and misses).
  traffic from two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a
          command that first streams a known number of bytes through HBM
          (bench.py --calibrate-copy MiB): the readings of that reference
          dispatch give the factors that turn each counter into bytes, and every
          kernel of the layer gets its scaled HBM bytes per dispatch.

The traffic file ends with a fenced json block that bench.py reads; it records
a hash of the kernel sources, so the figures are dropped once a kernel changes.

  python -m lora_mixture_experts_amd.profsum stats KERNEL_STATS.csv --cmd "..." --out FILE
  python -m lora_mixture_experts_amd.profsum counters COUNTERS.csv [...] --title T --cmd "..." --out FILE
  python -m lora_mixture_experts_amd.profsum traffic FETCH.csv WRITE.csv --copy-mib N \\
         --workload NAME --cmd "..." --out FILE
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import shlex
import sys
from collections import defaultdict

_PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_PKG, "csrc")
RUNTIME_COPY = "__amd_rocclr_copyBuffer"


def _is_stream_kernel(name: str) -> bool:
    """The elementwise negation bench.py runs as its streaming reference."""
    return "neg" in name and "elementwise" in name


def kernel_source_hash() -> str:
    """sha256 over the HIP sources and headers the library is built from."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def label(kernel_name: str) -> str | None:
    """Library kernel label of a demangled rocprofv3 kernel name, or None."""
    m = re.search(r"moelora::(k_\w+)(?:<([^>]*)>)?", kernel_name)
    if not m:
        return None
    fn, targs = m.group(1), (m.group(2) or "")
    if fn.startswith("k_gemm"):
        # the projection flag: the first template argument of the 16-row
        # kernel, the last one of the tiled and direct-load kernels
        args = [t.strip() for t in targs.split(",")] if targs else []
        flag = args[0] if fn == "k_gemm_skinny" and args else (args[-1] if args else "")
        return "gemm_gate_up" if flag == "true" else "gemm_down"
    return {"k_route": "route", "k_align": "align", "k_align_scatter": "align_scatter",
            "k_align_hist": "align_hist", "k_align_colscan": "align_colscan",
            "k_align_offsets": "align_offsets", "k_align_scatter_g": "align_scatter",
            "k_shrink": "shrink", "k_combine": "combine", "k_gather_f32": "gather_f32",
            "k_gather_bf16": "gather_bf16", "k_pack_skinny": "pack_weights (setup)",
            "k_align_one": "align", "k_align_count": "align_count", "k_align_place": "align_place",
            "k_zero": "clear (routing in gate_up)"}.get(fn, fn)


def _short(kernel_name: str) -> str:
    m = re.search(r"moelora::(k_\w+(?:<[^>]*>)?)", kernel_name)
    return m.group(1) if m else kernel_name


def _self_cmd() -> str:
    """This summarizer's own invocation, with --cmd standing for the profiled command(s)."""
    out, skip = [], False
    for a in sys.argv[1:]:
        if skip:
            skip = False
            continue
        if a == "--cmd":
            skip = True
            continue
        out.append(shlex.quote(a))
    return "python -m lora_mixture_experts_amd.profsum " + " ".join(out) + " --cmd '<the commands above>'"


def stats_summary(path: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(path)))
    lines = ["# Kernel durations (rocprofv3 --kernel-trace --stats)", "",
             "Commands (from the repository root):", "", "```", cmd, _self_cmd(), "```", "",
             f"Kernel sources hash: `{kernel_source_hash()}`", "",
             "| kernel | label | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short(r['Name'])}` | {label(r['Name']) or '-'} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(lines) + "\n"


def counters_summary(paths, title: str, cmd: str) -> str:
    vals = defaultdict(lambda: defaultdict(list))
    for path in paths:
        for r in csv.DictReader(open(path)):
            if label(r["Kernel_Name"]) is None:
                continue
            vals[_short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for per in vals.values() for c in per})
    lines = [f"# {title}", "", "Commands (from the repository root):", "", "```", cmd, _self_cmd(), "```", "",
             f"Kernel sources hash: `{kernel_source_hash()}`", "",
             "Average per dispatch (summed over the chip's counter instances).", "",
             "| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for k, per in vals.items():
        cells = [f"{sum(per[n]) / len(per[n]):.4g}" if per.get(n) else "-" for n in names]
        lines.append(f"| `{k}` | " + " | ".join(cells) + " |")
    return "\n".join(lines) + "\n"


def _per_kernel(path: str, counter: str):
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def traffic_summary(fetch_csv: str, write_csv: str, copy_mib: int, workload: str, cmd: str) -> str:
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0

    def reading(vals, pick):
        got = [max(v) for k, v in vals.items() if pick(k)]
        return max(got) if got else 0.0

    # the reference dispatches: the runtime's copy (largest copyBuffer
    # dispatch) and the elementwise stream kernel, both over copy_mib MiB
    f_rt, w_rt = reading(fetch, lambda k: k == RUNTIME_COPY), reading(write, lambda k: k == RUNTIME_COPY)
    f_el, w_el = reading(fetch, _is_stream_kernel), reading(write, _is_stream_kernel)
    if min(f_el, w_el) <= 0:
        raise SystemExit("no calibration dispatch found (run bench.py with --calibrate-copy)")
    ff, wf = copy_kib / f_el, copy_kib / w_el
    per = {}
    for name in sorted(set(fetch) | set(write)):
        lab = label(name)
        if lab is None:
            continue
        fk = sum(fetch.get(name, [0.0])) / max(len(fetch.get(name, [])), 1)
        wk = sum(write.get(name, [0.0])) / max(len(write.get(name, [])), 1)
        per[_short(name)] = dict(label=lab, dispatches=len(fetch.get(name, [])), fetch_kib=round(fk, 1),
                                 write_kib=round(wk, 1),
                                 bytes=int(round((fk * ff + wk * wf) * 1024)))
    lines = ["# HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
             f"Workload: {workload}", "", "Commands (from the repository root):", "", "```", cmd, _self_cmd(),
             "```", "",
             f"Calibration over {copy_mib} MiB ({copy_kib:.0f} KiB) read and written:", "",
             f"- elementwise stream kernel (ordinary vector loads and stores, like the layer's "
             f"kernels): FETCH_SIZE {f_el:.1f} KiB, WRITE_SIZE {w_el:.1f} KiB",
             f"- runtime device-to-device copy: FETCH_SIZE {f_rt:.1f} KiB, WRITE_SIZE {w_rt:.1f} KiB",
             "",
             f"Factors applied (from the elementwise kernel): fetch x{ff:.3f}, write x{wf:.3f}.", "",
             f"Kernel sources hash: `{kernel_source_hash()}`", "",
             "| kernel | label | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes |",
             "|---|---|---|---|---|---|"]
    for k, v in per.items():
        lines.append(f"| `{k}` | {v['label']} | {v['dispatches']} | {v['fetch_kib']} | {v['write_kib']} | "
                     f"{v['bytes'] / 1e6:.2f} MB |")
    blob = dict(workload=workload, source_hash=kernel_source_hash(), fetch_factor=round(ff, 4),
                write_factor=round(wf, 4),
                runtime_copy_factors=[round(copy_kib / f_rt, 4) if f_rt else None,
                                      round(copy_kib / w_rt, 4) if w_rt else None],
                kernels={v["label"]: v["bytes"] for v in per.values()
                         if v["label"] in ("gemm_gate_up", "gemm_down", "combine", "route")})
    lines += ["", "```json", json.dumps(blob), "```"]
    return "\n".join(lines) + "\n"


def read_traffic(path: str, label_: str):
    """Scaled HBM bytes per dispatch of `label_` from a traffic summary, or
    None if the file is missing or the kernel sources changed since."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    blob = json.loads(m.group(1))
    if blob.get("source_hash") != kernel_source_hash():
        return None
    return blob.get("kernels", {}).get(label_)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--title", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.mode == "stats":
        text = stats_summary(a.csv, a.cmd)
    elif a.mode == "counters":
        text = counters_summary(a.csv, a.title, a.cmd)
    else:
        text = traffic_summary(a.fetch_csv, a.write_csv, a.copy_mib, a.workload, a.cmd)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
