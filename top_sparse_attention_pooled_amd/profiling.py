"""Summaries of rocprofv3 runs: per-kernel durations and the HBM-side byte
counters (FETCH_SIZE, WRITE_SIZE) of a kernel, scaled by what the same
counters read for a plain streaming kernel of known size.

    python -m top_sparse_attention_pooled_amd.profiling traffic \\
        --fetch DIR --write DIR --kernel k_score_cand --workload decode250k \\
        --copy-mib 256 --out profiles/k_score_cand_decode250k_traffic

writes OUT.json (read by bench.py) and OUT.md.  The JSON carries a hash of
the kernel sources; bench.py reports the traffic only while the sources
still hash the same (a changed kernel makes the counters stale).

    python -m top_sparse_attention_pooled_amd.profiling kernels \
        --trace DIR --title "..." --command "..." --out profiles/NAME.md

writes a table of per-kernel device durations (min, median, p90, mean) from
a rocprofv3 --kernel-trace --stats run, followed by its kernel_stats.csv.

    python -m top_sparse_attention_pooled_amd.profiling counters \
        --pmc DIR [DIR ...] --match k_prefill --title "..." --command "..." \
        --out profiles/NAME.md

writes the per-dispatch mean of every counter collected in one or more
rocprofv3 --pmc runs, one row per kernel whose name contains --match.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
from typing import Dict, List

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
# the streaming kernel of known size: torch.neg over a float32 buffer (reads
# and writes copy_mib MiB each)
CALIBRATION_KERNEL = "neg"


# the source file that defines each profiled kernel
KERNEL_SOURCE = {"k_score_cand": "score.hip", "k_sel_attn": "attn.hip",
                 "k_attn_combine": "attn.hip", "k_rope_queries_delta": "prefill.hip",
                 "k_prefill_scores<0>": "prefill.hip", "k_prefill_scores<1>": "prefill.hip",
                 "k_prefill_tau<16>": "prefill.hip", "k_select_prefill": "prefill.hip"}


def _sources_of(name: str) -> List[str]:
    """The file and every local header it includes, transitively, in name order."""
    seen, todo = set(), [name]
    while todo:
        f = todo.pop()
        if f in seen or not os.path.exists(os.path.join(CSRC, f)):
            continue
        seen.add(f)
        with open(os.path.join(CSRC, f)) as fh:
            for line in fh:
                line = line.strip()
                if line.startswith('#include "') and not line.startswith('#include "../'):
                    todo.append(line.split('"')[1])
    return sorted(seen)


def source_hash(kernel: str = "k_score_cand") -> str:
    """sha256 over the sources the kernel is built from (its file and the
    local headers it includes), in name order."""
    h = hashlib.sha256()
    for f in _sources_of(KERNEL_SOURCE.get(kernel, "score.hip")):
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _rows(directory: str, suffix: str) -> List[dict]:
    files = glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    out = []
    for fn in files:
        with open(fn) as f:
            out.extend(csv.DictReader(f))
    return out


def counter_values(directory: str, counter: str) -> Dict[str, List[float]]:
    """Kernel name -> per-dispatch values of one counter (rocprofv3 --pmc CSV)."""
    out: Dict[str, List[float]] = {}
    for r in _rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def kernel_durations(directory: str) -> Dict[str, List[float]]:
    """Kernel name -> per-dispatch durations in microseconds (kernel trace)."""
    out: Dict[str, List[float]] = {}
    for r in _rows(directory, "kernel_trace.csv"):
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        out.setdefault(r["Kernel_Name"], []).append(d)
    return out


def _pick(values: Dict[str, List[float]], needle: str) -> List[float]:
    hits = [v for k, v in values.items() if needle in k]
    if len(hits) != 1:
        raise KeyError(f"{len(hits)} kernels match {needle!r}: "
                       f"{[k for k in values if needle in k]}")
    return hits[0]


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_mib: int) -> dict:
    fetch = counter_values(fetch_dir, "FETCH_SIZE")
    write = counter_values(write_dir, "WRITE_SIZE")
    known_kib = copy_mib * 1024.0
    cal_f = _pick(fetch, CALIBRATION_KERNEL)
    cal_w = _pick(write, CALIBRATION_KERNEL)
    f_scale = known_kib / statistics.mean(cal_f)
    w_scale = known_kib / statistics.mean(cal_w)
    kf = _pick(fetch, kernel)
    kw = _pick(write, kernel)
    fetch_b = statistics.mean(kf) * f_scale * 1024.0
    write_b = statistics.mean(kw) * w_scale * 1024.0
    return {
        "kernel": kernel,
        "dispatches": [len(kf), len(kw)],
        "fetch_kib_raw_mean": statistics.mean(kf),
        "write_kib_raw_mean": statistics.mean(kw),
        "calibration": {"kernel": CALIBRATION_KERNEL, "mib": copy_mib,
                        "fetch_kib_raw": statistics.mean(cal_f),
                        "write_kib_raw": statistics.mean(cal_w),
                        "fetch_scale": f_scale, "write_scale": w_scale},
        "fetch_bytes": fetch_b,
        "write_bytes": write_b,
        "traffic_bytes": fetch_b + write_b,
        "source_sha256": source_hash(kernel),
    }


def _quantile(v: List[float], q: float) -> float:
    s = sorted(v)
    return s[min(len(s) - 1, int(q * (len(s) - 1) + 0.5))]


def kernels_md(trace_dir: str, title: str, command: str, notes: str = "") -> str:
    """Markdown: per-kernel durations of a kernel trace, then the stats CSV."""
    dur = kernel_durations(trace_dir)
    lines = [f"# {title}", ""]
    if command:
        lines += ["Command:", "", "```", command.strip(), "```", ""]
    lines += ["Per-kernel device durations from the kernel trace (microseconds):", "",
              "| kernel | launches | min | median | p90 | mean |", "|---|---|---|---|---|---|"]
    order = sorted(dur.items(), key=lambda kv: -sum(kv[1]))
    for name, v in order:
        if "FillFunctor" in name or "copyBuffer" in name:
            continue
        short = name.replace("qsa::(anonymous namespace)::", "").replace("void ", "")
        short = short.split("(")[0]
        lines.append(f"| {short} | {len(v)} | {min(v):.2f} | {statistics.median(v):.2f} | "
                     f"{_quantile(v, 0.9):.2f} | {statistics.mean(v):.2f} |")
    lines.append("")
    if notes:
        lines += [notes.strip(), ""]
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        with open(stats[0]) as f:
            raw = f.read().strip().splitlines()
        lines += ["rocprofv3 --stats (kernel_stats.csv):", "", "```"] + raw[:12] + ["```", ""]
    return "\n".join(lines)


def counters_md(dirs: List[str], match: str, title: str, command: str, notes: str = "") -> str:
    """Markdown: per kernel (name containing match), the mean of each counter
    per dispatch over the --pmc runs in dirs."""
    per: Dict[str, Dict[str, List[float]]] = {}
    for d in dirs:
        for r in _rows(d, "counter_collection.csv"):
            name = r["Kernel_Name"]
            if match not in name:
                continue
            short = name.replace("qsa::(anonymous namespace)::", "").replace("void ", "")
            short = short.split("(")[0]
            per.setdefault(short, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    names = sorted({c for v in per.values() for c in v})
    lines = [f"# {title}", ""]
    if command:
        lines += ["Commands:", "", "```", command.strip(), "```", ""]
    lines += ["Mean per dispatch:", "", "| kernel | dispatches | " + " | ".join(names) + " |",
              "|---|---|" + "---|" * len(names)]
    for k in sorted(per):
        v = per[k]
        n = max(len(x) for x in v.values())
        cells = [f"{statistics.mean(v[c]):.4g}" if c in v else "" for c in names]
        lines.append(f"| {k} | {n} | " + " | ".join(cells) + " |")
    lines.append("")
    if notes:
        lines += [notes.strip(), ""]
    return "\n".join(lines)


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("--trace", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--command", default="")
    k.add_argument("--notes", default="")
    k.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--pmc", nargs="+", required=True)
    c.add_argument("--match", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", default="")
    c.add_argument("--notes", default="")
    c.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", default="", help="the profiling commands, for the record")
    t.add_argument("--notes", default="", help="lines appended to OUT.md")
    a = ap.parse_args()
    if a.cmd == "kernels":
        with open(a.out, "w") as f:
            f.write(kernels_md(a.trace, a.title, a.command, a.notes))
        return
    if a.cmd == "counters":
        with open(a.out, "w") as f:
            f.write(counters_md(a.pmc, a.match, a.title, a.command, a.notes))
        return
    res = traffic(a.fetch, a.write, a.kernel, a.copy_mib)
    res["workload"] = a.workload
    with open(a.out + ".json", "w") as f:
        json.dump(res, f, indent=1)
    c = res["calibration"]
    with open(a.out + ".md", "w") as f:
        f.write(f"# {a.kernel} HBM-side traffic, {a.workload}\n\n")
        if a.command:
            f.write("Commands:\n\n```\n" + a.command.strip() + "\n```\n\n")
        f.write(f"- dispatches (FETCH, WRITE runs): {res['dispatches']}\n")
        f.write(f"- raw FETCH_SIZE mean {res['fetch_kib_raw_mean']:.1f} KiB, "
                f"raw WRITE_SIZE mean {res['write_kib_raw_mean']:.1f} KiB per dispatch\n")
        f.write(f"- calibration: torch.{c['kernel']} over {c['mib']} MiB reads "
                f"{c['fetch_kib_raw']:.1f} KiB / writes {c['write_kib_raw']:.1f} KiB raw "
                f"-> scale {c['fetch_scale']:.4f} (fetch), {c['write_scale']:.4f} (write)\n")
        f.write(f"- scaled: fetch {res['fetch_bytes'] / 1e6:.3f} MB, write "
                f"{res['write_bytes'] / 1e6:.3f} MB, total "
                f"{res['traffic_bytes'] / 1e6:.3f} MB per dispatch\n")
        f.write(f"- kernel sources sha256 {res['source_sha256']}\n")
        if a.notes:
            f.write(a.notes.strip() + "\n")
    print(json.dumps(res))


if __name__ == "__main__":
    main()
