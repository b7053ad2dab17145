"""Phase timeline of the decode step from a stamps build (QSA_STAMPS).

    python -m top_sparse_attention_pooled_amd.build --stamps
    python -m top_sparse_attention_pooled_amd.stamps [--workload decode250k] [--steps 40]

Runs decode steps of one layer one at a time (eager launches), and after each
reads the per-workgroup real-time-clock stamps (100 MHz, 10 ns) the kernels
recorded at their numbered points.  Prints, over workgroups and steps, the
quantiles of each point's time from the first workgroup start of the step's
first kernel, and of each phase's duration.  Measurement only: the library
built with stamps is never the one the tests, smoke or the benchmark load.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SLOTS = 16
STAMP_WGS = 4096

# kernel -> (translation unit, {slot: point name}), for the decode step and
# for the prefill indexer
POINTS = {
    "k_score_cand": ("score", {0: "start", 2: "tile scored", 3: "end"}),
    "k_sel_attn": ("attn", {0: "start", 1: "keys counted", 7: "range reduced", 8: "round 1",
                            9: "round 2", 10: "round 3", 11: "round 4+", 2: "threshold",
                            3: "cells placed", 12: "chunk start", 13: "chunk scored",
                            14: "chunk done", 4: "end"}),
    "k_attn_combine": ("attn", {5: "start", 6: "end"}),
    # the split path's attention (several queries): the same slots, its last chunk
    "k_attn": ("attn", {0: "start", 12: "chunk start", 13: "chunk scored", 14: "chunk done",
                        4: "end"}),
}
PREFILL_POINTS = {
    "k_prefill_scores (maxima)": ("prefill", {0: "start", 1: "operands in",
                                              2: "first group", 3: "end"}),
    "k_prefill_scores (masks)": ("prefill", {4: "start", 5: "operands in",
                                             6: "first group", 7: "end"}),
    "k_prefill_tau": ("prefill", {8: "start", 9: "end"}),
    "k_select_prefill": ("prefill", {10: "start", 11: "band listed", 12: "bracket",
                                     13: "threshold", 14: "end"}),
}


def read(lib, unit):
    buf = np.zeros((STAMP_WGS, SLOTS), np.uint64)
    fn = getattr(lib, f"qsa_stamps_{unit}")
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int]
    rc = fn(buf.ctypes.data_as(ctypes.c_void_p), 1)
    if rc:
        raise RuntimeError(f"qsa_stamps_{unit} failed: {rc}")
    return buf.astype(np.int64)


def q(v):
    v = np.asarray(v, np.float64)
    return [round(float(np.percentile(v, p)), 2) for p in (0, 10, 50, 90, 100)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="decode250k")
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--skip", type=int, default=5, help="first steps left out (warm-up)")
    ap.add_argument("--json", default=None, help="also write the quantiles here")
    ap.add_argument("--again", action="store_true",
                    help="launch the selection + attention call a second time right after "
                         "the step and report that launch (warm caches)")
    args = ap.parse_args()

    import torch

    from . import qsa, runtime, synth
    lib = qsa.load(os.path.join(HERE, "libqsa_stamps.so"))
    if args.workload.startswith("prefill"):
        return prefill_main(args, lib, torch, qsa, runtime, synth)
    dev = "cuda:0"
    w = synth.WORKLOADS[args.workload]
    w = synth.Workload(**{**w.__dict__, "steps": max(w.steps, args.steps)})
    kidx, k, v = synth.make_kidx(w), synth.make_kv(w, synth.T_K), synth.make_kv(w, synth.T_V)
    layer = runtime.Layer(w, dev, kidx=kidx, k=k, v=v)
    layer.rebuild(np.full(w.n_seq, w.n_cells0, np.int32))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    torch.cuda.synchronize()
    for unit in ("score", "attn"):
        read(lib, unit)  # clear

    times = {name: {p: [] for p in pts[1].values()} for name, pts in POINTS.items()}
    durs = {}
    n_grp = -(-w.nb_max(0) // 256) * 4
    for step in range(args.steps):
        n = synth.n_cells_at(w, step)
        layer.set_n_cells(n)
        dirty = synth.dirty_blocks(w, step)
        q_idx, qq, q_seq, q_pos = synth.make_queries(w, step)
        bufs = runtime.StepBuffers(layer.dims, q_pos.size, w.nb_max(step), dev)
        torch.cuda.synchronize()
        args_t = (t(q_idx), t(qq), t(q_seq), t(q_pos))
        runtime.run_step(layer, bufs, *args_t, t(dirty.reshape(-1)), dirty.shape[0],
                         path="attend")
        if args.again:
            qsa.decode_select_attend(layer.dims, layer.seqs(), args_t[2], args_t[3],
                                     q_pos.size, bufs.nb_max, bufs.scores, bufs.ld,
                                     bufs.sel_blocks, bufs.sel_cells, bufs.n_sel, bufs.ws_fused,
                                     bufs.ws_fused_bytes, args_t[1], layer.k, layer.v, bufs.out,
                                     bufs.ws_attn, bufs.ws_attn_bytes)
        torch.cuda.synchronize()
        st = {u: read(lib, u) for u in ("score", "attn")}
        if step < args.skip:
            continue
        sc = st["score"][:n_grp * q_pos.size]
        t0 = sc[:, 0][sc[:, 0] > 0].min()
        for name, (unit, pts) in POINTS.items():
            tab = st[unit]
            first = min(pts)
            rows = tab[tab[:, first] > 0]
            if name == "k_score_cand":
                rows = sc[sc[:, 0] > 0]
            # slots 0 and 4 are either kernel's: the fused kernel's rows have
            # a threshold point, the split kernel's do not
            if name == "k_sel_attn":
                rows = rows[rows[:, 2] > 0]
            elif name == "k_attn":
                rows = rows[rows[:, 2] == 0]
            for slot, pname in pts.items():
                vals = rows[:, slot]
                vals = vals[vals > 0]
                times[name][pname] += list((vals - t0) * 0.01)
            sl = list(pts)
            for row in rows:  # phases between consecutive recorded points
                seen = [x for x in sl if row[x] > 0]
                for a_, b_ in zip(seen, seen[1:]):
                    key = f"{name}: {pts[a_]} -> {pts[b_]}"
                    durs.setdefault(key, []).append((row[b_] - row[a_]) * 0.01)
    out = {"workload": args.workload, "steps": args.steps - args.skip,
           "unit": "us; quantiles p0 p10 p50 p90 p100 over workgroups and steps",
           "points_from_first_score_start": {}, "phases": {}}
    print(f"# {args.workload}: {args.steps - args.skip} steps; microseconds, "
          "quantiles p0 p10 p50 p90 p100 over workgroups and steps")
    print("## time of each point from the first scoring workgroup's start")
    for name, pts in times.items():
        for pname, vals in pts.items():
            if vals:
                out["points_from_first_score_start"][f"{name}: {pname}"] = q(vals)
                print(f"{name:16s} {pname:16s} {q(vals)}")
    print("## phase durations within a workgroup")
    for key, vals in durs.items():
        if vals:
            out["phases"][key] = q(vals)
            print(f"{key:48s} {q(vals)}")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(out, f, indent=1)


def prefill_main(args, lib, torch, qsa, runtime, synth):
    """The prefill indexer (qsa_score_select_prefill) on the 512-token ubatch,
    repeated --steps times over the same blocks; per kernel, the quantiles
    over workgroups and repeats of each point's time from the kernel's first
    start, and of its phases."""
    dev = "cuda:0"
    w = synth.WORKLOADS[args.workload]
    kidx = synth.make_kidx(w)
    z = np.zeros((1, 1, 1, 1), np.uint8)
    layer = runtime.Layer(w, dev, kidx=kidx, k=z, v=z)
    layer.rebuild(np.full(1, w.n_cells0, np.int32))
    layer.set_n_cells(synth.n_cells_at(w, 0))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    q_idx, _, q_seq, q_pos = (t(x) for x in synth.make_queries(w, 0))
    dirty = synth.dirty_blocks(w, 0)
    dl = t(dirty.reshape(-1))
    nb = w.nb_max(0)
    bufs = runtime.StepBuffers(layer.dims, q_pos.numel(), nb, dev, prefill=True)
    torch.cuda.synchronize()
    read(lib, "prefill")
    times = {k: {p: [] for p in v[1].values()} for k, v in PREFILL_POINTS.items()}
    durs = {}
    for step in range(args.steps):
        qsa.score_select_prefill(layer.dims, layer.seqs(), layer.kidx, dl, dirty.shape[0],
                                 layer.pooled, layer.pooled_bf16, q_idx, q_seq, q_pos,
                                 q_pos.numel(), nb, bufs.sel_blocks, bufs.sel_cells, bufs.n_sel,
                                 bufs.ws_pf, bufs.ws_pf_bytes)
        torch.cuda.synchronize()
        tab = read(lib, "prefill")
        if step < args.skip:
            continue
        for name, (_, pts) in PREFILL_POINTS.items():
            first = min(pts)
            rows = tab[tab[:, first] > 0]
            if not len(rows):
                continue
            t0 = rows[:, first].min()
            for slot, pname in pts.items():
                vals = rows[:, slot]
                times[name][pname] += list((vals[vals > 0] - t0) * 0.01)
            sl = list(pts)
            for a_, b_ in zip(sl, sl[1:]):
                ok = (rows[:, a_] > 0) & (rows[:, b_] > 0)
                key = f"{name}: {pts[a_]} -> {pts[b_]}"
                durs.setdefault(key, []).extend(list((rows[ok, b_] - rows[ok, a_]) * 0.01))
    print(f"# {args.workload} indexer: {args.steps - args.skip} repeats; microseconds, "
          "quantiles p0 p10 p50 p90 p100 over workgroups and repeats")
    print("## time of each point from the kernel's first workgroup start")
    for name, pts in times.items():
        for pname, vals in pts.items():
            if vals:
                print(f"{name:28s} {pname:16s} {q(vals)}")
    print("## phase durations within a workgroup")
    for key, vals in durs.items():
        if vals:
            print(f"{key:60s} {q(vals)}")


if __name__ == "__main__":
    sys.exit(main())
