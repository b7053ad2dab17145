#!/usr/bin/env python3
"""Benchmark of the QSA sparse-attention step on one MI355X.

A decode step is one token through the whole hot path -- pooled-key update,
block scoring, block top-k, sparse attention -- in each of 12 QSA layers (the
pages' model has 12 QSA layers; 12 replicas of one layer's caches at distinct
addresses also keep the ~400 MB working set out of the 256 MB last-level
cache, so the bytes come from HBM).  The K timed steps are captured in one
HIP graph and replayed; inputs are resident in HBM before timing starts.

The default run (no --workload) measures the 250k-context decode step and,
in the same JSON line, the 512-token prefill ubatch at depth 198,628
("prefill"): the metric names both.  --workload picks one workload alone.

Prints one JSON line.  value = microseconds per token per QSA layer (lower is
better); step_device_us = per-step device time quantiles (events around
one-step graph replays); roofline = the kernel that takes the most time in the
step, against HBM peak, with every kernel's own fraction in roofline.kernels
and the whole step's in roofline.step; cpu_baseline = the CPU oracle on a
bounded sample of the same steps, on all host cores (OpenMP over independent
blocks and heads) and on one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP16_PEAK_TFLOPS = 2500.0
N_LAYERS = 12
METRIC = "QSA sparse-attn decode µs/token and HBM GB/s at 250k ctx; prefill t/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    choices=["decode50k", "decode250k", "decode5x250k", "verify5x250k",
                             "verify5x250k_ar1", "prefill", "prefill_ar1"],
                    help="one workload alone (default: decode250k plus the prefill ubatch)")
    ap.add_argument("--kv", default="q8_0", choices=["q8_0", "f16"],
                    help="K/V cache type of a decode workload (the workloads are defined "
                         "with q8_0; f16 is the type the pages' first fix required)")
    ap.add_argument("--layers", type=int, default=N_LAYERS)
    ap.add_argument("--prefill-steps", type=int, default=16,
                    help="timed prefill ubatch steps in the default run")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="budget of each CPU-oracle baseline leg (0 = skip)")
    ap.add_argument("--profile", action="store_true",
                    help="short run for a profiler: no CPU baseline, no per-step replays")
    ap.add_argument("--eager", action="store_true",
                    help="launch the steps directly instead of replaying a graph (for "
                         "hardware-counter runs)")
    ap.add_argument("--probe", action="store_true",
                    help="memory-traffic floors instead of the step: HBM, last-level-cache and "
                         "L2 streaming reads, and the prefill attention's K/V row gather alone "
                         "beside the attention kernel itself")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also copy an MIB-MiB buffer once: a kernel of known traffic "
                         "that scales the byte counters")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# host and oracle threads
# ---------------------------------------------------------------------------

def host_info():
    """CPU model, sockets and the cores this process may use."""
    model, sockets = None, set()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name") and model is None:
                    model = line.split(":", 1)[1].strip()
                elif line.startswith("physical id"):
                    sockets.add(line.split(":", 1)[1].strip())
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cores": aff, "cpu_model": model,
            "sockets": max(1, len(sockets))}


def oracle_threads(host):
    """All the cores this process may use, within OMP_NUM_THREADS if set."""
    n = host["usable_cores"] or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def algorithmic_bytes(w, step):
    """Bytes one layer-step must move at minimum, by part of the step."""
    from top_sparse_attention_pooled_amd import synth
    n = w.n_cells0 + (step + 1) * w.n_new
    nc = n // w.r
    nb = w.nb_max(step)
    n_q = w.n_seq * w.n_new
    tail = n - nc * w.r
    n_sel = min(nc, w.top_k // w.r) * w.r + tail
    row = synth.row_bytes(w.kv_type, w.D)
    return {
        # pooled keys of the complete blocks, the score row, the query
        "score": n_q * (nc * w.d * 4 + nb * 4 + w.d * 4),
        # the dirty block's r per-cell keys in, its f32 and bf16 key out
        "update": w.n_seq * (w.r * w.d * 4 + w.d * 4 + w.d * 2),
        # selection outputs (the candidates it reads are the score kernel's)
        "select": n_q * ((w.top_k // w.r + w.ld_cells) * 4),
        # K and V rows of the selected cells, Q in, O out, the cell list
        "attn": n_q * (n_sel * w.Hk * row * 2 + 2 * w.H * w.D * 4 + n_sel * 4),
    }


def setup(torch, dev, name, K, W, L, kv="q8_0"):
    """Caches of L layer replicas plus the per-step device inputs."""
    from top_sparse_attention_pooled_amd import runtime, synth
    w = synth.WORKLOADS[name]
    prefill = name.startswith("prefill")
    if not prefill and K + W > w.steps:
        w = synth.Workload(**{**w.__dict__, "steps": K + W})
    if not prefill and kv == "f16":
        w = synth.Workload(**{**w.__dict__, "kv_type": synth.KV_F16})
    t0 = time.time()
    kidx = synth.make_kidx(w)
    k = synth.make_kv(w, synth.T_K)
    v = synth.make_kv(w, synth.T_V)
    base = runtime.Layer(w, dev, kidx=kidx, k=k, v=v)
    n0 = np.full(w.n_seq, w.n_cells0, np.int32)
    base.rebuild(n0)
    layers = [base] + [runtime.Layer.clone_of(base) for _ in range(L - 1)]
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f}s ({name}, {L} layer replicas)",
          file=sys.stderr, flush=True)
    # per-step inputs for warmup + timed steps; a prefill step repeats the
    # same ubatch (re-dirtying the same blocks), a decode step appends a token
    T = W + K
    steps = [0] * T if prefill else list(range(T))
    qi, qq, qs, qp, nc_all, dl_all = [], [], [], [], [], []
    for t in steps:
        a, b, c, d = synth.make_queries(w, t)
        qi.append(a); qq.append(b); qs.append(c); qp.append(d)
        nc_all.append(synth.n_cells_at(w, t))
        dl_all.append(synth.dirty_blocks(w, t))
    to = lambda x: torch.from_numpy(np.ascontiguousarray(np.stack(x))).to(dev)
    inp = {"q_idx": to(qi), "q": to(qq), "q_seq": to(qs), "q_pos": to(qp),
           "n_cells": to(nc_all), "dirty": to([d.reshape(-1) for d in dl_all]),
           "n_dirty": dl_all[0].shape[0], "n_q": qp[0].shape[0],
           "nb_max": w.nb_max(max(steps))}
    host = dict(kidx=kidx, k=k, v=v, qi=qi, qq=qq, qs=qs, qp=qp, nc_all=nc_all, dl_all=dl_all)
    return w, layers, inp, host


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

class Timer:
    """HIP-graph capture and replay of a step function on one stream, with
    HIP events recorded on that stream around the replays (this runtime takes
    no event nodes inside a captured graph)."""

    def __init__(self, torch, stream, enqueue, eager=False):
        self.torch, self.stream, self.enqueue, self.eager = torch, stream, enqueue, eager

    def capture(self, steps, **kw):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for t in steps:
                self.enqueue(t, **kw)
        return g

    def run(self, W, T):
        """W warm-up steps, then steps W..T-1 timed as one graph replay (or
        launched directly when eager).  Returns seconds."""
        torch = self.torch
        if self.eager:
            with torch.cuda.stream(self.stream):
                for t in range(W):
                    self.enqueue(t)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            with torch.cuda.stream(self.stream):
                for t in range(W, T):
                    self.enqueue(t)
            torch.cuda.synchronize()
            return time.perf_counter() - t0
        g_warm = self.capture(range(W)) if W > 0 else None
        g_main = self.capture(range(W, T))
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            if g_warm is not None:
                g_warm.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g_main.replay()
            torch.cuda.synchronize()
        return time.perf_counter() - t0

    def part(self, W, T, n_launches, **kw):
        """Mean device time of one launch of a part of the step: a graph of
        just those launches over the timed steps, between two events."""
        torch = self.torch
        g = self.capture(range(W, T), **kw)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):  # a graph replays on the current stream
            g.replay()
            torch.cuda.synchronize()
            ev0.record(self.stream)
            g.replay()
            ev1.record(self.stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1000.0 / n_launches

    def per_step(self, W, T):
        """Device time of each timed step: one graph per step, replayed back
        to back with an event between consecutive replays.  Microseconds."""
        torch = self.torch
        graphs = [self.capture([t]) for t in range(W, T)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(graphs) + 1)]
        with torch.cuda.stream(self.stream):  # a graph replays on the current stream
            for g in graphs:  # warm every graph once
                g.replay()
            torch.cuda.synchronize()
            evs[0].record(self.stream)
            for g, e in zip(graphs, evs[1:]):
                g.replay()
                e.record(self.stream)
        torch.cuda.synchronize()
        return np.array([evs[i].elapsed_time(evs[i + 1]) * 1000.0 for i in range(len(graphs))])


def quantiles(us):
    return {"median": round(float(np.median(us)), 3), "p10": round(float(np.percentile(us, 10)), 3),
            "p90": round(float(np.percentile(us, 90)), 3), "n": int(len(us))}


def calibration_copy(args, torch, dev):
    if args.copy_calibration:  # one streaming kernel of known traffic
        n = args.copy_calibration * (1 << 20) // 4
        src_buf = torch.ones(n, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        torch.neg(src_buf, out=dst_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

# The decode step's kernels, in launch order, with the part of the step whose
# algorithmic bytes each one moves.
DECODE_KERNELS = [("k_score_cand", "score"), ("k_sel_attn", "attn"),
                  ("k_attn_combine", None)]


def run_decode(args, torch, dev, name):
    from top_sparse_attention_pooled_amd import qsa, runtime, synth
    K, W, L = args.steps, args.warmup, args.layers
    w, layers, inp, host = setup(torch, dev, name, K, W, L, args.kv)
    T = W + K
    q_idx, q, q_seq, q_pos = inp["q_idx"], inp["q"], inp["q_seq"], inp["q_pos"]
    n_cells, dirty, n_dirty = inp["n_cells"], inp["dirty"], inp["n_dirty"]
    n_q, nb_max = inp["n_q"], inp["nb_max"]
    bufs = [runtime.StepBuffers(layers[0].dims, n_q, nb_max, dev) for _ in range(L)]
    stream = torch.cuda.Stream()

    def enqueue(t, part="all"):
        """One decode token through every layer: update + scores + candidates,
        then selection fused into attention (+ the merge of partial states)."""
        for li, layer in enumerate(layers):
            layer.n_cells = n_cells[t]
            bf, d, sq = bufs[li], layer.dims, layer.seqs()
            if part in ("all", "score"):
                qsa.decode_score_candidates(d, sq, layer.kidx, dirty[t], n_dirty, layer.pooled,
                                            layer.pooled_bf16, q_idx[t], q_seq[t], q_pos[t],
                                            n_q, nb_max, bf.scores, bf.ld, bf.ws_fused,
                                            bf.ws_fused_bytes)
            if part in ("all", "select_attend"):
                qsa.decode_select_attend(d, sq, q_seq[t], q_pos[t], n_q, nb_max, bf.scores,
                                         bf.ld, bf.sel_blocks, bf.sel_cells, bf.n_sel,
                                         bf.ws_fused, bf.ws_fused_bytes, q[t], layer.k, layer.v,
                                         bf.out, bf.ws_attn, bf.ws_attn_bytes)

    calibration_copy(args, torch, dev)
    timer = Timer(torch, stream, enqueue, args.eager)
    t_main = timer.run(W, T)
    parts, steps_us = {}, None
    if not args.eager:
        parts["score"] = timer.part(W, T, K * L, part="score")
        # the selection reads the candidates its step's scoring left, so it is
        # not replayed alone (stale candidates, or one step replayed K times,
        # would send every replay down one step's path): its share is the
        # step's time less the scoring launch's
        parts["select_attend"] = t_main * 1e6 / (K * L) - parts["score"]
        if not args.profile:
            steps_us = timer.per_step(W, T) / L

    # correctness guard on the last step of layer 0 (selection sizes)
    n_sel = bufs[0].n_sel.cpu().numpy()
    assert np.all(n_sel > 0), "empty selections in the benchmark step"

    ms_per_step = t_main * 1000.0 / K
    us_per_step_layer = ms_per_step * 1000.0 / L
    us_per_token_layer = us_per_step_layer / n_q  # n_q tokens per step (one per session)
    ab = [algorithmic_bytes(w, t) for t in range(W, T)]
    mean_b = {k: float(np.mean([a[k] for a in ab])) for k in ab[0]}
    step_bytes = sum(mean_b.values())

    # per-kernel fractions: the scoring launch timed alone; the selection +
    # attention call holds two launches whose split comes from the kernel
    # trace, so its fraction is that of the call
    kernels = []
    if parts:
        kernels.append({"kernel": "k_score_cand", "avg_launch_us": round(parts["score"], 3),
                        "bytes_per_launch": round(mean_b["score"] + mean_b["update"]),
                        "frac": round((mean_b["score"] + mean_b["update"]) /
                                      (parts["score"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": recorded_traffic(name, "k_score_cand")})
        d0 = layers[0].dims
        hpk = d0.n_head // d0.n_head_kv
        n_set = -(-(d0.n_head // (2 if hpk % 2 == 0 else 1)) // 2)
        fused = n_q * -(-d0.ld_cells // 32) * n_set <= 512  # the library's fused-grid rule
        kernels.append({"kernel": ("k_sel_attn + k_attn_combine (one call)" if fused else
                                   "k_select_cand + k_attn + k_attn_combine (one call)"),
                        "avg_launch_us": round(parts["select_attend"], 3),
                        "bytes_per_launch": round(mean_b["attn"] + mean_b["select"]),
                        "frac": round((mean_b["attn"] + mean_b["select"]) /
                                      (parts["select_attend"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": (recorded_call_traffic(name, ["k_sel_attn", "k_attn_combine"])
                                    if fused else None)})
    dom = max(kernels, key=lambda k: k["avg_launch_us"]) if kernels else None
    step_frac = step_bytes / (us_per_step_layer * 1e-6) / 1e9 / HBM_PEAK_GBS
    result = {
        "metric": METRIC,
        "value": round(us_per_token_layer, 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {synth.KV_Q8_0: "f32 (q8_0 KV)", synth.KV_F16: "f32 (f16 KV)"}.get(w.kv_type, "f32"),
        "data": "synthetic: i.i.d. N(0,1) indexer keys, queries and K/V (%s), seeded"
                % {synth.KV_Q8_0: "q8_0-packed", synth.KV_F16: "rounded to f16"}.get(w.kv_type, "f32"),
        "config": {
            "workload": name if args.kv == "q8_0" else f"{name} (f16 KV)",
            "n_seq": w.n_seq, "n_kv_start": w.n_cells0 + w.n_new, "decode_steps": K,
            "q_heads": w.H, "kv_heads": w.Hk, "head_dim": w.D, "indexer_dim": w.d,
            "compress_ratio": w.r, "top_k": w.top_k,
            "layers_per_step": L, "graph_replay": not args.eager,
        },
        "tokens_per_s_per_layer": round(1e6 / us_per_token_layer, 1),
        "us_per_step_layer": round(us_per_step_layer, 3),
        "step_device_us": quantiles(steps_us) if steps_us is not None else None,
        "step_hbm_gbps": round(step_bytes / (us_per_step_layer * 1e-6) / 1e9, 1),
        "roofline": {
            "kernel": dom["kernel"] if dom else None,
            "timing": ("scoring: events around a graph of its K*L launches alone; the "
                       "selection + attention call: the step's time less the scoring's"),
            "bound": "hbm",
            "achieved": round(dom["bytes_per_launch"] / (dom["avg_launch_us"] * 1e-6) / 1e9, 1)
            if dom else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dom["frac"] if dom else None,
            "traffic": dom.get("traffic") if dom else None,
            "bytes_per_launch": dom["bytes_per_launch"] if dom else None,
            "avg_launch_us": dom["avg_launch_us"] if dom else None,
            "kernels": kernels,
            "step": {"bytes": round(step_bytes), "us": round(us_per_step_layer, 3),
                     "achieved": round(step_bytes / (us_per_step_layer * 1e-6) / 1e9, 1),
                     "frac": round(step_frac, 4)},
        },
    }
    if not args.profile and args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_decode(w, host, W, K, args.cpu_seconds)
    del layers, bufs, inp
    return result


# ---------------------------------------------------------------------------
# several tokens per sequence (a verify step)
# ---------------------------------------------------------------------------

def run_verify(args, torch, dev, name):
    """A step = the sequence's 5 new tokens through every layer: update,
    scores and candidates of all 5 (one call), the exact selection of each,
    then attention (a) over the union of the 5 lists, each K/V row staged once
    for the tokens that list it (qsa_sparse_attn_decode_union), or (b) per
    token (qsa_decode_select_attend, which selects and attends per query);
    and (c) the first token alone through the 1-token path.  value = us per
    token per layer of (a)."""
    from top_sparse_attention_pooled_amd import qsa, runtime, synth
    K, W, L = args.steps, args.warmup, args.layers
    w, layers, inp, host = setup(torch, dev, name, K, W, L)
    T = W + K
    q_idx, q, q_seq, q_pos = inp["q_idx"], inp["q"], inp["q_seq"], inp["q_pos"]
    n_cells, dirty, n_dirty = inp["n_cells"], inp["dirty"], inp["n_dirty"]
    n_q, nb_max = inp["n_q"], inp["nb_max"]
    d0 = layers[0].dims
    bufs = [runtime.StepBuffers(d0, n_q, nb_max, dev) for _ in range(L)]
    bufs1 = [runtime.StepBuffers(d0, 1, nb_max, dev) for _ in range(L)]
    u_bytes = qsa.workspace_size(d0, qsa.OP_ATTN_DECODE_UNION, n_q, n_q)
    u_ws = [torch.empty(max(u_bytes, 16), dtype=torch.uint8, device=dev) for _ in range(L)]
    stream = torch.cuda.Stream()

    def enqueue(t, part="union"):
        for li, layer in enumerate(layers):
            layer.n_cells = n_cells[t]
            d, sq = layer.dims, layer.seqs()
            bf = bufs[li] if part != "one" else bufs1[li]
            m = n_q if part != "one" else 1
            qsa.decode_score_candidates(d, sq, layer.kidx, dirty[t], n_dirty, layer.pooled,
                                        layer.pooled_bf16, q_idx[t], q_seq[t], q_pos[t], m,
                                        nb_max, bf.scores, bf.ld, bf.ws_fused, bf.ws_fused_bytes)
            if part == "union":
                qsa.decode_select_candidates(d, sq, q_seq[t], q_pos[t], m, nb_max, bf.scores,
                                             bf.ld, bf.sel_blocks, bf.sel_cells, bf.n_sel,
                                             bf.ws_fused, bf.ws_fused_bytes)
                qsa.sparse_attn_decode_union(d, sq, q[t], q_seq[t], m, m, layer.k, layer.v,
                                             bf.sel_cells, bf.n_sel, bf.out, u_ws[li], u_bytes)
            else:
                qsa.decode_select_attend(d, sq, q_seq[t], q_pos[t], m, nb_max, bf.scores,
                                         bf.ld, bf.sel_blocks, bf.sel_cells, bf.n_sel,
                                         bf.ws_fused, bf.ws_fused_bytes, q[t], layer.k, layer.v,
                                         bf.out, bf.ws_attn, bf.ws_attn_bytes)

    timer = Timer(torch, stream, enqueue, args.eager)
    t_main = timer.run(W, T)
    res_us = {"union": t_main * 1e6 / (K * L)}
    if not args.eager:
        for part in ("per_token", "one"):
            res_us[part] = timer.part(W, T, K * L, part=part)
    n_sel = bufs[0].n_sel.cpu().numpy()
    assert np.all(n_sel > 0), "empty selections in the benchmark step"
    # union size of the last step, layer 0 (the union workspace's n_union)
    ld = d0.ld_cells
    cap = n_q * ld
    rnd = lambda x: -(-x // 256) * 256
    n_union = int(u_ws[0][rnd(cap * 4) + rnd(cap):][:4].view(torch.int32).item())
    listed = int(n_sel.sum())
    per_tok = {k: round(v / (n_q if k != "one" else 1), 3) for k, v in res_us.items()}
    # algorithmic bytes per step: the pooled keys once, the union's K/V rows once
    nb = w.nb_max(K + W - 1)
    kv_row = w.Hk * synth.row_bytes(w.kv_type, w.D) * 2
    step_bytes = nb * w.d * 4 + n_union * kv_row
    result = {
        "metric": METRIC, "value": per_tok["union"], "unit": "us/token", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(t_main * 1000.0 / K, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 scores and selection; fp16 attention operands over q8_0 KV (fp32 sums)",
        "data": "synthetic: i.i.d. N(0,1) indexer keys, queries and K/V (q8_0-packed), seeded"
                + ("; indexer queries AR(1) along the step's tokens, rho %g" % w.extra["qidx_ar1"]
                   if w.extra.get("qidx_ar1") else ""),
        "config": {"workload": name, "n_seq": 1, "tokens_per_step": n_q,
                   "n_kv_start": w.n_cells0 + w.n_new, "decode_steps": K, "q_heads": w.H,
                   "kv_heads": w.Hk, "head_dim": w.D, "top_k": w.top_k, "layers_per_step": L,
                   "graph_replay": not args.eager},
        "us_per_token_layer": {"union_attention": per_tok["union"],
                               "per_token_attention": per_tok.get("per_token"),
                               "one_token_step": per_tok.get("one")},
        "us_per_step_layer": {k: round(v, 3) for k, v in res_us.items()},
        "union": {"rows": n_union, "listed_cells": listed,
                  "rows_per_listed": round(n_union / max(listed, 1), 3)},
        "roofline": {
            "kernel": "the whole verify step (update, scores, selection, union attention)",
            "timing": "graph replay of K steps x L layers",
            "bound": "hbm",
            "bytes_per_step": int(step_bytes),
            "achieved": round(step_bytes / (res_us["union"] * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(step_bytes / (res_us["union"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
    }
    del layers, bufs, bufs1, inp
    return result


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def run_prefill(args, torch, dev, name, K, W):
    """One step = the 512-token ubatch at depth 198,628 through every layer:
    pooled-key update of its 128 dirty blocks, bf16 MFMA block scores,
    per-query exact block top-k, sparse attention per query."""
    from top_sparse_attention_pooled_amd import qsa, runtime, synth
    L = args.layers
    w, layers, inp, host = setup(torch, dev, name, K, W, L)
    T = W + K
    q_idx, q, q_seq, q_pos = inp["q_idx"], inp["q"], inp["q_seq"], inp["q_pos"]
    n_cells, dirty, n_dirty = inp["n_cells"], inp["dirty"], inp["n_dirty"]
    n_q, nb_max = inp["n_q"], inp["nb_max"]
    bufs = [runtime.StepBuffers(layers[0].dims, n_q, nb_max, dev, prefill=True)
            for _ in range(L)]
    stream = torch.cuda.Stream()
    for layer in layers:
        layer.n_cells = n_cells[0]

    def enqueue(t, part="all"):
        for li, layer in enumerate(layers):
            bf, d, sq = bufs[li], layer.dims, layer.seqs()
            if part in ("all", "indexer"):
                qsa.score_select_prefill(d, sq, layer.kidx, dirty[t], n_dirty, layer.pooled,
                                         layer.pooled_bf16, q_idx[t], q_seq[t], q_pos[t], n_q,
                                         nb_max, bf.sel_blocks, bf.sel_cells, bf.n_sel,
                                         bf.ws_pf, bf.ws_pf_bytes)
            if part in ("all", "attn"):
                qsa.sparse_attn_prefill(d, sq, q[t], q_seq[t], n_q, layer.k, layer.v,
                                        bf.sel_cells, bf.n_sel, bf.out, bf.ws_attn,
                                        bf.ws_attn_bytes)

    calibration_copy(args, torch, dev)
    timer = Timer(torch, stream, enqueue, args.eager)
    t_main = timer.run(W, T)
    parts, steps_us = {}, None
    if not args.eager:
        for part in ("indexer", "attn"):
            parts[part] = timer.part(W, T, K * L, part=part)
        if not args.profile:
            steps_us = timer.per_step(W, T) / L
    n_sel = bufs[0].n_sel.cpu().numpy()
    assert np.all(n_sel > 0), "empty selections in the benchmark step"

    ms_per_step = t_main * 1000.0 / K
    us_per_layer = ms_per_step * 1000.0 / L
    pos = host["qp"][0]
    nc = (pos.astype(np.int64) + 1) // w.r
    flops = float(np.sum(nc)) * w.d * 2  # the dense query x block-key contraction
    n_sel_np = n_sel.astype(np.int64)
    attn_flops = float(np.sum(n_sel_np)) * w.H * w.D * 4  # QK and PV over the lists
    score_us, attn_us = parts.get("indexer"), parts.get("attn")
    tflops = flops / (score_us * 1e-6) / 1e12 if score_us else None
    attn_tflops = attn_flops / (attn_us * 1e-6) / 1e12 if attn_us else None
    res = {
        "t_s_per_layer": round(n_q / (us_per_layer * 1e-6), 1),
        "us_per_layer": round(us_per_layer, 2),
        "model_prefill_t_s": round(n_q / (ms_per_step * 1e-3), 1),
        "steps": K, "warmup": W,
        "step_device_us": quantiles(steps_us) if steps_us is not None else None,
        "parts_us": {k: round(v, 2) for k, v in parts.items()},
        "indexer_mfma": {"flops_per_launch": flops,
                         "achieved_tflops": round(tflops, 2) if tflops else None,
                         "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4) if tflops else None,
                         "traffic": (recorded_call_traffic(name, PREFILL_INDEXER_KERNELS)
                                     if name == "prefill" else None)},
        "attn_mfma": {"flops_per_launch": attn_flops,
                      "achieved_tflops": round(attn_tflops, 2) if attn_tflops else None,
                      "peak_tflops": MFMA_FP16_PEAK_TFLOPS,
                      "frac": round(attn_tflops / MFMA_FP16_PEAK_TFLOPS, 4) if attn_tflops else None},
        "config": {
            "workload": name, "n_seq": 1, "n_kv_start": w.n_cells0, "ubatch": n_q,
            "dirty_blocks": int(np.sum(host["dl_all"][0][:, 0] >= 0)),
            "q_heads": w.H, "kv_heads": w.Hk, "head_dim": w.D, "indexer_dim": w.d,
            "compress_ratio": w.r, "top_k": w.top_k, "layers_per_step": L,
            "graph_replay": not args.eager,
        },
        "data": ("synthetic: i.i.d. N(0,1) indexer keys, queries and K/V (q8_0-packed), seeded"
                 + ("; indexer queries AR(1) along the tokens, rho %g" % w.extra["qidx_ar1"]
                    if w.extra.get("qidx_ar1") else "")),
    }
    if not args.profile and args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_prefill(w, host, args.cpu_seconds)
    del layers, bufs, inp
    return res, ms_per_step, w


# ---------------------------------------------------------------------------
# counters and the CPU baseline
# ---------------------------------------------------------------------------

def recorded_traffic(workload, kernel="k_score_cand"):
    """HBM-side bytes per launch of `kernel` from the committed counter
    summary (two rocprofv3 --pmc runs, scaled by a streaming kernel of known
    size), or None if there is none or the kernel's sources changed since."""
    from top_sparse_attention_pooled_amd import profiling
    stem = kernel.replace("<", "_").replace(">", "")  # k_prefill_scores<0> -> k_prefill_scores_0
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != profiling.source_hash(kernel):
        return None
    return round(rec["traffic_bytes"])


# the launches of one qsa_score_select_prefill call at the 512-token ubatch
PREFILL_INDEXER_KERNELS = ["k_rope_queries_delta", "k_prefill_scores<0>", "k_prefill_tau<16>",
                           "k_prefill_scores<1>", "k_select_prefill"]


def recorded_call_traffic(workload, kernels):
    """The sum of recorded_traffic over the launches of one call, or None
    if any of them has no current figure."""
    parts = [recorded_traffic(workload, k) for k in kernels]
    return None if any(p is None for p in parts) else sum(parts)


def _decode_oracle_leg(w, host, W, K, budget, threads):
    """The oracle's decode steps (one layer): per step the pooled-key update,
    then scores, full-sort selection and fp64 attention.  Returns (us per
    token, steps done)."""
    import oracle
    oracle.set_threads(threads)
    kidx, k, v = host["kidx"], host["k"], host["v"]
    pooled = np.zeros((w.n_seq, w.cap_blocks, w.d), np.float32)
    n0 = np.full(w.n_seq, w.n_cells0, np.int32)
    pairs = [(s, b) for s in range(w.n_seq) for b in range(-(-w.n_cells0 // w.r))]
    oracle.update_pooled(kidx, n0, np.array(pairs, np.int32), pooled, w.r, w.theta, w.eps)
    done, spent = 0, 0.0
    for t in range(W + K):
        t0 = time.perf_counter()
        oracle.update_pooled(kidx, host["nc_all"][t], host["dl_all"][t], pooled, w.r, w.theta,
                             w.eps)
        oracle.step(host["qi"][t], host["qq"][t], host["qs"][t], host["qp"][t], pooled, k, v,
                    kv_type=w.kv_type, n_head_kv=w.Hk, r=w.r, top_k=w.top_k, theta=w.theta,
                    nb_out=w.nb_max(t))
        spent += time.perf_counter() - t0
        done += 1
        if spent > budget:
            break
    oracle.set_threads(1)
    n_q = w.n_seq * w.n_new
    return spent / done / n_q * 1e6, done


def cpu_baseline_decode(w, host, W, K, budget):
    """The oracle as it stands on the first decode steps of the same workload
    (one layer): on all usable host cores (OpenMP over the blocks of a score
    row, the heads of an attention call and the dirty entries of an update;
    each iteration's arithmetic and order unchanged), then on one thread."""
    hi = host_info()
    n = oracle_threads(hi)
    us_n, done_n = _decode_oracle_leg(w, host, W, K, budget, n)
    us_1, done_1 = _decode_oracle_leg(w, host, W, K, budget, 1)
    return {"value": round(us_n, 1), "unit": "us/token", "cores": n, "kind": "oracle",
            "sample": f"first {done_n} decode steps of one layer of {w.name} ({w.n_seq} seq), "
                      f"update+score+select+attend, fp32/fp64 C oracle, {n} OpenMP threads",
            "tokens_per_s": round(1e6 / us_n, 2),
            "single_thread": {"value": round(us_1, 1), "unit": "us/token", "cores": 1,
                              "sample": f"first {done_1} decode steps, 1 thread"},
            "host": hi}


def cpu_baseline_prefill(w, host, budget):
    """The oracle on one layer: the ubatch's pooled-key update, then bf16
    scores, selection and attention for as many of its queries as the budget
    allows, on all usable host cores; reported per query token."""
    import oracle
    hi = host_info()
    n = oracle_threads(hi)
    oracle.set_threads(n)
    kidx, k, v = host["kidx"], host["k"], host["v"]
    pooled = np.zeros((w.n_seq, w.cap_blocks, w.d), np.float32)
    n0 = np.full(w.n_seq, w.n_cells0, np.int32)
    pairs = [(0, b) for b in range(-(-w.n_cells0 // w.r))]
    oracle.update_pooled(kidx, n0, np.array(pairs, np.int32), pooled, w.r, w.theta, w.eps)
    t0 = time.perf_counter()
    oracle.update_pooled(kidx, host["nc_all"][0], host["dl_all"][0], pooled, w.r, w.theta,
                         w.eps)
    t_update = time.perf_counter() - t0
    qi, qq, qs, qp = host["qi"][0], host["qq"][0], host["qs"][0], host["qp"][0]
    done, spent = 0, 0.0
    for i in range(qp.shape[0]):
        t0 = time.perf_counter()
        oracle.step(qi[i:i + 1], qq[i:i + 1], qs[i:i + 1], qp[i:i + 1], pooled, k, v,
                    kv_type=w.kv_type, n_head_kv=w.Hk, r=w.r, top_k=w.top_k, theta=w.theta,
                    nb_out=w.nb_max(0), bf16_scores=True)
        spent += time.perf_counter() - t0
        done += 1
        if spent > budget:
            break
    oracle.set_threads(1)
    per_tok = spent / done + t_update / qp.shape[0]
    return {"value": round(1.0 / per_tok, 2), "unit": "t/s", "cores": n, "kind": "oracle",
            "sample": f"one layer of the prefill ubatch: its 128-block update, then {done} of "
                      f"{qp.shape[0]} queries (bf16 scores, selection, attention), fp32/fp64 C "
                      f"oracle, {n} OpenMP threads", "host": hi}


# ---------------------------------------------------------------------------

def run_probe(args, torch, dev):
    """Floors for the kernels' access patterns: qsa_probe_stream_read over 4
    GiB (sustained HBM reads, streaming loads) and over 32 MiB from HBM once
    per launch (a single pass like the 250k-cell scoring stream); then
    qsa_probe_gather_prefill -- the prefill
    attention's K/V row gather without its arithmetic -- and
    qsa_sparse_attn_prefill itself on the 512-token ubatch's selections.
    Each figure: events around a graph replay of n launches on one stream."""
    from top_sparse_attention_pooled_amd import qsa, runtime
    stream = torch.cuda.Stream()
    n_sink = 8192  # a word per wavefront: no two wavefronts fold into one word
    sink = torch.zeros(n_sink, dtype=torch.int32, device=dev)

    def timed(fn, n):
        """us per launch: n launches captured in one HIP graph (no host gaps
        between them), replayed once to warm up, then between two events."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                fn()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            ev0.record(stream)
            g.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1000.0 / n

    out = {"probe": "memory-traffic floors", "unit": "GB/s and us per launch"}
    # sustained: one 4 GiB pass per launch
    buf = torch.empty(4096 << 20, dtype=torch.uint8, device=dev)
    nb = buf.numel()
    us = timed(lambda: qsa.probe_stream_read(buf, nb, sink, n_sink, stream=stream), 20)
    out["hbm_stream_read"] = {"bytes": nb, "us": round(us, 2), "GBps": round(nb / us / 1e3, 1)}
    del buf
    # one cold 32 MiB pass per launch (the size of the 250k-cell scoring
    # stream): 16 buffers in turn, 512 MiB in all, more than the 256 MB
    # last-level cache holds
    bufs32 = [torch.empty(32 << 20, dtype=torch.uint8, device=dev) for _ in range(16)]
    turn = [0]

    def one_pass():
        b = bufs32[turn[0] % 16]
        turn[0] += 1
        qsa.probe_stream_read(b, b.numel(), sink, n_sink, stream=stream)

    us = timed(one_pass, 64)
    out["hbm_32mib_cold_pass"] = {"bytes": 32 << 20, "us": round(us, 2),
                                  "GBps": round((32 << 20) / us / 1e3, 1)}
    del bufs32
    torch.cuda.empty_cache()
    # the prefill ubatch's selections, then the gather alone and the kernel
    w, layers, inp, host = setup(torch, dev, "prefill", 1, 0, 1)
    layer = layers[0]
    n_q, nb_max = inp["n_q"], inp["nb_max"]
    bf = runtime.StepBuffers(layer.dims, n_q, nb_max, dev, prefill=True)
    layer.n_cells = inp["n_cells"][0]
    d, sq = layer.dims, layer.seqs()
    qsa.score_select_prefill(d, sq, layer.kidx, inp["dirty"][0], inp["n_dirty"], layer.pooled,
                             layer.pooled_bf16, inp["q_idx"][0], inp["q_seq"][0],
                             inp["q_pos"][0], n_q, nb_max, bf.sel_blocks, bf.sel_cells,
                             bf.n_sel, bf.ws_pf, bf.ws_pf_bytes)
    torch.cuda.synchronize()
    n_sel = bf.n_sel.cpu().numpy().astype(np.int64)
    # rows loaded: every slot of every 32-cell chunk, K and V, per KV head
    rows = int(np.sum(-(-n_sel // 32) * 32)) * w.Hk * 2
    gbytes = rows * 272
    g_us = timed(lambda: qsa.probe_gather_prefill(d, sq, inp["q_seq"][0], n_q, layer.k, layer.v,
                                                  bf.sel_cells, bf.n_sel, sink, n_sink,
                                                  stream=stream), 20)
    a_us = timed(lambda: qsa.sparse_attn_prefill(d, sq, inp["q"][0], inp["q_seq"][0], n_q,
                                                 layer.k, layer.v, bf.sel_cells, bf.n_sel,
                                                 bf.out, bf.ws_attn, bf.ws_attn_bytes,
                                                 stream=stream), 20)
    distinct = int(np.unique(bf.sel_cells.cpu().numpy()[bf.sel_cells.cpu().numpy() >= 0]).size)
    out["prefill_gather"] = {"rows_loaded": rows, "bytes": gbytes, "us": round(g_us, 2),
                             "GBps": round(gbytes / g_us / 1e3, 1),
                             "distinct_cells": distinct,
                             "distinct_bytes": distinct * w.Hk * 2 * 272}
    out["prefill_attn"] = {"us": round(a_us, 2), "GBps_of_gather": round(gbytes / a_us / 1e3, 1)}
    out["config"] = {"workload": "prefill", "ubatch": n_q, "n_kv": int(w.n_cells0),
                     "top_k": w.top_k, "kv_heads": w.Hk, "kv_type": "q8_0"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the QSA step is not sharded across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch

    from top_sparse_attention_pooled_amd import qsa

    qsa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload
    if args.probe:
        print(json.dumps(run_probe(args, torch, dev)), flush=True)
        return
    if name is None:  # the headline decode line, with the prefill ubatch in it
        result = run_decode(args, torch, dev, "decode250k")
        torch.cuda.empty_cache()
        pf, _, _ = run_prefill(args, torch, dev, "prefill", args.prefill_steps, 2)
        result["prefill_t_s"] = pf["t_s_per_layer"]
        result["prefill"] = pf
    elif name.startswith("verify"):
        result = run_verify(args, torch, dev, name)
    elif name.startswith("prefill"):
        pf, ms_per_step, w = run_prefill(args, torch, dev, name, args.steps, args.warmup)
        result = {
            "metric": METRIC, "value": pf["t_s_per_layer"], "unit": "t/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16 indexer (fp32 accumulate), fp16 attention operands over q8_0 KV "
                     "(fp32 accumulate)",
            "data": pf.pop("data"), "config": pf.pop("config"),
            "roofline": {
                "kernel": "qsa_score_select_prefill (its launches together), priced on the "
                          "dense query x block-key contraction",
                "timing": "events around a graph of the K*L indexer calls alone",
                "bound": "mfma",
                "achieved": pf["indexer_mfma"]["achieved_tflops"],
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": pf["indexer_mfma"]["frac"],
                "traffic": (recorded_call_traffic(name, PREFILL_INDEXER_KERNELS)
                            if name == "prefill" else None),
                "flops_per_launch": pf["indexer_mfma"]["flops_per_launch"],
                "avg_launch_us": pf["parts_us"].get("indexer"),
            },
            "prefill": pf,
        }
        if "cpu_baseline" in pf:
            result["cpu_baseline"] = pf.pop("cpu_baseline")
    else:
        result = run_decode(args, torch, dev, name)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
