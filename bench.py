#!/usr/bin/env python3
"""Benchmark of the QSA sparse-attention step on one MI355X.

A step is one decode token through the whole hot path -- pooled-key update,
block scoring, block top-k, sparse attention -- in each of 12 QSA layers (the
pages' model has 12 QSA layers; 12 replicas of one layer's caches at distinct
addresses also keep the ~400 MB working set out of the 256 MB last-level
cache, so the bytes come from HBM).  The K timed steps are captured in one
HIP graph and replayed; inputs are resident in HBM before timing starts.

Prints one JSON line.  value = microseconds per token per QSA layer (lower is
better); roofline = the dominant kernel (block scoring) against HBM peak;
cpu_baseline = the CPU oracle on a bounded sample of the same steps.
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
N_LAYERS = 12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode250k",
                    choices=["decode50k", "decode250k", "decode5x250k", "prefill", "prefill_ar1"])
    ap.add_argument("--kv", default="q8_0", choices=["q8_0", "f16"],
                    help="K/V cache type of a decode workload (the workloads are defined "
                         "with q8_0; f16 is the type the pages' first fix required)")
    ap.add_argument("--layers", type=int, default=N_LAYERS)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU-oracle baseline sample (0 = skip)")
    ap.add_argument("--profile", action="store_true",
                    help="short run for a profiler: no CPU baseline")
    ap.add_argument("--eager", action="store_true",
                    help="launch the steps directly instead of replaying a graph (for "
                         "hardware-counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also copy an MIB-MiB buffer once: a kernel of known traffic "
                         "that scales the byte counters")
    return ap.parse_args()


def algorithmic_bytes(w, step):
    """Bytes one layer-step must move at minimum, by kernel."""
    from top_sparse_attention_pooled_amd import synth
    n = w.n_cells0 + (step + 1) * w.n_new
    nc = n // w.r
    nb = w.nb_max(step)
    n_q = w.n_seq * w.n_new
    tail = n - nc * w.r
    n_sel = min(nc, w.top_k // w.r) * w.r + tail
    row = synth.row_bytes(w.kv_type, w.D)
    score = n_q * (nc * w.d * 4 + nb * 4 + w.d * 4)
    return {
        "score": score,
        "update": w.n_seq * (w.r * w.d * 4 + w.d * 4 + w.d * 2),
        "select": n_q * (nb * 4 + (w.top_k // w.r + w.ld_cells) * 4),
        "attn": n_q * (n_sel * w.Hk * row * 2 + 2 * w.H * w.D * 4 + n_sel * 4),
    }


def setup(args, torch, dev):
    """Caches of L layer replicas plus the per-step device inputs."""
    from top_sparse_attention_pooled_amd import runtime, synth
    w = synth.WORKLOADS[args.workload]
    K, W, L = args.steps, args.warmup, args.layers
    prefill = args.workload.startswith("prefill")
    if not prefill and K + W > w.steps:
        w = synth.Workload(**{**w.__dict__, "steps": K + W})
    if not prefill and args.kv == "f16":
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
    print(f"# inputs ready in {time.time() - t0:.1f}s ({args.workload}, {L} layer replicas)",
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


def timed_replay(args, torch, stream, enqueue, T, W):
    """W warm-up then K timed steps, replayed as one HIP graph (or launched
    directly with --eager); returns seconds for the K steps and the capture
    helper."""
    def capture(steps, **kw):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for t in steps:
                enqueue(t, **kw)
        return g

    if args.eager:
        with torch.cuda.stream(stream):
            for t in range(W):
                enqueue(t)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        with torch.cuda.stream(stream):
            for t in range(W, T):
                enqueue(t)
        torch.cuda.synchronize()
        return time.perf_counter() - t_start, capture
    g_warm = capture(range(W)) if W > 0 else None
    g_main = capture(range(W, T))
    torch.cuda.synchronize()
    if g_warm is not None:
        g_warm.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    g_main.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t_start, capture


def time_part(torch, stream, capture, T, W, n_launches, **kw):
    """Mean device time of one launch of a part of the step: a graph of just
    those launches over the timed steps, between two events on the stream
    (this runtime takes no event nodes inside a captured graph)."""
    g = capture(range(W, T), **kw)
    g.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1000.0 / n_launches


def calibration_copy(args, torch, dev):
    if args.copy_calibration:  # one streaming kernel of known traffic
        n = args.copy_calibration * (1 << 20) // 4
        src_buf = torch.ones(n, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        torch.neg(src_buf, out=dst_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf


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
    if args.workload.startswith("prefill"):
        result = run_prefill(args, torch, dev)
    else:
        result = run_decode(args, torch, dev)
    print(json.dumps(result), flush=True)


def run_decode(args, torch, dev):
    from top_sparse_attention_pooled_amd import qsa, runtime, synth
    w, layers, inp, host = setup(args, torch, dev)
    K, W, L = args.steps, args.warmup, args.layers
    T = W + K
    q_idx, q, q_seq, q_pos = inp["q_idx"], inp["q"], inp["q_seq"], inp["q_pos"]
    n_cells, dirty, n_dirty = inp["n_cells"], inp["dirty"], inp["n_dirty"]
    n_q, nb_max = inp["n_q"], inp["nb_max"]
    bufs = [runtime.StepBuffers(layers[0].dims, n_q, nb_max, dev) for _ in range(L)]
    stream = torch.cuda.Stream()

    def enqueue(t, only_score=False):
        """One decode token through every layer: update + scores + candidates,
        then selection fused into attention (+ the merge of partial states)."""
        for li, layer in enumerate(layers):
            layer.n_cells = n_cells[t]
            bf, d, sq = bufs[li], layer.dims, layer.seqs()
            qsa.decode_score_candidates(d, sq, layer.kidx, dirty[t], n_dirty, layer.pooled,
                                        layer.pooled_bf16, q_idx[t], q_seq[t], q_pos[t], n_q,
                                        nb_max, bf.scores, bf.ld, bf.ws_fused, bf.ws_fused_bytes)
            if only_score:
                continue
            qsa.decode_select_attend(d, sq, q_seq[t], q_pos[t], n_q, nb_max, bf.scores, bf.ld,
                                     bf.sel_blocks, bf.sel_cells, bf.n_sel, bf.ws_fused,
                                     bf.ws_fused_bytes, q[t], layer.k, layer.v, bf.out,
                                     bf.ws_attn, bf.ws_attn_bytes)

    calibration_copy(args, torch, dev)
    t_main, capture = timed_replay(args, torch, stream, enqueue, T, W)
    # live timing of the dominant kernel with HIP events on its stream
    score_us, timing = None, "eager run: not timed"
    if not args.eager:
        timing = "events around a graph of the K*L scoring launches alone"
        score_us = time_part(torch, stream, capture, T, W, K * L, only_score=True)

    # correctness guard on the last step of layer 0 (selection sizes)
    n_sel = bufs[0].n_sel.cpu().numpy()
    assert np.all(n_sel > 0), "empty selections in the benchmark step"

    ms_per_step = t_main * 1000.0 / K
    us_per_step_layer = ms_per_step * 1000.0 / L
    us_per_token_layer = us_per_step_layer / n_q  # n_q tokens per step (one per session)
    ab = [algorithmic_bytes(w, t) for t in range(W, T)]
    score_bytes = float(np.mean([a["score"] for a in ab]))
    step_bytes = float(np.mean([sum(a.values()) for a in ab]))
    achieved = score_bytes / (score_us * 1e-6) / 1e9 if score_us else None
    result = {
        "metric": "QSA sparse-attn decode \u00b5s/token and HBM GB/s at 250k ctx; prefill t/s",
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
            "workload": args.workload if args.kv == "q8_0" else f"{args.workload} (f16 KV)",
            "n_seq": w.n_seq, "n_kv_start": w.n_cells0 + w.n_new, "decode_steps": K,
            "q_heads": w.H, "kv_heads": w.Hk, "head_dim": w.D, "indexer_dim": w.d,
            "compress_ratio": w.r, "top_k": w.top_k,
            "layers_per_step": L, "graph_replay": not args.eager,
        },
        "tokens_per_s_per_layer": round(1e6 / us_per_token_layer, 1),
        "us_per_step_layer": round(us_per_step_layer, 3),
        "step_hbm_gbps": round(step_bytes / (us_per_step_layer * 1e-6) / 1e9, 1),
        "roofline": {
            "kernel": "k_score_cand",
            "timing": timing,
            "bound": "hbm",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
            "traffic": recorded_traffic(args.workload),
            "bytes_per_launch": round(score_bytes),
            "avg_launch_us": round(score_us, 3) if score_us else None,
        },
    }
    if not args.profile and args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, host, W, K, args.cpu_seconds)
    return result


def run_prefill(args, torch, dev):
    """One step = the 512-token ubatch at depth 198,628 through every layer:
    pooled-key update of its 128 dirty blocks, bf16 MFMA block scores,
    per-query exact block top-k, sparse attention per query."""
    from top_sparse_attention_pooled_amd import qsa, runtime, synth
    w, layers, inp, host = setup(args, torch, dev)
    K, W, L = args.steps, args.warmup, args.layers
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
    t_main, capture = timed_replay(args, torch, stream, enqueue, T, W)
    parts = {}
    if not args.eager:
        for part in ("indexer", "attn"):
            parts[part] = time_part(torch, stream, capture, T, W, K * L, part=part)
    n_sel = bufs[0].n_sel.cpu().numpy()
    assert np.all(n_sel > 0), "empty selections in the benchmark step"

    ms_per_step = t_main * 1000.0 / K
    us_per_layer = ms_per_step * 1000.0 / L
    pos = host["qp"][0]
    nc = (pos.astype(np.int64) + 1) // w.r
    flops = float(np.sum(nc)) * w.d * 2  # the dense query x block-key contraction
    score_us = parts.get("indexer")
    tflops = flops / (score_us * 1e-6) / 1e12 if score_us else None
    result = {
        "metric": "QSA sparse-attn decode \u00b5s/token and HBM GB/s at 250k ctx; prefill t/s",
        "value": round(n_q / (us_per_layer * 1e-6), 1),
        "unit": "t/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 indexer (fp32 accumulate), f32 attention over q8_0 KV",
        "data": ("synthetic: i.i.d. N(0,1) indexer keys, queries and K/V (q8_0-packed), seeded"
                 + ("; indexer queries AR(1) along the tokens, rho %g" % w.extra["qidx_ar1"]
                    if w.extra.get("qidx_ar1") else "")),
        "config": {
            "workload": args.workload, "n_seq": 1, "n_kv_start": w.n_cells0, "ubatch": n_q,
            "dirty_blocks": int(np.sum(host["dl_all"][0][:, 0] >= 0)),
            "q_heads": w.H, "kv_heads": w.Hk, "head_dim": w.D, "indexer_dim": w.d,
            "compress_ratio": w.r, "top_k": w.top_k, "layers_per_step": L,
            "graph_replay": not args.eager,
        },
        "us_per_layer": round(us_per_layer, 2),
        "model_prefill_t_s": round(n_q / (ms_per_step * 1e-3), 1),
        "parts_us": {k: round(v, 2) for k, v in parts.items()},
        "roofline": {
            "kernel": "qsa_score_select_prefill (update, rope, two MFMA passes: subgroup maxima, "
                      "then masks at tau - 2 Delta; exact rescoring of the masked blocks), priced "
                      "on the dense contraction once",
            "timing": "events around a graph of the K*L indexer calls alone",
            "bound": "mfma",
            "achieved": round(tflops, 2) if tflops else None,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4) if tflops else None,
            "traffic": None,
            "flops_per_launch": flops,
            "avg_launch_us": round(score_us, 3) if score_us else None,
        },
    }
    if not args.profile and args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_prefill(w, host, args.cpu_seconds)
    return result


def recorded_traffic(workload):
    """HBM-side bytes per scoring launch from the committed counter summary
    (two rocprofv3 --pmc runs, scaled by a streaming kernel of known size),
    or None if there is none or the kernel sources changed since."""
    from top_sparse_attention_pooled_amd import profiling
    path = os.path.join(ROOT, "profiles", f"k_score_cand_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != profiling.source_hash():
        return None
    return round(rec["traffic_bytes"])


def cpu_baseline(w, host, W, K, budget):
    """The oracle as it stands, single-threaded, on the first decode steps of
    the same workload (one layer): update, score, select, attend per step."""
    import oracle
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
    us = spent / done * 1e6
    return {"value": round(us, 1), "unit": "us/token", "cores": 1, "kind": "oracle",
            "sample": f"first {done} decode steps of one layer of {w.name} "
                      f"({w.n_seq} seq), update+score+select+attend, fp32/fp64 C oracle, "
                      f"1 thread", "tokens_per_s": round(1e6 / us, 2)}


def cpu_baseline_prefill(w, host, budget):
    """The oracle, single-threaded, on one layer: the ubatch's pooled-key
    update, then bf16 scores, selection and attention for as many of its
    queries as the budget allows; reported per query token."""
    import oracle
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
    per_tok = spent / done + t_update / qp.shape[0]
    return {"value": round(1.0 / per_tok, 2), "unit": "t/s", "cores": 1, "kind": "oracle",
            "sample": f"one layer of the prefill ubatch: its 128-block update, then {done} of "
                      f"{qp.shape[0]} queries (bf16 scores, selection, attention), fp32/fp64 C "
                      f"oracle, 1 thread"}


if __name__ == "__main__":
    main()
