"""GPU parity of qsa_sparse_attn_decode_union: several decode tokens per
sequence attended over the union of their cell lists, each K/V row staged
once for every token of its group that lists it (issue #28734, goodbadwolf's
comment, "Why the two phases disagree").  Each token's output against the
oracle's fp64 attention over that token's own list, and against
qsa_sparse_attn_prefill on the same lists (the same arithmetic, so near
equality), at 2, 3, 5 and 8 tokens per group, with lists that share most of
their cells, lists that share few, ragged groups, a token with no cells, an
invalid token, tokens of two sequences in one group and a list out of order.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from top_sparse_attention_pooled_amd import qsa, runtime, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATTN_TOL = 2e-3  # as for the prefill attention: fp16 operands, fp32 sums


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def token_lists(rng, n_present, n_tok, share, tail_pos):
    """Per-token ascending cell lists: a common draw of 2048 cells of which
    each token keeps a fraction `share`, the rest its own draws, plus the
    cells of its incomplete tail block (positions r*nc .. p)."""
    base = rng.choice(n_present - 8, size=2048, replace=False)
    out = []
    for t in range(n_tok):
        keep = rng.random(2048) < share
        own = rng.choice(n_present - 8, size=2048, replace=False)
        cells = np.unique(np.concatenate([base[keep], own[~keep][:int((~keep).sum())]]))
        p = tail_pos + t
        tail = np.arange(p - p % 4, p + 1)
        cells = np.unique(np.concatenate([cells, tail]))
        out.append(cells.astype(np.int32))
    return out


def run_both(layer, q, q_seq, cells, n_sel, t_group):
    n_q = q.shape[0]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    d, sq = layer.dims, layer.seqs()
    need = qsa.workspace_size(d, qsa.OP_ATTN_DECODE_UNION, n_q, t_group)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out_u = torch.full((n_q, d.n_head, d.head_dim), float("nan"), device=DEV)
    qsa.sparse_attn_decode_union(d, sq, t(q), t(q_seq), n_q, t_group, layer.k, layer.v,
                                 t(cells), t(n_sel), out_u, ws, need)
    bufs = runtime.StepBuffers(d, n_q, 64, DEV, prefill=True)
    qsa.sparse_attn_prefill(d, sq, t(q), t(q_seq), n_q, layer.k, layer.v, t(cells), t(n_sel),
                            bufs.out, bufs.ws_attn, bufs.ws_attn_bytes)
    torch.cuda.synchronize()
    return out_u.cpu().numpy(), bufs.out.cpu().numpy()


def check(w, layer, q, q_seq, cells, n_sel, n_present, t_group, what):
    g_u, g_p = run_both(layer, q, q_seq, cells, n_sel, t_group)
    k_np, v_np = layer.k.cpu().numpy(), layer.v.cpu().numpy()
    worst = worst_p = 0.0
    for i in range(q.shape[0]):
        s = int(q_seq[i])
        if s < 0 or s >= w.n_seq:
            assert np.all(g_u[i] == 0), (what, i)
            continue
        n = int(n_sel[i])
        c = cells[i, :n]
        c = c[(c >= 0) & (c < n_present[s])]
        r = oracle.attend(q[i], k_np[s], v_np[s], w.kv_type, c, w.Hk)
        err = float(np.abs(g_u[i] - r).max())
        worst = max(worst, err)
        assert err <= ATTN_TOL, (what, i, err)
        worst_p = max(worst_p, float(np.abs(g_u[i] - g_p[i]).max()))
    say(f"  {what}: worst vs oracle {worst:.2e}, vs prefill attention {worst_p:.2e}")
    assert worst_p <= 2e-4, (what, worst_p)


@pytest.mark.parametrize("t_group", [2, 3, 5, 8])
@pytest.mark.parametrize("share", [0.9, 0.1])
def test_union_matches_oracle(t_group, share):
    w = synth.Workload("uni", 60 + t_group, 2, 30000, n_new=1, steps=1)
    say(f"union decode attention: t_group {t_group}, shared fraction {share}")
    layer = runtime.Layer(w, DEV, kidx=np.zeros((w.n_seq, w.cap_cells, w.d), np.float32))
    n_present = np.array([30001, 29000], np.int32)
    layer.set_n_cells(n_present)
    rng = np.random.default_rng(1000 * t_group + int(share * 10))
    ld = w.ld_cells
    # two full groups of sequence 0 then a ragged one of sequence 1
    n_q = 2 * t_group + max(1, t_group - 1)
    q_seq = np.zeros(n_q, np.int32)
    q_seq[2 * t_group:] = 1
    cells = np.full((n_q, ld), -1, np.int32)
    n_sel = np.zeros(n_q, np.int32)
    for g0 in range(0, n_q, t_group):
        s = int(q_seq[g0])
        lists = token_lists(rng, int(n_present[s]), min(t_group, n_q - g0), share,
                            int(n_present[s]) - 8)
        for t, c in enumerate(lists):
            c = c[:ld]
            cells[g0 + t, :c.size] = c
            n_sel[g0 + t] = c.size
    q = synth.normal((n_q, w.H, w.D), 60 + t_group, 0, synth.T_Q)
    check(w, layer, q, q_seq, cells, n_sel, n_present, t_group, f"T={t_group} share={share}")


def test_union_edge_groups():
    """A token with no cells, an invalid token, a group mixing the two
    sequences, a list out of order and cells past the present ones (the
    mixed and unordered groups take the concatenated form)."""
    w = synth.Workload("une", 69, 2, 30000, n_new=1, steps=1)
    say("union decode attention: edge groups")
    layer = runtime.Layer(w, DEV, kidx=np.zeros((w.n_seq, w.cap_cells, w.d), np.float32))
    n_present = np.array([30001, 29000], np.int32)
    layer.set_n_cells(n_present)
    rng = np.random.default_rng(69)
    ld = w.ld_cells
    T = 4
    n_q = 4 * T
    q_seq = np.zeros(n_q, np.int32)
    q_seq[5] = -1             # group 1: an invalid token
    q_seq[8:12] = [0, 1, 0, 1]  # group 2: two sequences
    q_seq[12:] = 1
    cells = np.full((n_q, ld), -1, np.int32)
    n_sel = np.zeros(n_q, np.int32)
    for i in range(n_q):
        s = max(int(q_seq[i]), 0)
        n = 2048 if i != 1 else 0  # token 1: no cells
        c = np.sort(rng.choice(int(n_present[s]), size=n, replace=False)).astype(np.int32)
        if i == 13:  # group 3: one list out of order
            c = c[::-1].copy()
        if i == 14:  # cells past the present ones (ignored, as by every entry point)
            c[-5:] = np.arange(29990, 29995)
            c = np.sort(c)
        cells[i, :n] = c
        n_sel[i] = n
    q = synth.normal((n_q, w.H, w.D), 69, 0, synth.T_Q)
    check(w, layer, q, q_seq, cells, n_sel, n_present, T, "edge groups")
