"""GPU parity of the fused decode indexer calls (score+select, and
candidates then select+attend) against the oracle and against the separate
calls, with inputs built to drive every branch of its
selection: the common case, 64-block groups whose dropped keys compete (their
full key sets are re-admitted), so many such groups that the scores are
re-streamed, all-tied scores, and contexts with fewer blocks than the budget.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from top_sparse_attention_pooled_amd import qsa, runtime, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def aligned_cells(w, q_idx, p, blocks, kidx):
    """Make the given blocks score near the maximum for a query at position p:
    each of their cells holds the roped query rotated back to the block's
    position (numpy complex rotation; the oracle scores whatever results)."""
    d = w.d
    omega = w.theta ** (-2.0 * np.arange(d // 2) / d)
    z = (q_idx[:d // 2] + 1j * q_idx[d // 2:]) * np.exp(1j * p * omega)
    for b in blocks:
        zb = z * np.exp(-1j * b * w.r * omega)
        kidx[b * w.r:(b + 1) * w.r] = np.concatenate([zb.real, zb.imag]).astype(np.float32)


def run_case(name, w, n_cells, q_idx, kidx, n_q=3):
    """n_q queries at the last positions.  Three queries make the fused
    select+attend grid larger than the chip holds at once, so that call
    selects once per query and attends over the lists; one query runs the
    fused kernel, where every attention workgroup selects on its own."""
    say(f"fused select: {name} ({n_q} queries)")
    layer = runtime.Layer(w, DEV, kidx=kidx[None].copy() if kidx.ndim == 2 else kidx)
    layer.rebuild(np.array([n_cells], np.int32))
    ref_pooled = np.zeros((1, w.cap_blocks, w.d), np.float32)
    oracle.update_pooled(layer.kidx.cpu().numpy(), np.array([n_cells], np.int32),
                         np.array([(0, b) for b in range(-(-n_cells // w.r))], np.int32),
                         ref_pooled, w.r, w.theta, w.eps)
    positions = [p for p in range(n_cells - 1, n_cells - 1 - n_q, -1) if p >= 0]
    n_q = len(positions)
    qi = np.repeat(q_idx[None], n_q, axis=0).astype(np.float32)
    nb_max = -(-n_cells // w.r)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    q_seq, q_pos = t(np.zeros(n_q, np.int32)), t(np.array(positions, np.int32))
    fused = runtime.StepBuffers(layer.dims, n_q, nb_max, DEV)
    qsa.score_select_decode(layer.dims, layer.seqs(), None, None, 0, layer.pooled, None, t(qi),
                            q_seq, q_pos, n_q, nb_max, fused.scores, fused.ld, fused.sel_blocks,
                            fused.sel_cells, fused.n_sel, fused.ws_fused, fused.ws_fused_bytes)
    sep = runtime.StepBuffers(layer.dims, n_q, nb_max, DEV)
    qsa.score_blocks(layer.dims, layer.seqs(), t(qi), q_seq, q_pos, n_q, layer.pooled, None,
                     nb_max, sep.scores, sep.ld)
    qsa.select_topk_blocks(layer.dims, layer.seqs(), sep.scores, sep.ld, q_seq, q_pos, n_q,
                           nb_max, sep.sel_blocks, sep.sel_cells, sep.n_sel)
    # attention over the separate calls' selection, and the selection fused
    # into attention (each attention workgroup selects on its own)
    q = t(synth.normal((n_q, w.H, w.D), 95, 0, synth.T_Q))
    qsa.sparse_attn_decode(layer.dims, layer.seqs(), q, q_seq, n_q, layer.k, layer.v,
                           sep.sel_cells, sep.n_sel, sep.out, sep.ws_attn, sep.ws_attn_bytes)
    att = runtime.StepBuffers(layer.dims, n_q, nb_max, DEV)
    qsa.decode_score_candidates(layer.dims, layer.seqs(), None, None, 0, layer.pooled, None,
                                t(qi), q_seq, q_pos, n_q, nb_max, att.scores, att.ld,
                                att.ws_fused, att.ws_fused_bytes)
    qsa.decode_select_attend(layer.dims, layer.seqs(), q_seq, q_pos, n_q, nb_max, att.scores,
                             att.ld, att.sel_blocks, att.sel_cells, att.n_sel, att.ws_fused,
                             att.ws_fused_bytes, q, layer.k, layer.v, att.out, att.ws_attn,
                             att.ws_attn_bytes)
    torch.cuda.synchronize()
    for i, p in enumerate(positions):
        r_scores = oracle.score_query(qi[i], p, ref_pooled[0], nb_max, w.r, w.theta)
        rb, rc = oracle.select(r_scores, p, w.r, w.top_k)
        for bufs, label in ((fused, "fused"), (sep, "two-call"), (att, "select+attend")):
            gs = bufs.scores.cpu().numpy()[i, :nb_max]
            assert np.array_equal(gs.view(np.uint32), r_scores.view(np.uint32)), label
            gb = bufs.sel_blocks.cpu().numpy()[i]
            gc = bufs.sel_cells.cpu().numpy()[i]
            assert int(bufs.n_sel.cpu()[i]) == rc.size, (label, p)
            assert np.array_equal(gb[:rb.size], rb), (label, p)
            assert np.all(gb[rb.size:] == -1)
            assert np.array_equal(gc[:rc.size], rc), (label, p)
            assert np.all(gc[rc.size:] == -1)
    # same cells, same arithmetic: the fused attention output is identical
    assert np.array_equal(att.out.cpu().numpy().view(np.uint32),
                          sep.out.cpu().numpy().view(np.uint32))
    # the call only reads the candidate workspace: a second call over the
    # same candidates (no scoring call between) gives the same output
    att.out.fill_(float("nan"))
    qsa.decode_select_attend(layer.dims, layer.seqs(), q_seq, q_pos, n_q, nb_max, att.scores,
                             att.ld, att.sel_blocks, att.sel_cells, att.n_sel, att.ws_fused,
                             att.ws_fused_bytes, q, layer.k, layer.v, att.out, att.ws_attn,
                             att.ws_attn_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(att.out.cpu().numpy().view(np.uint32),
                          sep.out.cpu().numpy().view(np.uint32))
    return r_scores


def workload():
    return synth.Workload("fz", 95, 1, 40000, n_new=1, steps=1, top_k=2048)


@pytest.mark.parametrize("n_q", [3, 1])
def test_fused_common_case(n_q):
    w = workload()
    kidx = synth.make_kidx(w)[0]
    q = synth.normal((w.d,), 95, 0, synth.T_QIDX)
    run_case("i.i.d. keys", w, 40000, q, kidx, n_q)


@pytest.mark.parametrize("n_q", [3, 1])
def test_fused_expands_clustered_groups(n_q):
    w = workload()
    kidx = synth.make_kidx(w)[0]
    q = synth.normal((w.d,), 96, 0, synth.T_QIDX)
    aligned_cells(w, q, 39999, range(3000, 3700), kidx)  # 700 blocks over 12 groups of 64
    s = run_case("contiguous cluster (re-admits 12 groups)", w, 40000, q, kidx, n_q)
    kept, _ = oracle.select(s, 40000 - n_q, w.r, w.top_k)
    assert np.sum((kept >= 3000) & (kept < 3700)) >= 500  # the case really is clustered


@pytest.mark.parametrize("n_q", [3, 1])
def test_fused_streams_when_many_groups_compete(n_q):
    w = workload()
    kidx = synth.make_kidx(w)[0]
    q = synth.normal((w.d,), 97, 0, synth.T_QIDX)
    # 20 blocks at stride 3 in the first 64-block group of each of 36 spans
    # of 256: more than the 16 keys a group keeps at this context length, so
    # 36 groups (over the 32 re-admitted whole) compete
    blocks = [wg * 256 + 3 * j for wg in range(2, 38) for j in range(20)]
    aligned_cells(w, q, 39999, blocks, kidx)
    s = run_case("strided cluster (36 groups compete: re-stream)", w, 40000, q, kidx, n_q)
    kept, _ = oracle.select(s, 40000 - n_q, w.r, w.top_k)
    assert np.isin(kept, blocks).sum() >= 500


@pytest.mark.parametrize("n_q", [3, 1])
def test_fused_all_tied(n_q):
    w = workload()
    kidx = np.zeros((w.cap_cells, w.d), np.float32)  # every pooled key is 0: all scores tie
    q = synth.normal((w.d,), 98, 0, synth.T_QIDX)
    s = run_case("all scores equal", w, 40000, q, kidx, n_q)
    assert np.all(s[np.isfinite(s)] == 0)


@pytest.mark.parametrize("n_q", [3, 1])
def test_fused_fewer_blocks_than_budget(n_q):
    w = workload()
    kidx = synth.make_kidx(w)[0]
    q = synth.normal((w.d,), 99, 0, synth.T_QIDX)
    for n in (1, 3, 5, 1000, 2048, 2049, 8200):
        run_case(f"n_cells={n}", w, n, q, kidx, n_q)


def test_fused_readmits_a_group_at_250k():
    """248,278 cells (62,069 scored blocks): groups keep only their 6 best
    keys at this length.  Eight blocks of one group aligned with the query
    beat every other block, so that group's dropped key competes and its
    keys are re-admitted; one query runs the fused kernel (the bitmap path),
    three the per-query selection."""
    w = synth.Workload("fz250", 94, 1, 248278, n_new=1, steps=1, top_k=2048)
    kidx = synth.make_kidx(w)[0]
    q = synth.normal((w.d,), 94, 0, synth.T_QIDX)
    planted = [40000 + 5 * j for j in range(8)]  # one 64-block group (block 40000 // 64 * 64 on)
    assert len({b // 64 for b in planted}) == 1
    aligned_cells(w, q, 248277, planted, kidx)
    for n_q in (1, 3):
        s = run_case("one group with 8 winners at 250k", w, 248278, q, kidx, n_q)
        kept, _ = oracle.select(s, 248278 - n_q, w.r, w.top_k)
        assert np.isin(planted, kept).all()
