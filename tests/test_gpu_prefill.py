"""GPU parity of the prefill indexer (qsa_score_select_prefill): the exact
block top-k of many queries under the canonical order T over bf16-rounded
operands, computed from matrix-core scores plus exact rescoring, against the
oracle's T-ordered bf16 scores and full-sort selection -- bit for bit, on
mixed-sequence query tiles, small and early contexts, all-tied scores (the
path that rescores every block) and the 512-token ubatch at depth 198,628.
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


def oracle_pooled(w, kidx, n_cells):
    pooled = np.zeros((w.n_seq, w.cap_blocks, w.d), np.float32)
    pairs = [(s, b) for s in range(w.n_seq) for b in range(-(-int(n_cells[s]) // w.r))]
    oracle.update_pooled(kidx, np.asarray(n_cells, np.int32), np.array(pairs, np.int32),
                         pooled, w.r, w.theta, w.eps)
    return pooled


def run_prefill(w, layer, q_idx, q_seq, q_pos, nb_max, dirty=None):
    n_q = q_pos.size
    bufs = runtime.StepBuffers(layer.dims, n_q, nb_max, DEV, prefill=True)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    nd = 0 if dirty is None else dirty.shape[0]
    qsa.score_select_prefill(layer.dims, layer.seqs(), layer.kidx,
                             None if dirty is None else t(dirty.reshape(-1)), nd, layer.pooled,
                             layer.pooled_bf16, t(q_idx), t(q_seq), t(q_pos), n_q, nb_max,
                             bufs.sel_blocks, bufs.sel_cells, bufs.n_sel, bufs.ws_pf,
                             bufs.ws_pf_bytes)
    torch.cuda.synchronize()
    return bufs


def indexer_workspace(bufs, nb_max):
    """The indexer's intermediate arrays, as the library lays them out in the
    workspace (each 256-byte aligned, in this order): per query the
    largest matrix-core score of each 16-block subgroup [n_q][4 n_grp], the
    band threshold [n_q], the band mask of each 64-block group [n_q][n_grp],
    then the roped bf16 queries and the error bounds."""
    n_q = bufs.n_q
    n_grp = (nb_max + 255) // 256 * 4
    ws = bufs.ws_pf.cpu().numpy()
    off, views = 0, []
    for nbytes in (n_q * n_grp * 16, n_q * 4, n_q * n_grp * 8):
        views.append(ws[off:off + nbytes])
        off += (nbytes + 255) // 256 * 256
    smax = views[0].view(np.float32).reshape(n_q, 4 * n_grp)
    thr = views[1].view(np.float32)
    mask = views[2].view(np.uint64).reshape(n_q, n_grp)
    return smax, thr, mask


def check_workspace(w, ws, i, t_scores, q_idx_i, p, nb_max):
    """The band of query i against the oracle's T-order scores.  The
    matrix-core sums lie within Delta = 2^-15 |q| sqrt(d) (1 + 2^-8) of T's
    (the bound the band rests on, |q| of the roped bf16 query, gamma = 1), so:
    each causal subgroup's maximum is within Delta of T's and the others are
    -inf; the threshold lies between the B-th largest T maximum M_B less
    3 Delta and the two radix rounds' bin width (2^-12 |M_B|), and M_B less
    Delta (-inf with fewer than B subgroups); a block at least Delta above
    the threshold is in the mask, one more than Delta below it is not, and
    no block past the causal limit is.  The threshold is the library's own,
    bounded by the second check before the third uses it."""
    smax, thr, mask = ws
    nc = min(oracle.complete_blocks(p, w.r), nb_max)
    qr = oracle.round_bf16(oracle.rope(q_idx_i, p, w.theta)).astype(np.float64)
    delta = 2.0 ** -15 * np.sqrt((qr * qr).sum()) * np.sqrt(w.d) * (1 + 2.0 ** -8) * 1.001
    n_sub = -(-nc // 16)
    tpad = np.full(-(-max(nc, 1) // 64) * 64, -np.inf)
    tpad[:nc] = t_scores[:nc]
    tmax = tpad.reshape(-1, 16).max(axis=1)
    gm = smax[i, :tmax.size].astype(np.float64)
    assert np.all(np.isneginf(gm[n_sub:])), (i, "maxima past the causal limit")
    err = np.abs(gm[:n_sub] - tmax[:n_sub])
    assert np.all(err <= delta), (i, "subgroup maxima", float(err.max()), delta)
    B = w.top_k // w.r
    th = float(thr[i])
    if n_sub < B:
        assert th == -np.inf, (i, th)
    else:
        # out of range (the fp32 norm of q overflows or underflows, or Delta
        # leaves [2^-100, 2^100]): every causal block passes, threshold -inf
        qn = np.sqrt((qr * qr).sum())
        sure = 2.0 ** -60 < qn < 2.0 ** 60 and 2.0 ** -99 < delta < 2.0 ** 99
        if sure or th != -np.inf:
            m_b = float(np.sort(tmax[:n_sub])[::-1][B - 1])
            lo = m_b - 3.01 * delta - 2.0 ** -12 * abs(m_b)
            assert lo <= th <= m_b - 0.99 * delta, (i, "threshold", th, m_b, delta)
    n_g = -(-nc // 64)
    bits = (mask[i, :n_g, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)
    bits = bits.reshape(-1).astype(bool)
    blk = np.arange(bits.size)
    assert not np.any(bits[blk >= nc]), (i, "mask past the causal limit")
    must = (blk < nc) & (tpad[:bits.size] >= th + delta)
    never = (blk < nc) & (tpad[:bits.size] < th - delta)
    assert np.all(bits[must]), (i, "mask misses", int((must & ~bits).sum()))
    assert not np.any(bits[never]), (i, "mask extra", int((never & bits).sum()))


def check_against_oracle(w, bufs, ref_pooled, q_idx, q_seq, q_pos, nb_max, which):
    gb = bufs.sel_blocks.cpu().numpy()
    gc = bufs.sel_cells.cpu().numpy()
    gn = bufs.n_sel.cpu().numpy()
    ws = indexer_workspace(bufs, nb_max)
    for i in which:
        p = int(q_pos[i])
        if q_seq[i] < 0 or p < 0:
            assert gn[i] == 0
            continue
        r = oracle.score_query(q_idx[i], p, ref_pooled[q_seq[i]], nb_max, w.r, w.theta,
                               bf16=True)
        if oracle.complete_blocks(p, w.r) > 0:
            check_workspace(w, ws, i, r, q_idx[i], p, nb_max)
        rb, rc = oracle.select(r, p, w.r, w.top_k)
        assert gn[i] == rc.size, (i, gn[i], rc.size)
        assert np.array_equal(gb[i, :rb.size], rb), i
        assert np.all(gb[i, rb.size:] == -1), i
        assert np.array_equal(gc[i, :rc.size], rc), i
        assert np.all(gc[i, rc.size:] == -1), i


def test_prefill_selection_exact_mixed_sequences():
    """140 queries of two sequences (query tiles mix them), the ubatch's dirty
    blocks updated by the same call."""
    w = synth.Workload("pfx", 90, 2, 5000, n_new=70, steps=1, top_k=256)
    say("prefill select: 2 seqs x 70 new tokens at depth 5000")
    layer = runtime.Layer(w, DEV)
    kidx = layer.kidx.cpu().numpy()
    layer.rebuild(np.full(w.n_seq, w.n_cells0, np.int32))
    n = synth.n_cells_at(w, 0)
    layer.set_n_cells(n)
    dirty = synth.dirty_blocks(w, 0)
    q_idx, _, q_seq, q_pos = synth.make_queries(w, 0)
    nb_max = w.nb_max(0)
    bufs = run_prefill(w, layer, q_idx, q_seq, q_pos, nb_max, dirty)
    ref_pooled = oracle_pooled(w, kidx, n)
    check_against_oracle(w, bufs, ref_pooled, q_idx, q_seq, q_pos, nb_max, range(q_pos.size))


def test_prefill_selection_small_and_early_contexts():
    """Contexts shorter than the sample needs (every block is a candidate),
    positions before the first complete block (tail only), invalid queries."""
    w = synth.Workload("pfs", 91, 1, 3000, n_new=1, steps=1, top_k=256)
    layer = runtime.Layer(w, DEV)
    kidx = layer.kidx.cpu().numpy()
    layer.rebuild(np.array([3001], np.int32))
    q_pos = np.array([0, 1, 2, 3, 4, 7, 100, 255, 256, 257, 1000, 2047, 2048, 3000, -1, 5000],
                     np.int32)
    q_seq = np.zeros(q_pos.size, np.int32)
    q_idx = synth.normal((q_pos.size, w.d), 91, 0, synth.T_QIDX)
    nb_max = w.nb_max(0)
    bufs = run_prefill(w, layer, q_idx, q_seq, q_pos, nb_max)
    ref_pooled = oracle_pooled(w, kidx, np.array([3001]))
    gn = bufs.n_sel.cpu().numpy()
    assert gn[-1] == 0 and gn[-2] == 0  # p = -1 and p past the present cells
    check_against_oracle(w, bufs, ref_pooled, q_idx, q_seq, q_pos, nb_max,
                         range(q_pos.size - 2))


def test_prefill_selection_all_tied_rescoring_every_block():
    """Every pooled key zero: all scores tie at 0, every causal block passes
    the candidate threshold, more than the candidate list holds, so every
    block is rescored on each pass; ties go to the lower blocks."""
    w = synth.Workload("pft", 92, 1, 40000, n_new=8, steps=1, top_k=2048)
    kidx = np.zeros((1, w.cap_cells, w.d), np.float32)
    layer = runtime.Layer(w, DEV, kidx=kidx)
    n = synth.n_cells_at(w, 0)
    layer.rebuild(n)
    q_idx, _, q_seq, q_pos = synth.make_queries(w, 0)
    nb_max = w.nb_max(0)
    bufs = run_prefill(w, layer, q_idx, q_seq, q_pos, nb_max)
    ref_pooled = oracle_pooled(w, kidx, n)
    check_against_oracle(w, bufs, ref_pooled, q_idx, q_seq, q_pos, nb_max, range(q_pos.size))
    gb = bufs.sel_blocks.cpu().numpy()
    assert np.array_equal(gb[0], np.arange(512))  # the lowest blocks win every tie


@pytest.mark.parametrize("name", ["prefill", "prefill_ar1"])
def test_prefill_ubatch_at_depth(name):
    """The benchmarked prefill step: the 512-token ubatch at depth 198,628
    (128 dirty blocks), top_k 2048, q8_0 K/V.  All 512 selections against the
    oracle bit for bit; then qsa_sparse_attn_prefill over those lists, its
    outputs against the oracle's fp64 attention for 65 queries spread over the
    ubatch.  Also with AR(1) indexer queries (rho 0.9, selections only),
    whose neighbouring tokens select overlapping blocks."""
    w = synth.WORKLOADS[name]
    full = name == "prefill"
    say(f"{name}: 512-token ubatch at 198,628, all selections"
        + (", attention on 65 queries" if full else ""))
    kidx = synth.make_kidx(w)
    if full:
        k, v = synth.make_kv(w, synth.T_K), synth.make_kv(w, synth.T_V)
    else:
        k = v = np.zeros((1, 1, 1, 1), np.uint8)
    layer = runtime.Layer(w, DEV, kidx=kidx, k=k, v=v)
    layer.rebuild(np.full(1, w.n_cells0, np.int32))
    n = synth.n_cells_at(w, 0)
    layer.set_n_cells(n)
    dirty = synth.dirty_blocks(w, 0)
    assert int((dirty[:, 0] >= 0).sum()) == 128
    q_idx, q, q_seq, q_pos = synth.make_queries(w, 0)
    nb_max = w.nb_max(0)
    bufs = run_prefill(w, layer, q_idx, q_seq, q_pos, nb_max, dirty)
    ref_pooled = oracle_pooled(w, kidx, n)
    check_against_oracle(w, bufs, ref_pooled, q_idx, q_seq, q_pos, nb_max, range(q_pos.size))
    gn = bufs.n_sel.cpu().numpy()
    assert np.all(gn <= w.top_k + w.r - 1)
    assert np.all(gn >= w.top_k)  # every query sees more than top_k complete cells
    if not full:
        return
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    qsa.sparse_attn_prefill(layer.dims, layer.seqs(), t(q), t(q_seq), q_pos.size, layer.k,
                            layer.v, bufs.sel_cells, bufs.n_sel, bufs.out, bufs.ws_attn,
                            bufs.ws_attn_bytes)
    torch.cuda.synchronize()
    go = bufs.out.cpu().numpy()
    gc = bufs.sel_cells.cpu().numpy()
    worst = 0.0
    for i in list(range(0, 512, 8)) + [511]:
        r = oracle.attend(q[i], k[0], v[0], w.kv_type, gc[i, :gn[i]], w.Hk)
        worst = max(worst, float(np.abs(go[i] - r).max()))
    say(f"  attention on 65 queries: worst max-abs error {worst:.2e}")
    assert worst <= 2e-3


@pytest.mark.parametrize("depth", [100000, 520000])
def test_prefill_selection_long_contexts(depth):
    """Contexts of 25,000 and 130,000 blocks (the longest the indexer takes is
    131,072): the threshold step holds 32 and 128 subgroup maxima per lane
    (the 512-token ubatch at depth 198,628 takes 64, the small cases 16).
    Queries at the end of the context and at early positions of it."""
    w = synth.Workload("pfl", 96, 1, depth, n_new=6, steps=1, top_k=2048)
    say(f"prefill select: depth {depth}, 6 new tokens and 6 earlier positions")
    layer = runtime.Layer(w, DEV, k=np.zeros((1, 1, 1, 1), np.uint8),
                          v=np.zeros((1, 1, 1, 1), np.uint8))
    kidx = layer.kidx.cpu().numpy()
    n = synth.n_cells_at(w, 0)
    layer.rebuild(n)
    q_idx, _, q_seq, q_pos = synth.make_queries(w, 0)
    early = np.array([9000, 65535, 65536, depth // 2, depth - 3000, depth - 1], np.int32)
    q_pos = np.concatenate([q_pos, early])
    q_seq = np.zeros(q_pos.size, np.int32)
    q_idx = np.concatenate([q_idx, synth.normal((early.size, w.d), 96, 0, synth.T_QIDX, 1)])
    nb_max = w.nb_max(0)
    bufs = run_prefill(w, layer, q_idx, q_seq, q_pos, nb_max)
    ref_pooled = oracle_pooled(w, kidx, n)
    check_against_oracle(w, bufs, ref_pooled, q_idx, q_seq, q_pos, nb_max, range(q_pos.size))


def test_prefill_selection_extreme_query_norms():
    """Queries scaled far up and far down: their error bound Delta leaves the
    range where no partial sum can overflow or underflow, so every causal
    block is rescored in order T; ordinary queries beside them take the
    band path."""
    w = synth.Workload("pfn", 94, 1, 20000, n_new=12, steps=1, top_k=512)
    kidx = synth.make_kidx(w)
    layer = runtime.Layer(w, DEV, kidx=kidx)
    n = synth.n_cells_at(w, 0)
    layer.rebuild(n)
    q_idx, _, q_seq, q_pos = synth.make_queries(w, 0)
    q_idx = q_idx.copy()
    q_idx[0] *= 1e33
    q_idx[1] *= 1e-33
    q_idx[2] *= 1e30
    nb_max = w.nb_max(0)
    bufs = run_prefill(w, layer, q_idx, q_seq, q_pos, nb_max)
    ref_pooled = oracle_pooled(w, kidx, n)
    check_against_oracle(w, bufs, ref_pooled, q_idx, q_seq, q_pos, nb_max, range(q_pos.size))


def test_prefill_selection_no_scored_blocks():
    """nb_max = 0: no block competes, every query keeps only its tail."""
    w = synth.Workload("pfz", 95, 1, 3000, n_new=6, steps=1, top_k=256)
    layer = runtime.Layer(w, DEV)
    n = synth.n_cells_at(w, 0)
    layer.rebuild(n)
    q_idx, _, q_seq, q_pos = synth.make_queries(w, 0)
    bufs = run_prefill(w, layer, q_idx, q_seq, q_pos, 0)
    gb = bufs.sel_blocks.cpu().numpy()
    gc = bufs.sel_cells.cpu().numpy()
    gn = bufs.n_sel.cpu().numpy()
    for i, p in enumerate(q_pos):
        nc = (int(p) + 1) // w.r
        tail = np.arange(nc * w.r, int(p) + 1, dtype=np.int32)
        assert gn[i] == tail.size
        assert np.all(gb[i] == -1)
        assert np.array_equal(gc[i, :tail.size], tail)
        assert np.all(gc[i, tail.size:] == -1)


def test_prefill_step_end_to_end():
    """A whole prefill step through the ABI (exact indexer, then attention on
    the matrix cores) against the oracle's step with T-ordered bf16 scores:
    selections bit for bit, outputs within the attention tolerance."""
    w = synth.Workload("pfe", 93, 2, 6000, n_new=40, steps=1, top_k=512)
    say("prefill step: 2 seqs x 40 new tokens at depth 6000, q8_0 KV")
    kidx = synth.make_kidx(w)
    k = synth.make_kv(w, synth.T_K)
    v = synth.make_kv(w, synth.T_V)
    layer = runtime.Layer(w, DEV, kidx=kidx, k=k, v=v)
    layer.rebuild(np.full(w.n_seq, w.n_cells0, np.int32))
    n = synth.n_cells_at(w, 0)
    layer.set_n_cells(n)
    dirty = synth.dirty_blocks(w, 0)
    q_idx, q, q_seq, q_pos = synth.make_queries(w, 0)
    nb_max = w.nb_max(0)
    bufs = runtime.StepBuffers(layer.dims, q_pos.size, nb_max, DEV, prefill=True)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    out = runtime.run_step(layer, bufs, t(q_idx), t(q), t(q_seq), t(q_pos),
                           t(dirty.reshape(-1)), dirty.shape[0], mode=qsa.SCORE_BF16,
                           prefill=True, path="indexer")
    torch.cuda.synchronize()
    ref_pooled = oracle_pooled(w, kidx, n)
    ref = oracle.step(q_idx, q, q_seq, q_pos, ref_pooled, k, v, kv_type=w.kv_type,
                      n_head_kv=w.Hk, r=w.r, top_k=w.top_k, theta=w.theta, nb_out=nb_max,
                      bf16_scores=True)
    gb, gc = out.sel_blocks.cpu().numpy(), out.sel_cells.cpu().numpy()
    gn, go = out.n_sel.cpu().numpy(), out.out.cpu().numpy()
    worst = 0.0
    for i in range(q_pos.size):
        rb, rc = ref["blocks"][i], ref["cells"][i]
        assert gn[i] == rc.size
        assert np.array_equal(gb[i, :rb.size], rb)
        assert np.array_equal(gc[i, :rc.size], rc)
        worst = max(worst, float(np.abs(go[i] - ref["out"][i]).max()))
    say(f"  worst attention error {worst:.2e} (fp16 operands, fp32 sums)")
    assert worst <= 2e-3


def test_mixed_step_prefill_chunk_beside_decode_tokens():
    """One launch sequence serving a 256-token prefill chunk of one session
    next to a decode token of each of three other sessions at other depths
    (the llama.cpp-multigpu README, on mixed prefill and generation: prompts
    are prefilled in 256-token chunks beside the decoding slots).  Every query
    is scored against its own session's blocks only.  Each query's selection
    bit for bit, outputs within the attention tolerance."""
    w = synth.Workload("mix", 95, 4, 7000, n_new=256, steps=1, top_k=512)
    say("mixed step: 256-token chunk of seq 0 + one decode token of seqs 1-3, q8_0 KV")
    kidx = synth.make_kidx(w)
    k = synth.make_kv(w, synth.T_K)
    v = synth.make_kv(w, synth.T_V)
    layer = runtime.Layer(w, DEV, kidx=kidx, k=k, v=v)
    n0 = np.array([7000, 6001, 4502, 6999], np.int32)
    layer.rebuild(n0)
    n = n0 + np.array([256, 1, 1, 1], np.int32)
    layer.set_n_cells(n)
    q_seq = np.concatenate([np.zeros(256, np.int32), np.arange(1, 4, dtype=np.int32)])
    q_pos = np.concatenate([np.arange(7000, 7256, dtype=np.int32), n0[1:]]).astype(np.int32)
    n_q = q_pos.size
    q_idx = synth.normal((n_q, w.d), 95, 0, synth.T_QIDX)
    q = synth.normal((n_q, w.H, w.D), 95, 0, synth.T_Q)
    pairs = [(0, b) for b in range(7000 // w.r, 7255 // w.r + 1)]
    pairs += [(s, int(n0[s]) // w.r) for s in range(1, 4)]
    m = 4
    while m < len(pairs):
        m *= 2
    dirty = np.asarray(pairs + [(-1, -1)] * (m - len(pairs)), np.int32)
    nb_max = int(-(-int(n.max()) // w.r))
    bufs = runtime.StepBuffers(layer.dims, n_q, nb_max, DEV, prefill=True)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    out = runtime.run_step(layer, bufs, t(q_idx), t(q), t(q_seq), t(q_pos),
                           t(dirty.reshape(-1)), dirty.shape[0], mode=qsa.SCORE_BF16,
                           prefill=True, path="indexer")
    torch.cuda.synchronize()
    ref_pooled = oracle_pooled(w, kidx, n)
    ref = oracle.step(q_idx, q, q_seq, q_pos, ref_pooled, k, v, kv_type=w.kv_type,
                      n_head_kv=w.Hk, r=w.r, top_k=w.top_k, theta=w.theta, nb_out=nb_max,
                      bf16_scores=True)
    gb, gc = out.sel_blocks.cpu().numpy(), out.sel_cells.cpu().numpy()
    gn, go = out.n_sel.cpu().numpy(), out.out.cpu().numpy()
    worst = 0.0
    for i in range(n_q):
        rb, rc = ref["blocks"][i], ref["cells"][i]
        assert gn[i] == rc.size, i
        assert np.array_equal(gb[i, :rb.size], rb), i
        assert np.array_equal(gc[i, :rc.size], rc), i
        worst = max(worst, float(np.abs(go[i] - ref["out"][i]).max()))
    say(f"  worst attention error {worst:.2e}")
    assert worst <= 2e-3
