"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on
the same seeded inputs.  Bars: selected block and cell sets bit-exact; pooled
keys within 1e-3 relative; attention outputs within 2e-3 max-abs (fp32
accumulation).  Decode scores must match to the last bit: both sides
multiply in fp32 and sum in the fixed order T, with RoPE angles from the same
fp64 inverse frequencies.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from top_sparse_attention_pooled_amd import qsa, runtime, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATTN_TOL = 2e-3
POOLED_REL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def f32_keys(kidx):
    """The oracle's input: per-cell keys as float32 (bf16 bits widened exactly)."""
    return synth.widen_kidx(kidx.view(np.uint16) if kidx.dtype == np.int16 else kidx)


def oracle_pooled(w, kidx, n_cells):
    kidx = f32_keys(kidx)
    pooled = np.zeros((w.n_seq, w.cap_blocks, w.d), np.float32)
    pairs = [(s, b) for s in range(w.n_seq) for b in range(-(-int(n_cells[s]) // w.r))]
    oracle.update_pooled(kidx, np.asarray(n_cells, np.int32), np.array(pairs, np.int32),
                         pooled, w.r, w.theta, w.eps)
    return pooled


def check_pooled(gpu_rows, ref, w, n_cells):
    n_exact = n_tot = 0
    for s in range(w.n_seq):
        nb = -(-int(n_cells[s]) // w.r)
        g, r = gpu_rows[s, :nb], ref[s, :nb]
        err = np.abs(g.astype(np.float64) - r)
        assert np.all(err <= POOLED_REL * np.abs(r) + 1e-6), (s, float(err.max()))
        n_exact += int(np.sum(g.view(np.uint32) == r.view(np.uint32)))
        n_tot += g.size
    return n_exact / max(n_tot, 1)


def check_scores(g, r):
    """g, r: score rows of equal length.  The -inf pattern and every finite
    value bit-identical; a mismatch is reported with its block and both
    values."""
    assert np.array_equal(np.isneginf(g), np.isneginf(r))
    fin = np.isfinite(r)
    bad = np.flatnonzero(fin & (g.view(np.uint32) != r.view(np.uint32)))
    assert bad.size == 0, [(int(b), float(g[b]), float(r[b])) for b in bad[:8]]
    return 1.0


def small_workload(n_seq=3, cfg_id=50, top_k=64, kv_type=synth.KV_Q8_0, H=16, Hk=2):
    return synth.Workload("small", cfg_id, n_seq, 4000, n_new=1, steps=200, H=H, Hk=Hk,
                          top_k=top_k, kv_type=kv_type)


# --------------------------------------------------------------------------
# pooled keys
# --------------------------------------------------------------------------

def test_pooled_keys_match_oracle_ragged():
    w = small_workload()
    say("pooled: 3 seqs, ragged lengths")
    layer = runtime.Layer(w, DEV)
    kidx = layer.kidx.cpu().numpy()
    n_cells = np.array([4001, 2, 1023], np.int32)  # 1-cell, 2-cell and 3-cell tails
    layer.rebuild(n_cells)
    torch.cuda.synchronize()
    ref = oracle_pooled(w, kidx, n_cells)
    frac = check_pooled(layer.pooled_rows().cpu().numpy(), ref, w, n_cells)
    say(f"  pooled bit-exact fraction {frac:.6f}")
    assert frac >= 0.999
    # bf16 copy is the RNE rounding of the fp32 keys
    g32 = layer.pooled_rows().cpu().numpy()
    gb = layer.pooled_bf16.view(w.n_seq, w.cap_blocks, w.d).cpu().numpy().view(np.uint16)
    for s in range(w.n_seq):
        nb = -(-int(n_cells[s]) // w.r)
        want = oracle.round_bf16(g32[s, :nb]).view(np.uint32) >> 16
        assert np.array_equal(gb[s, :nb].astype(np.uint32), want)


def test_pooled_keys_from_bf16_storage():
    """bf16 per-cell keys: the pooled keys are those of their exact f32
    widening, bit for bit like the f32 case, on ragged lengths."""
    w = synth.Workload("small_bf16", 52, 3, 4000, n_new=1, steps=200, top_k=64,
                       kidx_type=synth.KIDX_BF16)
    say("pooled: bf16 per-cell keys, 3 seqs, ragged lengths")
    layer = runtime.Layer(w, DEV)
    assert layer.kidx.dtype == torch.int16
    kidx = layer.kidx.cpu().numpy()
    n_cells = np.array([4001, 3, 2046], np.int32)
    layer.rebuild(n_cells)
    torch.cuda.synchronize()
    ref = oracle_pooled(w, kidx, n_cells)
    frac = check_pooled(layer.pooled_rows().cpu().numpy(), ref, w, n_cells)
    say(f"  pooled bit-exact fraction {frac:.6f}")
    assert frac >= 0.999


def test_incremental_update_equals_full_rebuild():
    w = small_workload(n_seq=2, cfg_id=51)
    say("pooled: incremental appends vs full rebuild")
    layer = runtime.Layer(w, DEV)
    kidx = layer.kidx.cpu().numpy()
    n0 = np.full(w.n_seq, w.n_cells0, np.int32)
    layer.rebuild(n0)
    for step in range(9):
        n = synth.n_cells_at(w, step)
        layer.set_n_cells(n)
        dl = torch.from_numpy(synth.dirty_blocks(w, step).reshape(-1)).to(DEV)
        qsa.update_pooled_keys(layer.dims, layer.seqs(), layer.kidx, dl, dl.numel() // 2,
                               layer.pooled, layer.pooled_bf16)
    torch.cuda.synchronize()
    inc = layer.pooled_rows().cpu().numpy()
    full = runtime.Layer.clone_of(layer)
    full.pooled.zero_()
    full.rebuild(n)
    torch.cuda.synchronize()
    assert np.array_equal(inc.view(np.uint32), full.pooled_rows().cpu().numpy().view(np.uint32))
    check_pooled(inc, oracle_pooled(w, kidx, n), w, n)


# --------------------------------------------------------------------------
# scores
# --------------------------------------------------------------------------

def test_decode_scores_match_oracle():
    w = small_workload(n_seq=2, cfg_id=52)
    say("scores: fp32 decode, positions incl. early and block edges")
    layer = runtime.Layer(w, DEV)
    kidx = layer.kidx.cpu().numpy()
    n_cells = np.array([4100, 3000], np.int32)
    layer.rebuild(n_cells)
    ref_pooled = oracle_pooled(w, kidx, n_cells)
    positions = [(0, 0), (0, 1), (0, 2), (0, 3), (0, 4), (0, 255), (0, 256), (0, 4099),
                 (1, 2999), (1, 1234), (1, 64 * 4 * 3 - 1)]
    n_q = len(positions)
    q_idx = synth.normal((n_q, w.d), 52, 0, synth.T_QIDX)
    q_seq = np.array([p[0] for p in positions], np.int32)
    q_pos = np.array([p[1] for p in positions], np.int32)
    nb_max = 1030
    bufs = runtime.StepBuffers(layer.dims, n_q, nb_max, DEV)
    qsa.score_blocks(layer.dims, layer.seqs(), torch.from_numpy(q_idx).to(DEV),
                     torch.from_numpy(q_seq).to(DEV), torch.from_numpy(q_pos).to(DEV), n_q,
                     layer.pooled, layer.pooled_bf16, nb_max, bufs.scores, bufs.ld)
    torch.cuda.synchronize()
    g = bufs.scores.cpu().numpy()[:, :nb_max]
    for i in range(n_q):
        r = oracle.score_query(q_idx[i], int(q_pos[i]), ref_pooled[q_seq[i]], nb_max, w.r,
                               w.theta)
        check_scores(g[i], r)


# --------------------------------------------------------------------------
# selection, on identical score inputs
# --------------------------------------------------------------------------

def _score_cases(rng):
    cases = []
    for nb, top_k in [(1, 8), (2, 4), (63, 16), (64, 256), (65, 256), (1000, 256),
                      (5000, 2048), (62070, 2048), (20000, 16384)]:
        for kind in ("normal", "ties", "sorted", "equal", "special"):
            s = rng.standard_normal(nb).astype(np.float32) * 10
            if kind == "ties":
                s = np.round(s).astype(np.float32)
            elif kind == "sorted":
                s = np.sort(s)
            elif kind == "equal":
                s[:] = 1.5
            elif kind == "special":
                s[rng.integers(0, nb, size=max(1, nb // 7))] = -0.0
                s[rng.integers(0, nb, size=max(1, nb // 11))] = 0.0
                s[rng.integers(0, nb, size=max(1, nb // 13))] = np.nan
                s[rng.integers(0, nb, size=max(1, nb // 17))] = np.inf
                s[rng.integers(0, nb, size=max(1, nb // 19))] = -np.inf
            cases.append((s, top_k))
    return cases


def test_select_matches_oracle_on_shared_scores():
    rng = np.random.default_rng(60)
    say("select: shared scores, ties / signed zero / non-finite / sorted / equal")
    for s_row, top_k in _score_cases(rng):
        nb = s_row.size
        w = synth.Workload("sel", 60, 1, 0, top_k=top_k)
        dims = runtime.dims_of(w)
        # several query positions: full context, mid-block tails, early
        positions = sorted({nb * 4 - 1, nb * 4 - 2, max(0, nb * 4 - 3), nb * 2 + 1, 0, 2})
        positions = [p for p in positions if 0 <= p < nb * 4]
        n_q = len(positions)
        cap = synth.round_up(nb * 4 + 4, 256)
        ld = synth.round_up(nb, 64)
        scores = np.zeros((n_q, ld), np.float32)
        scores[:, :nb] = s_row
        n_cells = torch.tensor([nb * 4], dtype=torch.int32, device=DEV)
        seqs = qsa.Seqs(1, cap, n_cells)
        B = top_k // 4
        sel_b = torch.empty(n_q, B, dtype=torch.int32, device=DEV)
        sel_c = torch.empty(n_q, top_k + 3, dtype=torch.int32, device=DEV)
        n_sel = torch.empty(n_q, dtype=torch.int32, device=DEV)
        qsa.select_topk_blocks(dims, seqs, torch.from_numpy(scores).to(DEV), ld,
                               torch.zeros(n_q, dtype=torch.int32, device=DEV),
                               torch.tensor(positions, dtype=torch.int32, device=DEV), n_q, nb,
                               sel_b, sel_c, n_sel)
        torch.cuda.synchronize()
        gb, gc, gn = sel_b.cpu().numpy(), sel_c.cpu().numpy(), n_sel.cpu().numpy()
        for qi, p in enumerate(positions):
            rb, rc = oracle.select(s_row, p, 4, top_k)
            assert gn[qi] == rc.size, (nb, top_k, p)
            assert np.array_equal(gb[qi, :rb.size], rb), (nb, top_k, p)
            assert np.all(gb[qi, rb.size:] == -1)
            assert np.array_equal(gc[qi, :rc.size], rc), (nb, top_k, p)
            assert np.all(gc[qi, rc.size:] == -1)


def test_select_with_no_scored_blocks_reads_no_scores():
    """nb_max = 0 with no score row at all (NULL): no block competes, so the
    selection call must not read the row; every query keeps its tail cells
    only, as the oracle's selection over an empty row gives."""
    w = synth.Workload("sel0", 61, 1, 0, top_k=64)
    dims = runtime.dims_of(w)
    positions = [0, 1, 2, 3, 6, 4095]
    n_q = len(positions)
    seqs = qsa.Seqs(1, 4096, torch.tensor([4096], dtype=torch.int32, device=DEV))
    sel_b = torch.full((n_q, 16), 7, dtype=torch.int32, device=DEV)
    sel_c = torch.full((n_q, 64 + 3), 7, dtype=torch.int32, device=DEV)
    n_sel = torch.full((n_q,), 7, dtype=torch.int32, device=DEV)
    qsa.select_topk_blocks(dims, seqs, None, 0, torch.zeros(n_q, dtype=torch.int32, device=DEV),
                           torch.tensor(positions, dtype=torch.int32, device=DEV), n_q, 0,
                           sel_b, sel_c, n_sel)
    torch.cuda.synchronize()
    gb, gc, gn = sel_b.cpu().numpy(), sel_c.cpu().numpy(), n_sel.cpu().numpy()
    for qi, p in enumerate(positions):
        # no block below nb_max = 0 competes: the oracle's row is all -inf
        rb, rc = oracle.select(np.full(p // 4 + 1, -np.inf, np.float32), p, 4, 64)
        assert rb.size == 0 and gn[qi] == rc.size, (p, gn[qi], rc.size)
        assert np.all(gb[qi] == -1)
        assert np.array_equal(gc[qi, :rc.size], rc) and np.all(gc[qi, rc.size:] == -1)


# --------------------------------------------------------------------------
# attention, on identical cell lists
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kv_type,H,Hk", [(synth.KV_F32, 4, 1), (synth.KV_Q8_0, 16, 2),
                                          (synth.KV_Q8_0, 8, 4), (synth.KV_F32, 2, 2),
                                          (synth.KV_F16, 16, 2), (synth.KV_F16, 4, 1)])
def test_attention_matches_oracle_on_shared_cells(kv_type, H, Hk):
    w = synth.Workload("att", 70 + H, 2, 3000, n_new=1, steps=1, H=H, Hk=Hk, top_k=2048,
                       kv_type=kv_type)
    say(f"attention: kv_type={kv_type} H={H} Hk={Hk}")
    layer = runtime.Layer(w, DEV, kidx=np.zeros((w.n_seq, w.cap_cells, w.d), np.float32))
    n_cells = np.array([3001, 2500], np.int32)
    layer.set_n_cells(n_cells)
    rng = np.random.default_rng(70)
    sizes = [0, 1, 5, 63, 64, 65, 700, 2048, 2051]
    ld = w.ld_cells
    n_q = len(sizes)
    cells = np.full((n_q, ld), -1, np.int32)
    q_seq = np.array([i % 2 for i in range(n_q)], np.int32)
    for i, n in enumerate(sizes):
        c = np.sort(rng.choice(int(n_cells[q_seq[i]]), size=n, replace=False))
        cells[i, :n] = c
    q = synth.normal((n_q, H, w.D), 70, 0, synth.T_Q)
    k_np, v_np = layer.k.cpu().numpy(), layer.v.cpu().numpy()
    for entry in (qsa.sparse_attn_decode, qsa.sparse_attn_prefill):
        prefill = entry is qsa.sparse_attn_prefill
        bufs = runtime.StepBuffers(layer.dims, n_q, 64, DEV, prefill=prefill)
        entry(layer.dims, layer.seqs(), torch.from_numpy(q).to(DEV),
              torch.from_numpy(q_seq).to(DEV), n_q, layer.k, layer.v,
              torch.from_numpy(cells).to(DEV), torch.tensor(sizes, dtype=torch.int32, device=DEV),
              bufs.out, bufs.ws_attn, bufs.ws_attn_bytes)
        torch.cuda.synchronize()
        g = bufs.out.cpu().numpy()
        worst = 0.0
        for i, n in enumerate(sizes):
            r = oracle.attend(q[i], k_np[q_seq[i]], v_np[q_seq[i]], kv_type, cells[i, :n], Hk)
            err = float(np.abs(g[i] - r).max())
            worst = max(worst, err)
            assert err <= ATTN_TOL, (entry.__name__, n, err)
        say(f"  {entry.__name__}: worst max-abs error {worst:.2e}")
        # decode: fp32 operands and sums leave far more margin than the bar.
        # Prefill rounds Q*scale, K, V and P to fp16 for the matrix cores
        # (relative 2^-11 each): a one-cell set returns its V row rounded to
        # fp16, about 2.4e-4 * |v| off, so the bar itself applies.
        assert worst < (ATTN_TOL if prefill else 1e-4)


def test_decode_attention_on_the_longest_cell_lists():
    """The longest lists the ABI accepts: top_k/r = 4096 blocks of r = 16 cells
    (65,551 list positions, 2,049 runs of 32 cells, more runs than threads in
    a merge workgroup).  Sets of 40,000 and 33,001 cells (more than 32,768)
    and a one-cell set, q8_0 rows, against the oracle."""
    H, Hk = 4, 1
    w = synth.Workload("long", 75, 1, 40000, n_new=1, steps=1, H=H, Hk=Hk, r=16,
                       top_k=65536, kv_type=synth.KV_Q8_0)
    say(f"attention on long lists: ld_cells={w.ld_cells}")
    layer = runtime.Layer(w, DEV, kidx=np.zeros((w.n_seq, w.cap_cells, w.d), np.float32))
    n_cells = np.array([40000], np.int32)
    layer.set_n_cells(n_cells)
    rng = np.random.default_rng(75)
    sizes = [40000, 33001, 1]
    n_q, ld = len(sizes), w.ld_cells
    cells = np.full((n_q, ld), -1, np.int32)
    for i, n in enumerate(sizes):
        cells[i, :n] = np.sort(rng.choice(40000, size=n, replace=False))
    q_seq = np.zeros(n_q, np.int32)
    q = synth.normal((n_q, H, w.D), 75, 0, synth.T_Q)
    bufs = runtime.StepBuffers(layer.dims, n_q, 64, DEV)
    qsa.sparse_attn_decode(layer.dims, layer.seqs(), torch.from_numpy(q).to(DEV),
                           torch.from_numpy(q_seq).to(DEV), n_q, layer.k, layer.v,
                           torch.from_numpy(cells).to(DEV),
                           torch.tensor(sizes, dtype=torch.int32, device=DEV),
                           bufs.out, bufs.ws_attn, bufs.ws_attn_bytes)
    torch.cuda.synchronize()
    g = bufs.out.cpu().numpy()
    k_np, v_np = layer.k.cpu().numpy(), layer.v.cpu().numpy()
    worst = 0.0
    for i, n in enumerate(sizes):
        r = oracle.attend(q[i], k_np[0], v_np[0], w.kv_type, cells[i, :n], Hk)
        worst = max(worst, float(np.abs(g[i] - r).max()))
    say(f"  worst max-abs error {worst:.2e}")
    assert worst < 1e-4


# --------------------------------------------------------------------------
# whole steps on the benchmark workloads
# --------------------------------------------------------------------------

def _run_workload(name, steps, check_every=1, w=None, paths=("attend", "general")):
    """Steps of a workload through every call sequence in `paths` (each
    recomputes the same dirty blocks, so they can share the layer), each
    checked against the oracle: scores and selections bit-exact, attention
    within tolerance."""
    w = synth.WORKLOADS[name] if w is None else w
    say(f"end-to-end {name}: generating inputs")
    kidx = synth.make_kidx(w)
    k = synth.make_kv(w, synth.T_K)
    v = synth.make_kv(w, synth.T_V)
    layer = runtime.Layer(w, DEV, kidx=kidx, k=k, v=v)
    n0 = np.full(w.n_seq, w.n_cells0, np.int32)
    layer.rebuild(n0)
    ref_pooled = oracle_pooled(w, kidx, n0)
    worst = 0.0
    fracs = []
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    for step in range(steps):
        n = synth.n_cells_at(w, step)
        layer.set_n_cells(n)
        dirty = synth.dirty_blocks(w, step)
        q_idx, q, q_seq, q_pos = synth.make_queries(w, step)
        n_q = q_pos.size
        outs = {}
        for path in paths:
            bufs = runtime.StepBuffers(layer.dims, n_q, w.nb_max(step), DEV)
            outs[path] = runtime.run_step(layer, bufs, t(q_idx), t(q), t(q_seq), t(q_pos),
                                          t(dirty.reshape(-1)), dirty.shape[0], path=path)
        torch.cuda.synchronize()
        oracle.update_pooled(f32_keys(kidx), n, dirty, ref_pooled, w.r, w.theta, w.eps)
        if step % check_every:
            continue
        ref = oracle.step(q_idx, q, q_seq, q_pos, ref_pooled, k, v, kv_type=w.kv_type,
                          n_head_kv=w.Hk, r=w.r, top_k=w.top_k, theta=w.theta,
                          nb_out=w.nb_max(step))
        for path, out in outs.items():
            gs = out.scores.cpu().numpy()[:, :w.nb_max(step)]
            gb, gc = out.sel_blocks.cpu().numpy(), out.sel_cells.cpu().numpy()
            gn, go = out.n_sel.cpu().numpy(), out.out.cpu().numpy()
            for i in range(n_q):
                fracs.append(check_scores(gs[i], ref["scores"][i]))
                rb, rc = ref["blocks"][i], ref["cells"][i]
                assert gn[i] == rc.size, path
                assert np.array_equal(gb[i, :rb.size], rb), path
                assert np.all(gb[i, rb.size:] == -1), path
                assert np.array_equal(gc[i, :rc.size], rc), path
                assert np.all(gc[i, rc.size:] == -1), path
                worst = max(worst, float(np.abs(go[i] - ref["out"][i]).max()))
            assert worst <= ATTN_TOL, path
        # the call sequences run the same arithmetic: identical outputs
        first = outs[paths[0]]
        for path in paths[1:]:
            assert np.array_equal(outs[path].out.cpu().numpy().view(np.uint32),
                                  first.out.cpu().numpy().view(np.uint32)), path
    say(f"  {name} ({', '.join(paths)}): scores bit-exact {min(fracs):.6f}, "
        f"worst attention error {worst:.2e}")
    return w, layer


def test_end_to_end_tiny():
    w, _ = _run_workload("tiny", 1)
    assert w.top_k == 256


def test_end_to_end_decode50k():
    _run_workload("decode50k", 3)


def test_end_to_end_decode250k():
    _run_workload("decode250k", 5, check_every=2)


def test_end_to_end_decode5x250k():
    _run_workload("decode5x250k", 1)


def test_end_to_end_multi_token_decode():
    """Three new tokens per sequence per step (a short verify batch), two
    sequences: several queries share each dirty block."""
    w = synth.Workload("multi", 91, 2, 20001, n_new=3, steps=6)
    _run_workload("multi", 6, w=w)


def test_end_to_end_bf16_keys_decode():
    """bf16 per-cell indexer keys: the dirty block recomputed inside the
    scoring kernel and by the update call, both decode paths."""
    w = synth.Workload("bf16keys", 94, 2, 30001, n_new=1, steps=3,
                       kidx_type=synth.KIDX_BF16)
    _run_workload("bf16keys", 3, w=w)


def test_end_to_end_f16_kv_decode():
    """f16 KV, the type of the pages' first fix: two sequences, one token each
    per step, through both decode paths."""
    w = synth.Workload("f16", 93, 2, 30001, n_new=1, steps=3, kv_type=synth.KV_F16)
    _run_workload("f16", 3, w=w)


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_invalid_queries_are_inert():
    w = small_workload(n_seq=2, cfg_id=80, top_k=64)
    say("invalid queries: bad sequence, position past the present cells")
    layer = runtime.Layer(w, DEV)
    layer.rebuild(np.array([100, 50], np.int32))
    q_seq = np.array([0, 5, -1, 1, 1], np.int32)
    q_pos = np.array([99, 10, 10, 50, -3], np.int32)  # 2nd..5th invalid
    n_q = q_seq.size
    t = lambda x: torch.from_numpy(x).to(DEV)
    for path in runtime.PATHS:
        bufs = runtime.StepBuffers(layer.dims, n_q, 40, DEV)
        bufs.out.fill_(7.0)
        runtime.run_step(layer, bufs, t(synth.normal((n_q, w.d), 80, 0, 1)),
                         t(synth.normal((n_q, w.H, w.D), 80, 0, 2)), t(q_seq), t(q_pos),
                         None, 0, path=path)
        torch.cuda.synchronize()
        s = bufs.scores.cpu().numpy()[:, :40]
        assert np.all(np.isfinite(s[0, :25])) and np.all(np.isneginf(s[0, 25:])), path
        assert np.all(np.isneginf(s[1:])), path
        n_sel = bufs.n_sel.cpu().numpy()
        assert n_sel[0] == 16 * 4 and np.all(n_sel[1:] == 0), path  # top_k 64: 16 blocks
        assert np.all(bufs.sel_cells.cpu().numpy()[1:] == -1), path
        assert np.all(bufs.out.cpu().numpy()[1:] == 0.0), path


def test_repeat_runs_are_bit_identical():
    w = small_workload(n_seq=1, cfg_id=81, top_k=256)
    layer = runtime.Layer(w, DEV)
    layer.rebuild(np.array([4000], np.int32))
    t = lambda x: torch.from_numpy(x).to(DEV)
    n_q = 3
    args = (t(synth.normal((n_q, w.d), 81, 0, 1)), t(synth.normal((n_q, w.H, w.D), 81, 0, 2)),
            t(np.zeros(n_q, np.int32)), t(np.array([3999, 2000, 17], np.int32)))
    outs = []
    for path in ("attend", "attend", "general"):  # twice, then another call sequence
        bufs = runtime.StepBuffers(layer.dims, n_q, 1000, DEV)
        o = runtime.run_step(layer, bufs, *args, None, 0, path=path)
        torch.cuda.synchronize()
        # only columns < nb_max of the score rows are defined
        outs.append([x.cpu().numpy().copy()
                     for x in (o.scores[:, :1000], o.sel_cells, o.n_sel, o.out)])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


# --------------------------------------------------------------------------
# prefill scores on the matrix cores
# --------------------------------------------------------------------------

def test_prefill_bf16_scores_within_bound():
    w = synth.Workload("pf", 90, 2, 5000, n_new=70, steps=1, top_k=256)
    say("prefill: bf16 MFMA scores vs T-ordered bf16 oracle scores")
    layer = runtime.Layer(w, DEV)
    kidx = layer.kidx.cpu().numpy()
    n = synth.n_cells_at(w, 0)
    layer.rebuild(n)
    ref_pooled = oracle_pooled(w, kidx, n)
    q_idx, _, q_seq, q_pos = synth.make_queries(w, 0)
    n_q = q_pos.size  # 140 queries over 2 sequences: tiles mix sequences
    nb_max = w.nb_max(0)
    bufs = runtime.StepBuffers(layer.dims, n_q, nb_max, DEV, prefill=True)
    t = lambda x: torch.from_numpy(x).to(DEV)
    qsa.score_blocks(layer.dims, layer.seqs(), t(q_idx), t(q_seq), t(q_pos), n_q, layer.pooled,
                     layer.pooled_bf16, nb_max, bufs.scores, bufs.ld, qsa.SCORE_BF16,
                     bufs.ws_score, bufs.ws_score_bytes)
    torch.cuda.synchronize()
    g = bufs.scores.cpu().numpy()[:, :nb_max]
    worst = 0.0
    for i in range(n_q):
        r = oracle.score_query(q_idx[i], int(q_pos[i]), ref_pooled[q_seq[i]], nb_max, w.r,
                               w.theta, bf16=True)
        assert np.array_equal(np.isneginf(g[i]), np.isneginf(r))
        fin = np.isfinite(r)
        qh = oracle.round_bf16(oracle.rope(q_idx[i], int(q_pos[i]), w.theta)).astype(np.float64)
        kh = oracle.round_bf16(ref_pooled[q_seq[i], :fin.sum()]).astype(np.float64)
        bound = 2 * 127 * 2.0 ** -24 * np.abs(kh * qh[None]).sum(axis=1)
        diff = np.abs(g[i][fin].astype(np.float64) - r[fin])
        assert np.all(diff <= bound + 1e-30), i
        worst = max(worst, float((diff / np.maximum(bound, 1e-30)).max()))
    say(f"  worst |mfma - T| / bound = {worst:.3f}")
