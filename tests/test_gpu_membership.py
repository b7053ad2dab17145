"""General block membership on the GPU: a unified per-cell store whose rows
sequences reach through a cell table, and the dirty blocks found by comparing
each block's member cells with those it was built from (llama.cpp issue
#28734, fix summary, "lever2": a structural compare that also catches
defrag, rollback and sequence edits).  Everything is checked against the
oracle on each sequence's gathered contiguous view."""
import sys

import numpy as np
import pytest
import torch

import oracle
from top_sparse_attention_pooled_amd import qsa, runtime, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
ATTN_TOL = 2e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Unified:
    """A workload's caches in one store of n_rows rows, sequence s's position
    p at row table[s][p] (a random permutation, with spare rows for moves)."""

    def __init__(self, w, seed, spare=4096):
        rng = np.random.default_rng(seed)
        self.w = w
        kidx = synth.make_kidx(w)
        k = synth.make_kv(w, synth.T_K)
        v = synth.make_kv(w, synth.T_V)
        n_pos = w.n_seq * w.cap_cells
        self.n_rows = n_pos + spare
        perm = rng.permutation(self.n_rows)
        self.table = perm[:n_pos].reshape(w.n_seq, w.cap_cells).astype(np.int32)
        self.free = list(perm[n_pos:])
        self.kidx = np.zeros((self.n_rows, w.d), kidx.dtype)
        self.kidx[self.table.reshape(-1)] = kidx.reshape(n_pos, w.d)
        self.k = np.zeros((self.n_rows,) + k.shape[2:], k.dtype)
        self.k[self.table.reshape(-1)] = k.reshape((n_pos,) + k.shape[2:])
        self.v = np.zeros((self.n_rows,) + v.shape[2:], v.dtype)
        self.v[self.table.reshape(-1)] = v.reshape((n_pos,) + v.shape[2:])
        self.layer = runtime.Layer(w, DEV, kidx=self.kidx, k=self.k, v=self.v)
        self.t_table = torch.from_numpy(self.table).to(DEV)
        lay = self.layer
        lay.seqs = lambda n_cells=None: qsa.Seqs(
            w.n_seq, w.cap_cells, lay.n_cells if n_cells is None else n_cells, self.t_table,
            self.n_rows)

    def views(self):
        """Each sequence's contiguous kidx, K and V (the oracle's inputs)."""
        t = self.table
        return self.kidx[t], self.k[t], self.v[t]

    def sync(self):
        """Push the host-side store and table to the device."""
        lay = self.layer
        lay.kidx.copy_(torch.from_numpy(self.kidx))
        lay.k.copy_(torch.from_numpy(self.k))
        lay.v.copy_(torch.from_numpy(self.v))
        self.t_table.copy_(torch.from_numpy(self.table))


def oracle_pooled(w, kidx_view, n_cells):
    pooled = np.zeros((w.n_seq, w.cap_blocks, w.d), np.float32)
    pairs = [(s, b) for s in range(w.n_seq) for b in range(-(-int(n_cells[s]) // w.r))]
    oracle.update_pooled(np.ascontiguousarray(kidx_view), np.asarray(n_cells, np.int32),
                         np.array(pairs, np.int32), pooled, w.r, w.theta, w.eps)
    return pooled


def check_pooled(u, n_cells):
    w = u.w
    g = u.layer.pooled_rows().cpu().numpy()
    ref = oracle_pooled(w, u.views()[0], n_cells)
    for s in range(w.n_seq):
        nb = -(-int(n_cells[s]) // w.r)
        assert np.array_equal(g[s, :nb].view(np.uint32), ref[s, :nb].view(np.uint32)), s


def test_unified_store_steps_match_oracle():
    """Decode steps through both decode paths and a prefill-path step, every
    row read through the cell table: selections bit for bit, attention within
    tolerance, pooled keys bit for bit."""
    w = synth.Workload("unified", 96, 3, 9001, n_new=1, steps=2, top_k=512)
    u = Unified(w, 96)
    say("unified store: 3 seqs x 9001 cells scattered over", u.n_rows, "rows")
    n0 = np.full(w.n_seq, w.n_cells0, np.int32)
    u.layer.rebuild(n0)
    check_pooled(u, n0)
    kidx_v, k_v, v_v = u.views()
    ref_pooled = oracle_pooled(w, kidx_v, n0)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    for step in range(w.steps):
        n = synth.n_cells_at(w, step)
        u.layer.set_n_cells(n)
        dirty = synth.dirty_blocks(w, step)
        q_idx, q, q_seq, q_pos = synth.make_queries(w, step)
        n_q = q_pos.size
        runs = {}
        for path in ("attend", "general"):
            bufs = runtime.StepBuffers(u.layer.dims, n_q, w.nb_max(step), DEV)
            runs[path] = runtime.run_step(u.layer, bufs, t(q_idx), t(q), t(q_seq), t(q_pos),
                                          t(dirty.reshape(-1)), dirty.shape[0], path=path)
        bufs = runtime.StepBuffers(u.layer.dims, n_q, w.nb_max(step), DEV, prefill=True)
        runs["prefill"] = runtime.run_step(u.layer, bufs, t(q_idx), t(q), t(q_seq), t(q_pos),
                                           t(dirty.reshape(-1)), dirty.shape[0],
                                           mode=qsa.SCORE_BF16, prefill=True, path="indexer")
        torch.cuda.synchronize()
        oracle.update_pooled(np.ascontiguousarray(kidx_v), n, dirty, ref_pooled, w.r, w.theta,
                             w.eps)
        for path, out in runs.items():
            ref = oracle.step(q_idx, q, q_seq, q_pos, ref_pooled, k_v, v_v, kv_type=w.kv_type,
                              n_head_kv=w.Hk, r=w.r, top_k=w.top_k, theta=w.theta,
                              nb_out=w.nb_max(step), bf16_scores=(path == "prefill"))
            gc, gn, go = out.sel_cells.cpu().numpy(), out.n_sel.cpu().numpy(), out.out.cpu().numpy()
            worst = 0.0
            for i in range(n_q):
                rc = ref["cells"][i]
                assert gn[i] == rc.size, (path, i)
                assert np.array_equal(gc[i, :rc.size], rc), (path, i)
                worst = max(worst, float(np.abs(go[i] - ref["out"][i]).max()))
            say(f"  step {step} {path}: worst attention error {worst:.2e}")
            assert worst <= ATTN_TOL
    check_pooled(u, synth.n_cells_at(w, w.steps - 1))


def _detect(u, snap, max_dirty):
    w = u.w
    dl = torch.empty(max(max_dirty, 1) * 2, dtype=torch.int32, device=DEV)
    found = torch.zeros(1, dtype=torch.int32, device=DEV)
    qsa.detect_dirty_blocks(u.layer.dims, u.layer.seqs(), snap, dl, max_dirty, found)
    torch.cuda.synchronize()
    pairs = dl.cpu().numpy().reshape(-1, 2)[:max_dirty]
    return pairs, int(found.cpu().numpy()[0]), dl


def _expect(u, n_cells, snap_host):
    return oracle.dirty_blocks(u.table, n_cells, snap_host, u.w.r)


def test_dirty_detection_follows_defrag_rollback_and_rewrite():
    w = synth.Workload("members", 97, 2, 3000, n_new=1, steps=1, top_k=256)
    u = Unified(w, 97)
    rng = np.random.default_rng(97)
    r = w.r
    snap = torch.zeros(w.n_seq * w.cap_blocks * (r + 1), dtype=torch.int32, device=DEV)
    snap_host = np.zeros((w.n_seq, w.cap_blocks, r + 1), np.int64)
    n = np.array([2999, 2602], np.int32)
    u.layer.set_n_cells(n)

    def round_trip(label, max_dirty):
        nonlocal snap_host
        want, snap_next = _expect(u, n, snap_host)
        pairs, found, dl = _detect(u, snap, max_dirty)
        got = sorted(tuple(p) for p in pairs if p[0] >= 0)
        say(f"  {label}: {found} changed blocks, list of {max_dirty}")
        assert found == len(want)
        assert got == sorted(want)
        assert np.all(pairs[len(want):] == -1)
        qsa.update_pooled_keys(u.layer.dims, u.layer.seqs(), u.layer.kidx, dl, max_dirty,
                               u.layer.pooled, u.layer.pooled_bf16)
        torch.cuda.synchronize()
        got_snap = snap.cpu().numpy().reshape(snap_host.shape)
        assert np.array_equal(got_snap, snap_next)
        snap_host = snap_next
        check_pooled(u, n)

    # 1. first call: every present block
    round_trip("first build", 2048)
    # 2. nothing changed
    pairs, found, _ = _detect(u, snap, 16)
    assert found == 0 and np.all(pairs == -1)
    # 3. defrag: 60 cells of both sequences move to spare rows
    for _ in range(60):
        s = int(rng.integers(0, w.n_seq))
        p = int(rng.integers(0, n[s]))
        new = int(u.free.pop())
        old = int(u.table[s, p])
        u.kidx[new], u.k[new], u.v[new] = u.kidx[old], u.k[old], u.v[old]
        u.table[s, p] = new
    u.sync()
    round_trip("defrag", 128)
    # 4. rollback of 9 cells of sequence 1, then 9 different cells written at
    #    those positions (fresh rows, new contents)
    n[1] -= 9
    u.layer.set_n_cells(n)
    round_trip("rollback", 8)
    for p in range(int(n[1]), int(n[1]) + 9):
        new = int(u.free.pop())
        u.kidx[new] = rng.standard_normal(w.d).astype(u.kidx.dtype)
        u.table[1, p] = new
    n[1] += 9
    u.sync()
    u.layer.set_n_cells(n)
    round_trip("rewrite", 8)
    # 5. more changes than the list holds: the rest is found by the next call
    for s in range(w.n_seq):
        for p in range(0, 40, r):
            new = int(u.free.pop())
            old = int(u.table[s, p])
            u.kidx[new] = u.kidx[old]
            u.table[s, p] = new
    u.sync()
    want, _ = _expect(u, n, snap_host)
    pairs, found, dl = _detect(u, snap, 4)
    assert found == len(want) == 20
    got = [tuple(p) for p in pairs]
    assert len(set(got)) == 4 and set(got) <= set(want)
    qsa.update_pooled_keys(u.layer.dims, u.layer.seqs(), u.layer.kidx, dl, 4, u.layer.pooled,
                           u.layer.pooled_bf16)
    pairs2, found2, dl2 = _detect(u, snap, 32)
    assert found2 == 16 and set(tuple(p) for p in pairs2[:16]) == set(want) - set(got)
    qsa.update_pooled_keys(u.layer.dims, u.layer.seqs(), u.layer.kidx, dl2, 32, u.layer.pooled,
                           u.layer.pooled_bf16)
    torch.cuda.synchronize()
    check_pooled(u, n)
