"""CPU oracle for the QSA sparse-attention step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library: the arithmetic lives in ``qsa_oracle.c`` (plain C, built
with ``-ffp-contract=off``), and this module only moves numpy arrays across
ctypes and loops over queries.

What each function follows (pages cited by title and section):

* ``pooled_key`` / ``update_pooled`` / ``build_pooled`` -- the persistent
  pooled block-key cache: a block's cells are mean-pooled, RMS-normed and roped
  at the block position, and only dirtied blocks are recomputed (llama.cpp issue
  #28734, fix summary, "lever2").
* ``score_query`` -- block scoring with fully-future blocks at -inf and the
  incomplete tail left out of the competition (issue #28734, "lever3").
* ``select`` -- block-granular top-k expanded to cells, plus the tail cells
  (issue #28734, "lever3"); its capacity top_k + r - 1 is the n_kv_max that
  goodbadwolf's comment on the same issue derives.
* ``attend`` -- attention over only the selected cells, which is what passing
  the top-k width as n_kv_max buys (issue #28734, "lever1"); q8_0 rows are
  dequantised before use (discussion #30071, the two-problems paragraph).
* ``select_dense_cells`` / ``attend_dense_masked`` / full re-pooling -- the
  pages' own slow forms, kept as cross-checks.
* ``dirty_blocks`` -- which blocks to recompute: those whose member cells
  changed since they were built, found by comparing the members with a
  snapshot (issue #28734, fix summary, "lever2": the structural compare that
  also catches defrag, rollback and sequence edits).  With a cell table the
  method itself reads positions' contents; callers gather each sequence's
  rows into a contiguous view for the other functions.

Pins: every function here is checked against something other than itself in
``tests/test_oracle_pins.py`` (closed forms, library routines, brute force,
the equivalences the pages state).  Pooled-key element values and fp32 score
bits have no printed values on the pages to compare with; they are pinned by
invariants and by fp64 error bounds, as listed in that test file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "libqsa_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-unsafe-math-optimizations", "-fopenmp", "-Wall"]


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, f32, f64, vp = (ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                              ctypes.c_double, ctypes.c_void_p)
    sig = {
        "qo_set_threads": (i32, [i32]),
        "qo_half_to_float": (f32, [ctypes.c_uint16]),
        "qo_round_bf16": (f32, [f32]),
        "qo_tree_sum": (f32, [_f32p, i32]),
        "qo_tree_dot": (f32, [_f32p, _f32p, i32]),
        "qo_inv_freq": (i32, [f64, i32, _f64p]),
        "qo_rope_coeffs": (i32, [f64, i32, i64, _f32p, _f32p]),
        "qo_rope": (i32, [_f32p, i32, i64, f64, _f32p]),
        "qo_pooled_key": (i32, [_f32p, i32, i32, f32, _f32p, i64, f64, _f32p]),
        "qo_block_key": (i32, [_f32p, i64, i32, i32, f32, _f32p, f64, i64, _f32p]),
        "qo_update_pooled": (i32, [_f32p, i64, _i32p, i32, i32, i32, f32, _f32p,
                                   f64, _i32p, i32, _f32p, i64]),
        "qo_complete_blocks": (i64, [i64, i32]),
        "qo_score_query": (i32, [_f32p, i32, i64, f64, i32, _f32p, i64, i64, i32,
                                 _f32p]),
        "qo_select": (i32, [_f32p, i64, i32, i32, _i32p, _i32p, _i32p]),
        "qo_select_dense_cells": (i32, [_f32p, i64, i32, i32, _i32p]),
        "qo_attend": (i32, [_f32p, i32, i32, i32, vp, vp, i32, _i32p, i32, f32,
                            _f32p]),
        "qo_attend_dense_masked": (i32, [_f32p, i32, i32, i32, vp, vp, i32, _u8p,
                                         i64, f32, _f32p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a, ty):
    return a.ctypes.data_as(ty)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc < 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")
    return rc


# --------------------------------------------------------------------------
# scalars and building blocks
# --------------------------------------------------------------------------

def set_threads(n: int) -> int:
    """Threads of the oracle's parallel loops (update entries, score blocks,
    attention heads); returns the count in force.  Results do not depend on
    it: each iteration runs the single-threaded arithmetic in its order."""
    return int(_load().qo_set_threads(int(n)))


def half_to_float(bits: int) -> float:
    return float(_load().qo_half_to_float(int(bits)))


def round_bf16(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib.qo_round_bf16(float(v)) for v in x.ravel()],
                    dtype=np.float32).reshape(x.shape)


def tree_sum(v) -> np.float32:
    v = _c(v, np.float32).copy()
    return np.float32(_load().qo_tree_sum(_p(v, _f32p), v.size))


def tree_dot(a, b) -> np.float32:
    a, b = _c(a, np.float32), _c(b, np.float32)
    return np.float32(_load().qo_tree_dot(_p(a, _f32p), _p(b, _f32p), a.size))


def inv_freq(theta: float, d: int) -> np.ndarray:
    out = np.zeros(d // 2, dtype=np.float64)
    _check(_load().qo_inv_freq(theta, d, _p(out, _f64p)), "inv_freq")
    return out


def rope_coeffs(theta: float, d: int, pos: int):
    c = np.zeros(d // 2, dtype=np.float32)
    s = np.zeros(d // 2, dtype=np.float32)
    _check(_load().qo_rope_coeffs(theta, d, int(pos), _p(c, _f32p), _p(s, _f32p)),
           "rope_coeffs")
    return c, s


def rope(x, pos: int, theta: float) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.zeros_like(x)
    _check(_load().qo_rope(_p(x, _f32p), x.size, int(pos), theta, _p(out, _f32p)),
           "rope")
    return out


def pooled_key(cells, pos: int, theta: float, eps: float, gamma=None) -> np.ndarray:
    """Pooled key of one block from its m present cells ([m][d])."""
    cells = _c(cells, np.float32)
    m, d = cells.shape
    out = np.zeros(d, dtype=np.float32)
    g = None if gamma is None else _c(gamma, np.float32)
    _check(_load().qo_pooled_key(_p(cells, _f32p), m, d, eps,
                                 None if g is None else _p(g, _f32p), int(pos),
                                 theta, _p(out, _f32p)), "pooled_key")
    return out


# --------------------------------------------------------------------------
# the method's steps
# --------------------------------------------------------------------------

def update_pooled(kidx, n_cells, dirty, pooled, r: int, theta: float, eps: float,
                  gamma=None) -> None:
    """Recompute the listed (seq, block) pairs of ``pooled`` in place.

    kidx: [n_seq][cap_cells][d] f32; n_cells: [n_seq] i32; dirty: [n][2] i32;
    pooled: [n_seq][cap_blocks][d] f32 (row-major)."""
    assert kidx.dtype == np.float32 and kidx.flags.c_contiguous
    assert pooled.dtype == np.float32 and pooled.flags.c_contiguous
    n_seq, cap_cells, d = kidx.shape
    cap_blocks = pooled.shape[1]
    nc = _c(n_cells, np.int32)
    dl = _c(dirty, np.int32).reshape(-1, 2)
    g = None if gamma is None else _c(gamma, np.float32)
    _check(_load().qo_update_pooled(
        _p(kidx, _f32p), cap_cells, _p(nc, _i32p), n_seq, d, r, eps,
        None if g is None else _p(g, _f32p), theta, _p(dl, _i32p), dl.shape[0],
        _p(pooled, _f32p), cap_blocks), "update_pooled")


def build_pooled(kidx_seq, n_cells: int, r: int, theta: float, eps: float,
                 gamma=None) -> np.ndarray:
    """Every block of one sequence, each from scratch (the full re-pool)."""
    kidx_seq = _c(kidx_seq, np.float32)
    d = kidx_seq.shape[-1]
    nb = -(-n_cells // r)
    out = np.zeros((nb, d), dtype=np.float32)
    lib = _load()
    g = None if gamma is None else _c(gamma, np.float32)
    for b in range(nb):
        row = out[b]
        _check(lib.qo_block_key(_p(kidx_seq, _f32p), n_cells, d, r, eps,
                                None if g is None else _p(g, _f32p), theta, b,
                                row.ctypes.data_as(_f32p)), "block_key")
    return out


def complete_blocks(pos: int, r: int) -> int:
    return int(_load().qo_complete_blocks(int(pos), r))


def score_query(q_idx, pos: int, pooled_seq, nb_out: int, r: int, theta: float,
                bf16: bool = False) -> np.ndarray:
    """Scores of one query against one sequence's pooled keys ([nb][d])."""
    q_idx = _c(q_idx, np.float32)
    pooled_seq = _c(pooled_seq, np.float32)
    out = np.zeros(nb_out, dtype=np.float32)
    _check(_load().qo_score_query(_p(q_idx, _f32p), q_idx.size, int(pos), theta, r,
                                  _p(pooled_seq, _f32p), pooled_seq.shape[0],
                                  nb_out, int(bf16), _p(out, _f32p)), "score_query")
    return out


def select(scores, pos: int, r: int, top_k: int):
    """(sel_blocks, sel_cells) of one query; both ascending int32 arrays."""
    scores = _c(scores, np.float32)
    B = top_k // r
    blocks = np.full(max(B, 1), -1, dtype=np.int32)
    cells = np.full(top_k + r, -1, dtype=np.int32)
    nb = np.zeros(1, dtype=np.int32)
    n = _check(_load().qo_select(_p(scores, _f32p), int(pos), r, top_k,
                                 _p(blocks, _i32p), _p(cells, _i32p),
                                 _p(nb, _i32p)), "select")
    return blocks[:nb[0]].copy(), cells[:n].copy()


def select_dense_cells(scores, pos: int, r: int, top_k: int) -> np.ndarray:
    scores = _c(scores, np.float32)
    cells = np.full(top_k + r + 1, -1, dtype=np.int32)
    n = _check(_load().qo_select_dense_cells(_p(scores, _f32p), int(pos), r, top_k,
                                             _p(cells, _i32p)), "select_dense")
    return cells[:n].copy()


def attend(q, k_seq, v_seq, kv_type: int, cells, n_head_kv: int,
           scale: float = 0.0) -> np.ndarray:
    """fp64 attention of one query ([H][D]) over one sequence's listed cells.

    k_seq / v_seq: that sequence's cache rows, fp32 [cap][Hk][D], q8_0 uint8
    [cap][Hk][D/32*34] (kv_type 1) or binary16 [cap][Hk][D] (kv_type 2)."""
    q = _c(q, np.float32)
    H, D = q.shape
    cells = _c(cells, np.int32)
    k_seq = np.ascontiguousarray(k_seq)
    v_seq = np.ascontiguousarray(v_seq)
    out = np.zeros((H, D), dtype=np.float32)
    _check(_load().qo_attend(_p(q, _f32p), H, n_head_kv, D, k_seq.ctypes.data,
                             v_seq.ctypes.data, kv_type, _p(cells, _i32p),
                             cells.size, scale, _p(out, _f32p)), "attend")
    return out


def attend_dense_masked(q, k_seq, v_seq, kv_type: int, sel_mask, pos: int,
                        n_head_kv: int, scale: float = 0.0) -> np.ndarray:
    q = _c(q, np.float32)
    H, D = q.shape
    mask = _c(sel_mask, np.uint8)
    assert mask.size >= pos + 1
    k_seq = np.ascontiguousarray(k_seq)
    v_seq = np.ascontiguousarray(v_seq)
    out = np.zeros((H, D), dtype=np.float32)
    _check(_load().qo_attend_dense_masked(_p(q, _f32p), H, n_head_kv, D,
                                          k_seq.ctypes.data, v_seq.ctypes.data,
                                          kv_type, _p(mask, _u8p), int(pos), scale,
                                          _p(out, _f32p)), "attend_dense")
    return out


# --------------------------------------------------------------------------
# a whole step for a batch of queries
# --------------------------------------------------------------------------

def step(q_idx, q, q_seq, q_pos, pooled, k_cache, v_cache, *, kv_type: int,
         n_head_kv: int, r: int, top_k: int, theta: float, nb_out: int,
         bf16_scores: bool = False, scale: float = 0.0):
    """Scores, selection and attention for every query (after the pooled
    update).  pooled: [n_seq][cap_blocks][d] row-major; caches per sequence
    first.  Returns dict(scores [n_q][nb_out], blocks list, cells list,
    out [n_q][H][D])."""
    n_q = len(q_pos)
    scores = np.zeros((n_q, nb_out), dtype=np.float32)
    blocks, cells = [], []
    out = np.zeros(np.asarray(q).shape, dtype=np.float32)
    for i in range(n_q):
        s, p = int(q_seq[i]), int(q_pos[i])
        scores[i] = score_query(q_idx[i], p, pooled[s], nb_out, r, theta,
                                bf16=bf16_scores)
        b, c = select(scores[i], p, r, top_k)
        blocks.append(b)
        cells.append(c)
        out[i] = attend(q[i], k_cache[s], v_cache[s], kv_type, c, n_head_kv, scale)
    return {"scores": scores, "blocks": blocks, "cells": cells, "out": out}


def dirty_blocks(cell_rows, n_cells, snapshot, r: int):
    """Structural dirty detection.

    cell_rows: [n_seq][cap_cells] int, the row of each position of each
    sequence; n_cells: [n_seq] present positions; snapshot: [n_seq][cap_blocks]
    [r + 1] int, per block the member count and member rows it was last built
    from.  A block's members are the rows of its present positions b*r ..
    b*r + m - 1, m = min(r, n - b*r).  Returns (the (seq, block) pairs whose
    non-empty member list changed, in (seq, block) order; the updated
    snapshot, in which emptied blocks are recorded as empty)."""
    rows = np.asarray(cell_rows)
    snap = np.array(snapshot, copy=True)
    n_seq, cap_blocks = snap.shape[0], snap.shape[1]
    out = []
    for s in range(n_seq):
        n = int(n_cells[s])
        for b in range(cap_blocks):
            m = max(0, min(r, n - b * r))
            members = [int(rows[s][b * r + j]) for j in range(m)]
            old_m = int(snap[s][b][0])
            if old_m == m and [int(x) for x in snap[s][b][1:1 + m]] == members:
                continue
            snap[s][b][0] = m
            if m == 0:
                continue
            snap[s][b][1:1 + m] = members
            out.append((s, b))
    return out, snap
