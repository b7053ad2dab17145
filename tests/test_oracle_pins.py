"""Pins for the CPU oracle: each oracle function is checked against something
other than itself -- values derived from the pages, closed forms, library
routines (numpy, math.fsum, torch CPU in fp64), brute force on tiny inputs, and
the equivalences the pages state between the fast forms and their slow forms.

Which pin covers which oracle function:
  half_to_float      -> numpy float16 conversion of all 65,536 bit patterns
  round_bf16         -> torch's float32 -> bfloat16 conversion (RNE)
  tree_sum/tree_dot  -> hand-derived order fixtures, exact integer sums,
                        pairwise-summation error bound against math.fsum
  inv_freq           -> Python pow, and the closed form theta^(-1/2) = 1/100
  rope_coeffs/rope   -> numpy complex rotation, identity at position 0,
                        unit-vector sign convention, relative-position invariance
  pooled_key         -> torch rms_norm + numpy complex rotation (fp64), exact
                        scale invariance at eps = 0, unit RMS
  update_pooled      -> full re-pool of every block (the pages' slow form)
  score_query        -> -inf closed form, fp64 dot within the pairwise bound,
                        relative-position invariance, exact bf16 products
  select             -> numpy lexsort brute force, the dense cell-level sort
                        (the pages' slow form), page counts, capacity, ties
  attend             -> torch scaled_dot_product_attention in fp64, dense
                        masked attention (the pages' slow form), closed forms
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from top_sparse_attention_pooled_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
THETA = 1.0e4
EPS = 1.0e-6
U32 = 2.0 ** -24


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# scalars
# --------------------------------------------------------------------------

def test_half_to_float_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 37,
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 65504.0], dtype=np.float32),
        # exact ties between two bf16 values (low 16 bits = 0x8000)
        (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------
# T, the fixed summation order
# --------------------------------------------------------------------------

def test_tree_sum_order_fixtures():
    for case in _gold("tree_sum_order.json")["cases"]:
        v = np.zeros(case["n"], dtype=np.float32)
        for k, val in case["nonzero"].items():
            v[int(k)] = val
        assert float(oracle.tree_sum(v)) == case["stride_halving"]
        # the fixture really separates the orders: left to right differs
        acc = np.float32(0)
        for x in v:
            acc = np.float32(acc + x)
        assert float(acc) == case["left_to_right"]


def test_tree_sum_exact_integers():
    rng = np.random.default_rng(1)
    for n in (2, 8, 128, 1024):
        v = rng.integers(-1000, 1000, size=n).astype(np.float32)
        assert float(oracle.tree_sum(v)) == float(v.astype(np.int64).sum())


def test_tree_sum_error_bound_vs_fsum():
    rng = np.random.default_rng(2)
    for _ in range(200):
        v = (rng.standard_normal(128) * rng.uniform(0.1, 100)).astype(np.float32)
        exact = math.fsum(float(x) for x in v)
        k = 7  # log2(128) levels, each one rounding
        bound = k * U32 / (1 - k * U32) * float(np.abs(v.astype(np.float64)).sum())
        assert abs(float(oracle.tree_sum(v)) - exact) <= bound


def test_tree_dot_bound_vs_fp64_dot():
    rng = np.random.default_rng(3)
    for _ in range(200):
        a = rng.standard_normal(128).astype(np.float32)
        b = rng.standard_normal(128).astype(np.float32)
        exact = float(np.dot(a.astype(np.float64), b.astype(np.float64)))
        k = 8  # one rounding per product + 7 levels
        bound = k * U32 / (1 - k * U32) * float(np.abs(a.astype(np.float64) * b).sum())
        assert abs(float(oracle.tree_dot(a, b)) - exact) <= bound


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def test_inv_freq_vs_pow_and_closed_form():
    d = 128
    w = oracle.inv_freq(THETA, d)
    ref = np.array([THETA ** (-2.0 * t / d) for t in range(d // 2)])
    assert w[0] == 1.0
    assert w[32] == 1.0 / 100.0        # theta^(-1/2) = 1/sqrt(1e4)
    assert np.all(np.abs(w - ref) <= 8 * np.spacing(ref))
    assert np.all(np.diff(w) < 0)
    assert oracle._load().qo_inv_freq(THETA, 96, (np.zeros(48)).ctypes.data_as(
        oracle._f64p)) == -1  # d/2 must be a power of two


def test_rope_identity_at_zero():
    x = np.random.default_rng(4).standard_normal(128).astype(np.float32)
    c, s = oracle.rope_coeffs(THETA, 128, 0)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    assert np.array_equal(oracle.rope(x, 0, THETA), x)


def test_rope_is_complex_rotation_of_split_halves():
    rng = np.random.default_rng(6)
    d = 128
    omega = THETA ** (-2.0 * np.arange(d // 2) / d)
    for pos in (1, 7, 4095, 49677, 248277, 1 << 20):
        x = rng.standard_normal(d).astype(np.float32)
        z = (x[:64].astype(np.float64) + 1j * x[64:].astype(np.float64)) * \
            np.exp(1j * pos * omega)
        ref = np.concatenate([z.real, z.imag])
        got = oracle.rope(x, pos, THETA).astype(np.float64)
        # fp32 rounding of cos/sin and of 2 products + 1 add; the angle itself
        # differs from the pow-based one by a few ulp of pos*omega
        tol = 1e-6 * np.abs(x).max() * 4 + 4 * pos * 2.0 ** -52 * np.abs(x).max()
        assert np.max(np.abs(got - ref)) <= tol + 1e-6


def test_rope_unit_vector_sign():
    d, pos, t = 128, 3, 5
    e = np.zeros(d, dtype=np.float32)
    e[t] = 1.0
    out = oracle.rope(e, pos, THETA)
    phi = pos * THETA ** (-2.0 * t / d)
    nz = np.nonzero(out)[0].tolist()
    assert nz == [t, t + 64]
    assert abs(out[t] - math.cos(phi)) < 1e-7
    assert abs(out[t + 64] - math.sin(phi)) < 1e-7


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(7)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)
    for p, pk, delta in ((100, 40, 1000), (248277, 12, 4), (5, 5, 200000)):
        a = float(np.dot(oracle.rope(q, p, THETA).astype(np.float64),
                         oracle.rope(k, pk, THETA).astype(np.float64)))
        b = float(np.dot(oracle.rope(q, p + delta, THETA).astype(np.float64),
                         oracle.rope(k, pk + delta, THETA).astype(np.float64)))
        assert abs(a - b) <= 2e-4 * (1 + abs(a))


def test_rope_preserves_norm():
    x = np.random.default_rng(8).standard_normal(128).astype(np.float32)
    for pos in (0, 3, 1000, 248000):
        y = oracle.rope(x, pos, THETA)
        assert abs(np.linalg.norm(y.astype(np.float64)) -
                   np.linalg.norm(x.astype(np.float64))) < 1e-5


# --------------------------------------------------------------------------
# pooled key
# --------------------------------------------------------------------------

def _pooled_ref_fp64(cells, pos, eps, gamma=None):
    """mean -> torch rms_norm -> complex rotation, all fp64 library routines."""
    a = np.mean(cells.astype(np.float64), axis=0)
    w = None if gamma is None else torch.from_numpy(gamma.astype(np.float64))
    n = torch.nn.functional.rms_norm(torch.from_numpy(a)[None], (a.size,),
                                     weight=w, eps=eps)[0].numpy()
    d = a.size
    omega = THETA ** (-2.0 * np.arange(d // 2) / d)
    z = (n[:d // 2] + 1j * n[d // 2:]) * np.exp(1j * pos * omega)
    return np.concatenate([z.real, z.imag])


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_pooled_key_vs_fp64_libraries(m):
    rng = np.random.default_rng(10 + m)
    for trial in range(20):
        cells = rng.standard_normal((m, 128)).astype(np.float32)
        pos = int(rng.integers(0, 250000)) // 4 * 4
        gamma = None if trial % 2 else rng.uniform(0.5, 1.5, 128).astype(np.float32)
        got = oracle.pooled_key(cells, pos, THETA, EPS, gamma)
        ref = _pooled_ref_fp64(cells, pos, EPS, gamma)
        assert np.max(np.abs(got - ref)) <= 3e-6 * max(1.0, np.abs(ref).max()) + \
            4 * pos * 2.0 ** -52 * np.abs(ref).max()


def test_pooled_key_eps_matters_at_small_scale():
    """Cells whose mean square is comparable to eps: the eps term must enter
    exactly as rms_norm's does."""
    rng = np.random.default_rng(14)
    for scale in (1e-3, 3e-4):
        cells = (rng.standard_normal((4, 128)) * scale).astype(np.float32)
        got = oracle.pooled_key(cells, 4, THETA, EPS)
        ref = _pooled_ref_fp64(cells, 4, EPS)
        assert np.max(np.abs(got - ref)) <= 3e-6 * max(1.0, np.abs(ref).max())
        no_eps = _pooled_ref_fp64(cells, 4, 0.0)
        assert np.max(np.abs(no_eps - ref)) > 1e-2  # the case is sensitive


def test_pooled_key_scale_invariant_exactly():
    rng = np.random.default_rng(12)
    cells = rng.standard_normal((4, 128)).astype(np.float32)
    base = oracle.pooled_key(cells, 64, THETA, 0.0)
    for k in (-6, -1, 3, 10):
        scaled = (cells * np.float32(2.0 ** k)).astype(np.float32)
        assert np.array_equal(oracle.pooled_key(scaled, 64, THETA, 0.0), base)


def test_pooled_key_unit_rms_and_mean_semantics():
    rng = np.random.default_rng(13)
    cells = rng.standard_normal((4, 128)).astype(np.float32)
    y = oracle.pooled_key(cells, 8, THETA, 0.0).astype(np.float64)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-6
    # a partial block (m = 2) uses only its present cells
    y2 = oracle.pooled_key(cells[:2], 8, THETA, EPS)
    ref2 = _pooled_ref_fp64(cells[:2], 8, EPS)
    assert np.max(np.abs(y2 - ref2)) < 1e-5


def test_incremental_update_equals_full_repool():
    """Lever2's claim: recomputing only dirtied blocks leaves the cache equal,
    bit for bit, to re-pooling every block from scratch."""
    w = synth.Workload("t", 77, 2, 37, n_new=1, steps=30, H=4, Hk=1, top_k=16,
                       kv_type=synth.KV_F32)
    kidx = synth.make_kidx(w)
    pooled = np.zeros((w.n_seq, w.cap_blocks, w.d), dtype=np.float32)
    # prebuild the existing cells, then append one token per step per seq
    n0 = np.full(w.n_seq, w.n_cells0, dtype=np.int32)
    all_b = [(s, b) for s in range(w.n_seq) for b in range(-(-w.n_cells0 // w.r))]
    oracle.update_pooled(kidx, n0, np.array(all_b + [(-1, -1)] * 3), pooled,
                         w.r, THETA, EPS)
    for step in range(w.steps):
        n = synth.n_cells_at(w, step)
        oracle.update_pooled(kidx, n, synth.dirty_blocks(w, step), pooled, w.r,
                             THETA, EPS)
        for s in range(w.n_seq):
            full = oracle.build_pooled(kidx[s], int(n[s]), w.r, THETA, EPS)
            assert np.array_equal(pooled[s, :full.shape[0]], full), (step, s)


def test_update_skips_padding_and_absent_blocks():
    kidx = synth.normal((1, 64, 128), 9, 0, 0)
    pooled = np.full((1, 16, 128), 7.0, dtype=np.float32)
    n = np.array([10], dtype=np.int32)  # blocks 0..2 present, 3.. absent
    oracle.update_pooled(kidx, n, np.array([[-1, -1], [0, 5], [0, 2], [-1, 0]]),
                         pooled, 4, THETA, EPS)
    assert np.all(pooled[0, 5] == 7.0) and np.all(pooled[0, 0] == 7.0)
    assert not np.all(pooled[0, 2] == 7.0)


# --------------------------------------------------------------------------
# scores
# --------------------------------------------------------------------------

def _random_pooled(rng, nb, d=128):
    k = rng.standard_normal((nb, d)).astype(np.float32)
    return (k / np.sqrt(np.mean(k.astype(np.float64) ** 2, axis=1,
                                keepdims=True))).astype(np.float32)


def test_score_future_blocks_are_minus_inf():
    rng = np.random.default_rng(20)
    pooled = _random_pooled(rng, 40)
    q = rng.standard_normal(128).astype(np.float32)
    for pos in range(0, 150):
        s = oracle.score_query(q, pos, pooled, 40, 4, THETA)
        nc = (pos + 1) // 4
        assert np.all(np.isneginf(s[nc:])) and np.all(np.isfinite(s[:nc]))


def test_score_within_pairwise_bound_of_fp64():
    rng = np.random.default_rng(21)
    pooled = _random_pooled(rng, 64)
    q = rng.standard_normal(128).astype(np.float32)
    pos = 257
    s = oracle.score_query(q, pos, pooled, 64, 4, THETA)
    qr = oracle.rope(q, pos, THETA).astype(np.float64)
    for b in range(64):
        prod = qr * pooled[b].astype(np.float64)
        bound = 8 * U32 / (1 - 8 * U32) * np.abs(prod).sum()
        assert abs(float(s[b]) - prod.sum()) <= bound


def test_score_relative_position_invariance():
    """Shifting the query and all cells by a whole number of blocks leaves the
    scores unchanged up to fp32 rounding: q and k use one angle convention."""
    rng = np.random.default_rng(22)
    kidx = rng.standard_normal((64, 128)).astype(np.float32)
    q = rng.standard_normal(128).astype(np.float32)
    pos = 63
    base = oracle.build_pooled(kidx, 64, 4, THETA, EPS)
    s0 = oracle.score_query(q, pos, base, 16, 4, THETA)
    shift = 4 * 1000
    kidx2 = np.zeros((64 + shift, 128), dtype=np.float32)
    kidx2[shift:] = kidx
    sh = oracle.build_pooled(kidx2, 64 + shift, 4, THETA, EPS)
    s1 = oracle.score_query(q, pos + shift, sh, 16 + 1000, 4, THETA)[1000:]
    assert np.max(np.abs(s0 - s1)) < 2e-3


def test_score_bf16_products_are_exact():
    rng = np.random.default_rng(23)
    pooled = _random_pooled(rng, 32)
    q = rng.standard_normal(128).astype(np.float32)
    s = oracle.score_query(q, 127, pooled, 32, 4, THETA, bf16=True)
    qh = torch.from_numpy(oracle.rope(q, 127, THETA)).to(torch.bfloat16).double()
    kh = torch.from_numpy(pooled).to(torch.bfloat16).double()
    exact = (kh @ qh).numpy()
    for b in range(32):
        # only the 7 levels of additions round: products of bf16 are exact
        bound = 7 * U32 / (1 - 7 * U32) * float((kh[b] * qh).abs().sum())
        assert abs(float(s[b]) - exact[b]) <= bound


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def _brute_select(scores, pos, r, top_k):
    nc = (pos + 1) // r
    idx = np.arange(nc)
    s = scores[:nc].astype(np.float64)
    fin = np.isfinite(s)
    idx, s = idx[fin], s[fin]
    order = np.lexsort((idx, -s))  # score desc, then index asc
    keep = np.sort(idx[order[: top_k // r]])
    cells = (keep[:, None] * r + np.arange(r)[None]).ravel()
    return keep, np.concatenate([cells, np.arange(nc * r, pos + 1)])


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_lexsort_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(40):
        r = 4
        top_k = int(rng.choice([4, 8, 16, 64]))
        n = int(rng.integers(1, 90))
        pos = n - 1
        nb = -(-n // r)
        scores = rng.standard_normal(nb).astype(np.float32)
        if seed % 2:  # many exact ties
            scores = np.round(scores * 2).astype(np.float32) / 2
        scores[(pos + 1) // r:] = -np.inf
        b, c = oracle.select(scores, pos, r, top_k)
        rb, rc = _brute_select(scores, pos, r, top_k)
        assert np.array_equal(b, rb) and np.array_equal(c, rc)


def test_select_equals_dense_cell_sort():
    """Lever3's claim: selecting whole blocks first gives the same cells as
    expanding block scores to every cell and sorting all of them."""
    rng = np.random.default_rng(30)
    for _ in range(60):
        n = int(rng.integers(1, 3000))
        pos = n - 1
        top_k = int(rng.choice([8, 64, 256, 2048]))
        nb = -(-n // 4)
        scores = np.round(rng.standard_normal(nb) * 8).astype(np.float32)
        scores[(pos + 1) // 4:] = -np.inf
        _, c = oracle.select(scores, pos, 4, top_k)
        assert np.array_equal(c, oracle.select_dense_cells(scores, pos, 4, top_k))


def test_select_all_when_budget_covers_context():
    rng = np.random.default_rng(31)
    for n in (1, 2, 3, 4, 5, 63, 64, 65, 200):
        pos = n - 1
        scores = rng.standard_normal(-(-n // 4)).astype(np.float32)
        _, c = oracle.select(scores, pos, 4, 4 * (n + 4))
        assert np.array_equal(c, np.arange(n))


def test_select_counts_and_capacity_from_pages():
    g = _gold("page_counts.json")
    top_k, r = g["n_kv_max"]["top_k"], g["n_kv_max"]["r"]
    rng = np.random.default_rng(32)
    deep = g["deep_prompt"]
    n = deep["n_tokens"]
    assert -(-n // r) == deep["pooled_blocks"]
    assert n // r == deep["complete_blocks"] and n - r * (n // r) == deep["tail_cells"]
    scores = rng.standard_normal(deep["pooled_blocks"]).astype(np.float32)
    b, c = oracle.select(scores, n - 1, r, top_k)
    assert b.size == top_k // r and c.size == top_k + deep["tail_cells"]
    assert b.size + 1 == g["selected_blocks_approx"]["value"]  # + the tail block
    # capacity: the largest set over every tail length is top_k + r - 1
    worst = max(oracle.select(scores, n - 1 - k, r, top_k)[1].size for k in range(r))
    assert worst == g["n_kv_max"]["value"] == top_k + r - 1
    assert g["prefill_n_gather"]["value"] == g["prefill_n_gather"]["ubatch"] * worst
    assert g["union_threshold"]["value"] == 2 * g["union_threshold"]["ncols1"] * worst
    assert g["verify_threshold"]["n_gather"] == g["verify_threshold"]["batch"] * worst
    pd = g["prefill_dirty"]
    w = synth.WORKLOADS["prefill"]
    dl = synth.dirty_blocks(w, 0)
    blocks = dl[dl[:, 0] >= 0, 1]
    assert (blocks.min(), blocks.max(), blocks.size) == (
        pd["first_block"], pd["last_block"], pd["n_blocks"])


def test_select_causal_and_whole_blocks():
    rng = np.random.default_rng(33)
    for _ in range(50):
        n = int(rng.integers(1, 5000))
        pos = n - 1
        scores = rng.standard_normal(-(-n // 4)).astype(np.float32)
        b, c = oracle.select(scores, pos, 4, 256)
        nc = (pos + 1) // 4
        assert c.max() <= pos and np.all(np.diff(c) > 0)
        assert b.size <= 64 and np.all(b < nc)
        full = c[: 4 * b.size].reshape(-1, 4)
        assert np.array_equal(full, b[:, None] * 4 + np.arange(4))
        assert 4 * b.size <= 256 and c.size <= 256 + 3


def test_select_ties_signed_zero_and_nonfinite():
    scores = np.array([0.0, -0.0, 1.0, 1.0, np.nan, np.inf, -np.inf, 1.0],
                      dtype=np.float32)
    # budget of 3 blocks: the three 1.0s (blocks 2, 3, 7)
    b, _ = oracle.select(scores, 31, 4, 12)
    assert b.tolist() == [2, 3, 7]
    # budget of 4 blocks: then the zeros tie; -0 == +0 so block 0 wins
    b, _ = oracle.select(scores, 31, 4, 16)
    assert b.tolist() == [0, 2, 3, 7]
    # non-finite scores never compete
    b, _ = oracle.select(scores, 31, 4, 64)
    assert b.tolist() == [0, 1, 2, 3, 7]


def test_select_early_positions_tail_only():
    for pos in range(3):
        b, c = oracle.select(np.array([5.0], dtype=np.float32), pos, 4, 2048)
        assert b.size == 0 and c.tolist() == list(range(pos + 1))


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _deq(rows, kv_type, D):
    if kv_type in (synth.KV_F32, synth.KV_F16):
        return rows.astype(np.float64)
    blk = rows.reshape(*rows.shape[:-1], D // 32, 34)
    scale = blk[..., :2].copy().view(np.float16)[..., 0].astype(np.float64)
    q = blk[..., 2:].view(np.int8).astype(np.float64)
    return (scale[..., None] * q).reshape(*rows.shape[:-1], D)


def _sdpa_ref(q, k_rows, v_rows, kv_type, Hk, scale=None):
    H, D = q.shape
    K = _deq(k_rows, kv_type, D)  # [n][Hk][D]
    V = _deq(v_rows, kv_type, D)
    G = H // Hk
    Kt = torch.from_numpy(np.repeat(K.transpose(1, 0, 2), G, axis=0))
    Vt = torch.from_numpy(np.repeat(V.transpose(1, 0, 2), G, axis=0))
    Q = torch.from_numpy(q.astype(np.float64))[:, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, scale=scale)
    return o[:, 0, :].numpy()


def _store(x, kv_type):
    if kv_type == synth.KV_F32:
        return x
    if kv_type == synth.KV_F16:
        return x.astype(np.float16)
    return synth.quantize_q8_0(x)


@pytest.mark.parametrize("kv_type", [synth.KV_F32, synth.KV_Q8_0, synth.KV_F16])
def test_attend_vs_torch_sdpa(kv_type):
    rng = np.random.default_rng(40 + kv_type)
    H, Hk, D, n = 8, 2, 256, 300
    x_k = rng.standard_normal((n, Hk, D)).astype(np.float32)
    x_v = rng.standard_normal((n, Hk, D)).astype(np.float32)
    kc = _store(x_k, kv_type)
    vc = _store(x_v, kv_type)
    q = rng.standard_normal((H, D)).astype(np.float32)
    cells = np.sort(rng.choice(n, size=77, replace=False)).astype(np.int32)
    got = oracle.attend(q, kc, vc, kv_type, cells, Hk)
    ref = _sdpa_ref(q, kc[cells], vc[cells], kv_type, Hk)
    assert np.max(np.abs(got - ref)) < 1e-6


def test_attend_q8_dequant_exact_on_grid():
    """Values already on the q8_0 grid survive quantise -> dequantise."""
    rng = np.random.default_rng(41)
    D = 256
    scale = np.float32(np.float16(0.03125))
    q = rng.integers(-127, 128, size=(1, 1, D)).astype(np.float32)
    q[..., ::32] = 127  # make amax/127 land exactly on the scale
    x = (q * scale).astype(np.float32)
    rows = synth.quantize_q8_0(x)
    assert np.array_equal(_deq(rows, 1, D), x.astype(np.float64))
    # attention over one cell returns exactly that (dequantised) V row
    qv = rng.standard_normal((2, D)).astype(np.float32)
    out = oracle.attend(qv, rows, rows, 1, np.array([0], np.int32), 1)
    assert np.array_equal(out[0], x[0, 0]) and np.array_equal(out[1], x[0, 0])


def test_attend_f16_rows_equal_their_f32_widening():
    """binary16 -> binary32 is exact, so attention over an f16 cache equals,
    bit for bit, attention over the same values stored as f32 (the widening
    here is numpy's, not the oracle's)."""
    rng = np.random.default_rng(44)
    H, Hk, D, n = 8, 2, 256, 120
    kh = (rng.standard_normal((n, Hk, D)) * 3).astype(np.float16)
    vh = (rng.standard_normal((n, Hk, D)) * 3).astype(np.float16)
    q = rng.standard_normal((H, D)).astype(np.float32)
    cells = np.sort(rng.choice(n, size=41, replace=False)).astype(np.int32)
    got = oracle.attend(q, kh, vh, synth.KV_F16, cells, Hk)
    ref = oracle.attend(q, kh.astype(np.float32), vh.astype(np.float32), synth.KV_F32, cells, Hk)
    assert np.array_equal(got, ref)


def test_attend_f16_one_cell_returns_the_row_exactly():
    """Over a one-cell set the output is that V row; binary16 edge values
    (subnormals, -0, the largest finite 65504) come through unchanged."""
    D = 256
    v = np.zeros((1, 1, D), dtype=np.float16)
    specials = np.array([65504.0, -65504.0, 2.0 ** -24, -(2.0 ** -24), 2.0 ** -14, -0.0, 1.0,
                         -2.5, 0.1, 1000.0], dtype=np.float16)
    v[0, 0, :specials.size] = specials
    v[0, 0, specials.size:] = np.arange(D - specials.size, dtype=np.float16) / np.float16(7)
    k = np.ones((1, 1, D), dtype=np.float16)
    q = np.random.default_rng(45).standard_normal((2, D)).astype(np.float32)
    out = oracle.attend(q, k, v, synth.KV_F16, np.array([0], np.int32), 1)
    want = v[0, 0].astype(np.float32)
    assert np.array_equal(out[0], want) and np.array_equal(out[1], want)


def test_attend_identical_keys_gives_mean_of_values():
    rng = np.random.default_rng(42)
    n, D = 50, 256
    k = np.repeat(rng.standard_normal((1, 1, D)).astype(np.float32), n, axis=0)
    v = rng.standard_normal((n, 1, D)).astype(np.float32)
    q = rng.standard_normal((4, D)).astype(np.float32)
    cells = np.array([3, 9, 10, 11, 40], dtype=np.int32)
    out = oracle.attend(q, k, v, 0, cells, 1)
    ref = v[cells, 0].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(out - ref[None])) < 1e-6


def test_attend_equals_dense_masked_and_dense_when_budget_covers():
    """Lever1: attention over the selected set equals dense attention with the
    other cells masked to -inf; with top_k >= n_kv it is plain dense causal
    attention."""
    rng = np.random.default_rng(43)
    H, Hk, D, n = 4, 1, 256, 200
    kc = synth.quantize_q8_0(rng.standard_normal((n, Hk, D)).astype(np.float32))
    vc = synth.quantize_q8_0(rng.standard_normal((n, Hk, D)).astype(np.float32))
    q = rng.standard_normal((H, D)).astype(np.float32)
    pos = n - 1
    scores = rng.standard_normal(n // 4).astype(np.float32)
    _, cells = oracle.select(scores, pos, 4, 64)
    mask = np.zeros(n, dtype=np.uint8)
    mask[cells] = 1
    a = oracle.attend(q, kc, vc, 1, cells, Hk)
    b = oracle.attend_dense_masked(q, kc, vc, 1, mask, pos, Hk)
    assert np.max(np.abs(a - b)) < 1e-7
    _, allc = oracle.select(scores, pos, 4, 4 * n)
    dense = _sdpa_ref(q, kc[:n], vc[:n], 1, Hk)
    assert np.max(np.abs(oracle.attend(q, kc, vc, 1, allc, Hk) - dense)) < 1e-6


def test_step_on_tiny_workload_runs():
    w = synth.WORKLOADS["tiny"]
    kidx = synth.make_kidx(w)
    k = synth.make_kv(w, synth.T_K)
    v = synth.make_kv(w, synth.T_V)
    q_idx, q, q_seq, q_pos = synth.make_queries(w, 0)
    n = synth.n_cells_at(w, 0)
    pooled = np.zeros((w.n_seq, w.cap_blocks, w.d), dtype=np.float32)
    oracle.update_pooled(kidx, n, np.array([(0, b) for b in range(w.nb_max())]),
                         pooled, w.r, w.theta, w.eps)
    res = oracle.step(q_idx, q, q_seq, q_pos, pooled, k, v, kv_type=w.kv_type,
                      n_head_kv=w.Hk, r=w.r, top_k=w.top_k, theta=w.theta,
                      nb_out=w.nb_max())
    assert res["blocks"][0].size == 64 and res["cells"][0].size == 256
    assert np.all(np.isfinite(res["out"]))


# --------------------------------------------------------------------------
# structural dirty detection
# --------------------------------------------------------------------------

def _contig_rows(n_seq, cap):
    return np.arange(n_seq * cap, dtype=np.int64).reshape(n_seq, cap)


def test_dirty_blocks_first_call_lists_every_present_block():
    r, cap = 4, 64
    rows = _contig_rows(2, cap)
    snap = np.zeros((2, cap // r, r + 1), np.int64)
    d, snap = oracle.dirty_blocks(rows, [10, 17], snap, r)
    assert d == [(0, b) for b in range(3)] + [(1, b) for b in range(5)]
    assert oracle.dirty_blocks(rows, [10, 17], snap, r)[0] == []  # nothing changed


def test_dirty_blocks_append_and_rollback():
    r, cap = 4, 64
    rows = _contig_rows(1, cap)
    _, snap = oracle.dirty_blocks(rows, [10], np.zeros((1, cap // r, r + 1), np.int64), r)
    # one appended cell touches only the tail block (positions 8..10 -> 8..11)
    d, snap = oracle.dirty_blocks(rows, [11], snap, r)
    assert d == [(0, 2)]
    # positions 11 and 12: block 2 fills up, block 3 starts
    d, snap = oracle.dirty_blocks(rows, [13], snap, r)
    assert d == [(0, 2), (0, 3)]
    # rollback to 6 cells: block 1 loses members, blocks 2, 3 empty (recorded, not listed)
    d, snap = oracle.dirty_blocks(rows, [6], snap, r)
    assert d == [(0, 1)]
    assert snap[0][2][0] == 0 and snap[0][3][0] == 0
    # growing back over the emptied blocks lists them again
    d, snap = oracle.dirty_blocks(rows, [13], snap, r)
    assert d == [(0, 1), (0, 2), (0, 3)]


def test_dirty_blocks_moved_cell_marks_its_block_only():
    """Defrag: a cell moved to another row dirties the one block holding it."""
    r, cap = 4, 64
    rows = _contig_rows(2, cap).copy()
    _, snap = oracle.dirty_blocks(rows, [40, 40], np.zeros((2, cap // r, r + 1), np.int64), r)
    rows[1][21] = 1000  # position 21 of sequence 1 now lives in row 1000
    rows[0][3], rows[0][2] = rows[0][2], rows[0][3]  # two cells of block 0 swap rows
    d, _ = oracle.dirty_blocks(rows, [40, 40], snap, r)
    assert d == [(0, 0), (1, 5)]


# --------------------------------------------------------------------------
# threads
# --------------------------------------------------------------------------

def test_threaded_oracle_is_bit_identical_to_one_thread():
    """The parallel loops (update entries, score blocks, attention heads) give
    the single-threaded results bit for bit: each iteration keeps its order."""
    rng = np.random.default_rng(41)
    d, r, cap, H, Hk = 128, 4, 4096, 16, 2
    kidx = rng.standard_normal((2, cap, d)).astype(np.float32)
    n_cells = np.array([4000, 3001], np.int32)
    pairs = np.array([(s, b) for s in range(2) for b in range(-(-int(n_cells[s]) // r))],
                     np.int32)
    w = synth.Workload("thr", 41, 1, 3000, H=H, Hk=Hk)
    k = synth.make_kv(w, synth.T_K)[0]
    v = synth.make_kv(w, synth.T_V)[0]
    q = rng.standard_normal((H, 256)).astype(np.float32)
    q_idx = rng.standard_normal(d).astype(np.float32)
    cells = np.sort(rng.choice(3001, size=2051, replace=False)).astype(np.int32)
    outs = []
    for n_threads in (1, 8):
        got = oracle.set_threads(n_threads)
        assert got >= 1 and (n_threads == 1) == (got == 1) or os.cpu_count() == 1
        pooled = np.zeros((2, cap // r, d), np.float32)
        oracle.update_pooled(kidx, n_cells, pairs, pooled, r, THETA, EPS)
        sc = oracle.score_query(q_idx, 3999, pooled[0], 1000, r, THETA)
        sb = oracle.score_query(q_idx, 3999, pooled[0], 1000, r, THETA, bf16=True)
        at = oracle.attend(q, k, v, synth.KV_Q8_0, cells, Hk)
        outs.append((pooled, sc, sb, at))
    oracle.set_threads(1)
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
