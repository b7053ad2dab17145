"""Structured attention parity: inputs for which the exact output is known in
closed form and any lost or repeated cell moves it far beyond the tolerance.

Every K row is zero, so every logit is exactly 0 and the softmax weights are
all equal: the output of a head is the plain mean of the V rows of the listed
cells (issue #28734, fix summary, "lever1": attention visits exactly the
selected cells).  Each cell's V row holds integers in [-127, 127] (q8_0 scale 1),
exact in every cache type and in the fp16 operands the prefill path feeds the
matrix cores, and the sums stay below 2^24, so the
expected output is the fp64 mean rounded once.  The V patterns are chosen so
that dropping or repeating any one listed cell changes some output element by
more than ten times the attention bar, which the test asserts before it
compares.  Both attention entry points, list lengths across the 32-cell chunk
and 128-cell tile edges up to the 2051-cell capacity.
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
SIZES = [1, 31, 32, 33, 127, 128, 129, 2048, 2051]
Q8_SCALE = 1.0  # every V value is an integer: exact in binary16 and fp32


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def v_integers(n_cells, Hk, D):
    """Integer V pattern [cells][Hk][D] in [-127, 127]: an integer hash of
    (cell, head, dim), so every cell's row spreads over the whole range and
    differs from any mean in many dims."""
    m = np.uint64(0xFFFFFFFF)
    j = np.arange(n_cells, dtype=np.uint64)[:, None, None]
    g = np.arange(Hk, dtype=np.uint64)[None, :, None]
    t = np.arange(D, dtype=np.uint64)[None, None, :]
    h = (j * np.uint64(0x9E3779B1) + t * np.uint64(0x85EBCA77) + g * np.uint64(0xC2B2AE3D)) & m
    h ^= h >> np.uint64(15)
    h = (h * np.uint64(0x2C1B3C6D)) & m
    h ^= h >> np.uint64(12)
    h = (h * np.uint64(0x297A2D39)) & m
    h ^= h >> np.uint64(15)
    return (h % np.uint64(255)).astype(np.int64) - 127


def pack_kv(vals, kv_type):
    """Zero K and integer-valued V in the cache's storage type."""
    n_cells, Hk, D = vals.shape
    if kv_type == synth.KV_Q8_0:
        rb = synth.row_bytes(kv_type, D)
        k = np.zeros((n_cells, Hk, rb), np.uint8)
        v = np.zeros((n_cells, Hk, D // 32, 34), np.uint8)
        v[..., 0:2] = np.array([Q8_SCALE], np.float16).view(np.uint8)
        v[..., 2:] = vals.reshape(n_cells, Hk, D // 32, 32).astype(np.int8).view(np.uint8)
        return k, v.reshape(n_cells, Hk, rb), vals.astype(np.float64) * Q8_SCALE
    real = vals.astype(np.float64) * Q8_SCALE
    dt = np.float32 if kv_type == synth.KV_F32 else np.float16
    return np.zeros(vals.shape, dt), real.astype(dt), real


@pytest.mark.parametrize("kv_type,H,Hk", [(synth.KV_Q8_0, 16, 2), (synth.KV_F16, 16, 2),
                                          (synth.KV_F32, 4, 1)])
def test_attention_mean_of_listed_cells(kv_type, H, Hk):
    n_cap = 8192
    w = synth.Workload("struct", 77, 1, n_cap - 1, n_new=1, steps=1, H=H, Hk=Hk, top_k=2048,
                       kv_type=kv_type)
    assert w.ld_cells == 2051
    vals = v_integers(w.cap_cells, Hk, w.D)
    k_np, v_np, v_real = pack_kv(vals, kv_type)
    k_np, v_np = k_np[None], v_np[None]
    layer = runtime.Layer(w, DEV, kidx=np.zeros((1, w.cap_cells, w.d), np.float32),
                          k=k_np, v=v_np)
    layer.set_n_cells(np.array([n_cap], np.int32))
    rng = np.random.default_rng(77)
    n_q = len(SIZES) + 2
    ld = w.ld_cells
    cells = np.full((n_q, ld), -1, np.int32)
    sizes = list(SIZES) + [2051, 129]
    for i, n in enumerate(SIZES):
        cells[i, :n] = np.sort(rng.choice(n_cap, size=n, replace=False))
    cells[len(SIZES), :2051] = np.arange(n_cap - 2051, n_cap)  # contiguous, the last cells
    cells[len(SIZES) + 1, :129] = np.arange(129)               # the first cells
    q_seq = np.zeros(n_q, np.int32)
    q = synth.normal((n_q, H, w.D), 77, 0, synth.T_Q)
    G = H // Hk

    # the expected outputs in closed form, and the power of the check
    want = np.zeros((n_q, H, w.D), np.float64)
    for i, n in enumerate(sizes):
        c = cells[i, :n]
        mean = v_real[c].mean(axis=0)  # [Hk][D]
        want[i] = np.repeat(mean, G, axis=0)
        if n > 1:
            # dropping cell j moves the mean by (v_j - mean) / (n - 1); repeating
            # it by (v_j - mean) / (n + 1)
            dev = np.abs(v_real[c] - mean[None]).max(axis=(1, 2)) / (n + 1)
            assert dev.min() > 10 * ATTN_TOL, (n, float(dev.min()))
    for i, n in enumerate(sizes):  # the oracle agrees with the closed form
        r = oracle.attend(q[i], k_np[0], v_np[0], kv_type, cells[i, :n], Hk)
        assert float(np.abs(r - want[i]).max()) <= 1e-5 * max(1.0, float(np.abs(want[i]).max()))

    for entry in (qsa.sparse_attn_decode, qsa.sparse_attn_prefill):
        prefill = entry is qsa.sparse_attn_prefill
        bufs = runtime.StepBuffers(layer.dims, n_q, 64, DEV, prefill=prefill)
        bufs.out.fill_(123.0)
        entry(layer.dims, layer.seqs(), torch.from_numpy(q).to(DEV),
              torch.from_numpy(q_seq).to(DEV), n_q, layer.k, layer.v,
              torch.from_numpy(cells).to(DEV), torch.tensor(sizes, dtype=torch.int32, device=DEV),
              bufs.out, bufs.ws_attn, bufs.ws_attn_bytes)
        torch.cuda.synchronize()
        g = bufs.out.cpu().numpy().astype(np.float64)
        worst = 0.0
        for i, n in enumerate(sizes):
            err = float(np.abs(g[i] - want[i]).max())
            worst = max(worst, err)
            assert err <= ATTN_TOL, (entry.__name__, n, err)
        say(f"  {entry.__name__} kv_type={kv_type}: worst |out - mean| {worst:.2e}")
        # the inputs are exact in every operand type, so only the final
        # division rounds: far inside the bar
        assert worst <= 1e-4, (entry.__name__, worst)
