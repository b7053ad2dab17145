"""The allocation-free decode attention entry point (for callers that cannot
allocate: code under graph capture, tight serving loops) against the entry
point with a workspace: the same kernels, so the same outputs bit for bit, on
two calls in a row, the second with fewer queries and shorter lists; both
within the attention tolerance of the oracle."""
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


def _run(layer, w, sizes, seed):
    rng = np.random.default_rng(seed)
    n_q, ld = len(sizes), w.ld_cells
    n_cells = int(layer.n_cells.cpu()[0])
    cells = np.full((n_q, ld), -1, np.int32)
    for i, n in enumerate(sizes):
        cells[i, :n] = np.sort(rng.choice(n_cells, size=n, replace=False))
    q = synth.normal((n_q, w.H, w.D), seed, 0, synth.T_Q)
    q_seq = np.zeros(n_q, np.int32)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    args = (t(q), t(q_seq), n_q, layer.k, layer.v, t(cells),
            torch.tensor(sizes, dtype=torch.int32, device=DEV))
    bufs = runtime.StepBuffers(layer.dims, n_q, 64, DEV)
    qsa.sparse_attn_decode(layer.dims, layer.seqs(), *args, bufs.out, bufs.ws_attn,
                           bufs.ws_attn_bytes)
    out2 = torch.full_like(bufs.out, 7.0)
    qsa.sparse_attn_decode_noalloc(layer.dims, layer.seqs(), *args, out2)
    torch.cuda.synchronize()
    a, b = bufs.out.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    k_np, v_np = layer.k.cpu().numpy(), layer.v.cpu().numpy()
    worst = 0.0
    for i, n in enumerate(sizes):
        r = oracle.attend(q[i], k_np[0], v_np[0], w.kv_type, cells[i, :n], w.Hk)
        worst = max(worst, float(np.abs(b[i] - r).max()))
    assert worst <= 2e-3
    return worst


def test_noalloc_decode_attention_equals_workspace_call():
    w = synth.Workload("noalloc", 97, 1, 6000, n_new=1, steps=1, top_k=2048)
    layer = runtime.Layer(w, DEV, kidx=np.zeros((1, w.cap_cells, w.d), np.float32))
    layer.set_n_cells(np.array([6001], np.int32))
    say("noalloc: 5 queries up to 2051 cells, then 2 shorter ones")
    e1 = _run(layer, w, [2051, 2048, 700, 33, 1], 97)
    e2 = _run(layer, w, [129, 5], 98)
    say(f"  worst error vs oracle {max(e1, e2):.2e}; outputs equal the workspace call's")


def test_noalloc_rejects_more_than_its_scratch():
    w = synth.Workload("noalloc_big", 97, 1, 6000, n_new=1, steps=1, top_k=2048)
    layer = runtime.Layer(w, DEV, kidx=np.zeros((1, w.cap_cells, w.d), np.float32))
    n_q = 64  # 64 x 65 runs x 16 heads x 258 floats: more than the 8 MiB scratch
    z = torch.zeros(n_q, w.H, w.D, dtype=torch.float32, device=DEV)
    zi = torch.zeros(n_q, dtype=torch.int32, device=DEV)
    cells = torch.zeros(n_q, w.ld_cells, dtype=torch.int32, device=DEV)
    with pytest.raises(qsa.QsaError) as e:
        qsa.sparse_attn_decode_noalloc(layer.dims, layer.seqs(), z, zi, n_q, layer.k, layer.v,
                                       cells, zi, z)
    assert e.value.code == qsa.QSA_EWS
