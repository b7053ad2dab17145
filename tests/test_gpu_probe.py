"""GPU checks of the memory-traffic probes (include/qsa_probe.h): the XOR of
the sink after a call equals the XOR of exactly the 32-bit words the probe
is defined to load, computed on the host -- every word of a streamed buffer
once, and for the gather every K and V row of every slot of every 32-cell
chunk of each query's list (padding slots and cells not present read the
sequence's cell 0), per KV head.  A probe that skipped or repeated loads
would be timed on the wrong traffic."""
import sys

import numpy as np
import pytest
import torch

from top_sparse_attention_pooled_amd import qsa

pytestmark = pytest.mark.gpu
DEV = "cuda"
Q8_ROW = 272


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel(),
                                     initial=np.uint32(0)))


@pytest.mark.parametrize("n_sink", [7, 8192])  # shared words (atomic) / a word per wavefront
@pytest.mark.parametrize("n_bytes,nontemporal", [(16, True), (4096 + 48, False),
                                                 (64 * 2**20 + 16 * 7, True)])
def test_stream_read_loads_every_word_once(n_bytes, nontemporal, n_sink):
    say(f"probe stream read: {n_bytes} bytes, nontemporal {nontemporal}, {n_sink} sink words")
    rng = np.random.default_rng(n_bytes)
    host = rng.integers(0, 2**32, n_bytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.uint8)).to(DEV)
    sink = torch.zeros(n_sink, dtype=torch.int32, device=DEV)
    qsa.probe_stream_read(src, n_bytes, sink, n_sink, nontemporal=nontemporal)
    torch.cuda.synchronize()
    got = xor_words(sink.cpu().numpy())
    assert got == xor_words(host)


@pytest.mark.parametrize("n_sink", [3, 8192])
def test_gather_prefill_loads_the_attention_rows(n_sink):
    say("probe gather: 2 sequences, 9 queries, ragged lists")
    d = qsa.Dims()  # 2 KV heads, q8_0, lists of top_k + r - 1 = 2051 cells
    n_seq, cap = 2, 4096
    n_present = np.array([3000, 4096], np.int32)
    rng = np.random.default_rng(5)
    kv_bytes = n_seq * cap * d.n_head_kv * Q8_ROW
    k_host = rng.integers(0, 256, kv_bytes, dtype=np.uint8)
    v_host = rng.integers(0, 256, kv_bytes, dtype=np.uint8)
    ld = d.ld_cells
    n_sel = np.array([0, 1, 31, 32, 33, 2051, 700, 129, 2051], np.int32)
    q_seq = np.array([0, 1, 0, 1, 0, 1, 0, -1, 1], np.int32)
    cells = np.full((n_sel.size, ld), -1, np.int32)
    for i, n in enumerate(n_sel):
        cells[i, :n] = np.sort(rng.choice(cap, size=n, replace=False))  # some past n_present
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    seqs = qsa.Seqs(n_seq, cap, t(n_present))
    sink = torch.zeros(n_sink, dtype=torch.int32, device=DEV)
    qsa.probe_gather_prefill(d, seqs, t(q_seq), q_seq.size, t(k_host), t(v_host), t(cells),
                             t(n_sel), sink, n_sink)
    torch.cuda.synchronize()
    k_rows = k_host.reshape(-1, Q8_ROW)
    v_rows = v_host.reshape(-1, Q8_ROW)
    want = 0
    for i in range(q_seq.size):
        s = int(q_seq[i])
        if s < 0 or s >= n_seq:
            continue
        n = min(max(int(n_sel[i]), 0), ld)
        for c0 in range(0, n, 32):
            for slot in range(32):
                cc = c0 + slot
                cell = int(cells[i, min(cc, ld - 1)]) if cc < n else -1
                ok = 0 <= cell < n_present[s]
                for g in range(d.n_head_kv):
                    row = (s * cap + (cell if ok else 0)) * d.n_head_kv + g
                    want ^= xor_words(k_rows[row]) ^ xor_words(v_rows[row])
    assert xor_words(sink.cpu().numpy()) == want
