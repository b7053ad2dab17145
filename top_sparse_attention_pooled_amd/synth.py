"""Seeded synthetic inputs for the QSA sparse-attention step.

This module draws the inputs that both the HIP path and the CPU oracle consume.
It holds none of the method's arithmetic: it only draws N(0, 1) values from
numpy generators seeded by (config, sequence, tensor, step) and packs them into
the storage formats the caches use.  Packing the KV cache into q8_0 (how the
model writes its cache, not part of the attention step) lives here; reading it
back (dequantisation) is done separately by each side.

The workloads mirror the pages' benchmark grid: synthetic word-list prompts of
4,992 / 49,678 / 148,978 / 198,628 / 248,278 tokens, 128 greedy decode tokens,
one or five sessions, q8_0 KV, 512-token prefill ubatches (the llama.cpp-multigpu
README, section 1 and section 8).  Real prompts, weights or KV states are not
used: every tensor is i.i.d. N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

T_KIDX, T_QIDX, T_Q, T_K, T_V = 0, 1, 2, 3, 4

KV_F32 = 0
KV_Q8_0 = 1
KV_F16 = 2
KIDX_F32 = 0
KIDX_BF16 = 1
Q8_BLOCK = 32
Q8_BYTES = 34  # binary16 scale + 32 int8
TILE = 64      # pooled-key tile width in blocks (capacity granularity)


def generator(cfg_id: int, seq_id: int, tensor_id: int, step: int = 0):
    return np.random.default_rng([cfg_id, seq_id, tensor_id, step])


def normal(shape, cfg_id: int, seq_id: int, tensor_id: int, step: int = 0):
    return generator(cfg_id, seq_id, tensor_id, step).standard_normal(
        size=shape, dtype=np.float32)


def quantize_q8_0(x: np.ndarray) -> np.ndarray:
    """Pack fp32 rows [..., D] into q8_0 bytes [..., D/32*34].

    Per block of 32: scale = binary16(amax/127); q = clamp(round half away
    from zero(x/scale), -127, 127); a zero block stores scale 0, q 0."""
    x = np.asarray(x, dtype=np.float32)
    *lead, D = x.shape
    assert D % Q8_BLOCK == 0
    xb = x.reshape(-1, D // Q8_BLOCK, Q8_BLOCK)
    amax = np.abs(xb).max(axis=-1)
    scale16 = (amax / np.float32(127.0)).astype(np.float16)
    scale32 = scale16.astype(np.float32)
    safe = np.where(scale32 > 0, scale32, np.float32(1.0))
    v = xb / safe[..., None]
    q = np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))
    q = np.clip(q, -127, 127).astype(np.int8)
    q[scale32 == 0] = 0
    out = np.empty(xb.shape[:-1] + (Q8_BYTES,), dtype=np.uint8)
    out[..., 0:2] = scale16.view(np.uint8).reshape(scale16.shape + (2,))
    out[..., 2:] = q.view(np.uint8)
    return out.reshape(*lead, D // Q8_BLOCK * Q8_BYTES)


def row_bytes(kv_type: int, D: int) -> int:
    if kv_type == KV_F32:
        return D * 4
    if kv_type == KV_F16:
        return D * 2
    return D // Q8_BLOCK * Q8_BYTES


def round_up(x: int, m: int) -> int:
    return -(-x // m) * m


@dataclass
class Workload:
    """One synthetic QSA workload (one layer's caches and one step's queries)."""
    name: str
    cfg_id: int
    n_seq: int
    n_cells0: int            # cells already present in each sequence
    n_new: int = 1           # query tokens per sequence per step (appended cells)
    steps: int = 1           # consecutive steps (each appends n_new cells)
    H: int = 16
    Hk: int = 2
    D: int = 256
    d: int = 128
    r: int = 4
    top_k: int = 2048
    kv_type: int = KV_Q8_0
    kidx_type: int = KIDX_F32
    theta: float = 1.0e4
    eps: float = 1.0e-6
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def cap_cells(self) -> int:
        return round_up(self.n_cells0 + self.n_new * self.steps, TILE * self.r)

    @property
    def cap_blocks(self) -> int:
        return self.cap_cells // self.r

    @property
    def ld_cells(self) -> int:
        return self.top_k + self.r - 1

    def nb_max(self, step: int = 0) -> int:
        """Score width covering every block any query of the step can see."""
        n = self.n_cells0 + self.n_new * (step + 1)
        return -(-n // self.r)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 4096 - 1, n_new=1, H=4, Hk=1, top_k=256,
                     kv_type=KV_F32,
                     note="1 seq, n_kv=4096 f32 cells, 1 query, 4 q heads / 1 KV head"),
    "decode50k": Workload("decode50k", 1, 1, 49678 - 1, n_new=1, steps=128,
                          note="1 seq, n_kv=49,678, q8_0 KV, 16/2 heads"),
    "decode250k": Workload("decode250k", 2, 1, 248278 - 1, n_new=1, steps=128,
                           note="1 seq, n_kv=248,278, q8_0 KV, 128 decode steps"),
    "decode5x250k": Workload("decode5x250k", 3, 5, 248278 - 1, n_new=1, steps=128,
                             note="5 independent seqs at n_kv=248,278, one token each"),
    "verify5x250k": Workload("verify5x250k", 5, 1, 248278 - 5, n_new=5, steps=64,
                             note="1 seq at n_kv=248,278, 5 query tokens per step (a "
                                  "speculative verify step), i.i.d. indexer queries"),
    "verify5x250k_ar1": Workload("verify5x250k_ar1", 5, 1, 248278 - 5, n_new=5, steps=64,
                                 note="the verify step with AR(1) indexer queries (rho 0.9) "
                                      "along its 5 tokens",
                                 extra={"qidx_ar1": 0.9}),
    "prefill": Workload("prefill", 4, 1, 198628, n_new=512, steps=1,
                        note="512-token ubatch appended at depth 198,628"),
    "prefill_ar1": Workload("prefill_ar1", 4, 1, 198628, n_new=512, steps=1,
                            note="the prefill ubatch with AR(1) indexer queries (rho 0.9) "
                                 "along the tokens",
                            extra={"qidx_ar1": 0.9}),
}


def ar1_rows(x: np.ndarray, rho: float) -> np.ndarray:
    """Rows of i.i.d. N(0,1) draws turned into an AR(1) series along axis 0
    with unit variance: y_0 = x_0, y_t = rho y_{t-1} + sqrt(1 - rho^2) x_t
    (float64 recursion, rounded to float32)."""
    y = np.empty(x.shape, np.float64)
    c = np.sqrt(1.0 - rho * rho)
    y[0] = x[0]
    for t in range(1, x.shape[0]):
        y[t] = rho * y[t - 1] + c * x[t]
    return y.astype(np.float32)


def make_kidx(w: Workload) -> np.ndarray:
    """Per-cell indexer keys [n_seq][cap_cells][d] (cells past the last step are
    zero): float32, or for kidx_type KIDX_BF16 their bfloat16 bits (uint16,
    rounded to nearest even)."""
    n_fill = w.n_cells0 + w.n_new * w.steps
    out = np.zeros((w.n_seq, w.cap_cells, w.d), dtype=np.float32)
    for s in range(w.n_seq):
        out[s, :n_fill] = normal((n_fill, w.d), w.cfg_id, s, T_KIDX)
    return to_bf16_bits(out) if w.kidx_type == KIDX_BF16 else out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def widen_kidx(kidx: np.ndarray) -> np.ndarray:
    """Per-cell keys as float32: bfloat16 bits widened exactly, float32 as is."""
    if kidx.dtype == np.uint16:
        return (kidx.astype(np.uint32) << 16).view(np.float32)
    return kidx


def make_kv(w: Workload, tensor_id: int) -> np.ndarray:
    """K (tensor_id T_K) or V (T_V) cache for every sequence: f32 [n_seq][cap]
    [Hk][D], f16 [n_seq][cap][Hk][D] (values rounded to nearest binary16) or
    q8_0 uint8 [n_seq][cap][Hk][D/32*34]."""
    n_fill = w.n_cells0 + w.n_new * w.steps
    rb = row_bytes(w.kv_type, w.D)
    if w.kv_type == KV_F32:
        out = np.zeros((w.n_seq, w.cap_cells, w.Hk, w.D), dtype=np.float32)
    elif w.kv_type == KV_F16:
        out = np.zeros((w.n_seq, w.cap_cells, w.Hk, w.D), dtype=np.float16)
    else:
        out = np.zeros((w.n_seq, w.cap_cells, w.Hk, rb), dtype=np.uint8)
    chunk = 1 << 16
    for s in range(w.n_seq):
        g = generator(w.cfg_id, s, tensor_id)
        for c0 in range(0, n_fill, chunk):
            c1 = min(n_fill, c0 + chunk)
            x = g.standard_normal(size=(c1 - c0, w.Hk, w.D), dtype=np.float32)
            if w.kv_type == KV_F32:
                out[s, c0:c1] = x
            elif w.kv_type == KV_F16:
                out[s, c0:c1] = x.astype(np.float16)
            else:
                out[s, c0:c1] = quantize_q8_0(x)
    return out


def make_queries(w: Workload, step: int):
    """Queries of one step: (q_idx [n_q][d], q [n_q][H][D], q_seq, q_pos).
    Step t appends cells n_cells0 + t*n_new ... + n_new - 1 of every sequence;
    each new cell is one query at its own position."""
    q_idx, q, seqs, pos = [], [], [], []
    for s in range(w.n_seq):
        qi = normal((w.n_new, w.d), w.cfg_id, s, T_QIDX, step)
        rho = w.extra.get("qidx_ar1")
        q_idx.append(ar1_rows(qi, rho) if rho else qi)
        q.append(normal((w.n_new, w.H, w.D), w.cfg_id, s, T_Q, step))
        base = w.n_cells0 + step * w.n_new
        seqs.append(np.full(w.n_new, s, dtype=np.int32))
        pos.append(np.arange(base, base + w.n_new, dtype=np.int32))
    return (np.concatenate(q_idx), np.concatenate(q), np.concatenate(seqs),
            np.concatenate(pos))


def n_cells_at(w: Workload, step: int) -> np.ndarray:
    """Cells present in each sequence once step ``step`` has appended."""
    return np.full(w.n_seq, w.n_cells0 + (step + 1) * w.n_new, dtype=np.int32)


def dirty_blocks(w: Workload, step: int, pad_pow2: bool = True) -> np.ndarray:
    """(seq, block) pairs touched by step ``step``'s appended cells, padded with
    (-1, -1) to a power of two of at least 4 entries."""
    pairs = []
    for s in range(w.n_seq):
        base = w.n_cells0 + step * w.n_new
        for b in range(base // w.r, (base + w.n_new - 1) // w.r + 1):
            pairs.append((s, b))
    n = len(pairs)
    if pad_pow2:
        m = 4
        while m < n:
            m *= 2
        pairs += [(-1, -1)] * (m - n)
    return np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
