"""Device buffers of one QSA layer and the call sequence of one step.

Plumbing only: torch allocates and holds device memory; every part of the
step runs in libqsa's kernels through the binding in ``qsa.py``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import qsa
from . import synth


def dims_of(w: synth.Workload) -> qsa.Dims:
    return qsa.Dims(n_head=w.H, n_head_kv=w.Hk, head_dim=w.D, d_idx=w.d, r=w.r,
                    top_k=w.top_k, kv_type=w.kv_type, kq_scale=0.0,
                    rope_theta=w.theta, rms_eps=w.eps, kidx_type=w.kidx_type)


def untile_pooled(flat: torch.Tensor, n_seq: int, cap_blocks: int, d: int = 128) -> torch.Tensor:
    """Tiled pooled-key buffer -> [n_seq][cap_blocks][d] (a layout view for
    inspection; the kernels read the tiled form)."""
    t = flat.view(n_seq, cap_blocks // qsa.TILE, d // 4, qsa.TILE, 4)
    return t.permute(0, 1, 3, 2, 4).reshape(n_seq, cap_blocks, d)


@dataclass
class StepOut:
    scores: torch.Tensor
    sel_blocks: torch.Tensor
    sel_cells: torch.Tensor
    n_sel: torch.Tensor
    out: torch.Tensor


class Layer:
    """One QSA layer's caches on the GPU: per-cell indexer keys, K and V, the
    tiled fp32 pooled-key cache and its bf16 copy."""

    def __init__(self, w: synth.Workload, device="cuda", kidx: Optional[np.ndarray] = None,
                 k: Optional[np.ndarray] = None, v: Optional[np.ndarray] = None,
                 bf16: bool = True):
        self.w = w
        self.dims = dims_of(w)
        self.device = torch.device(device)
        kidx = synth.make_kidx(w) if kidx is None else kidx
        k = synth.make_kv(w, synth.T_K) if k is None else k
        v = synth.make_kv(w, synth.T_V) if v is None else v
        # bf16 keys travel as int16 (torch's uint16 lacks device copies here)
        kidx = kidx.view(np.int16) if kidx.dtype == np.uint16 else kidx
        self.kidx = torch.from_numpy(kidx).to(self.device)
        self.k = torch.from_numpy(k).to(self.device)
        self.v = torch.from_numpy(v).to(self.device)
        self.cap_blocks = w.cap_blocks
        self.pooled = torch.zeros(qsa.pooled_numel(w.n_seq, w.cap_cells, w.r, w.d),
                                  dtype=torch.float32, device=self.device)
        self.pooled_bf16 = (torch.zeros(w.n_seq * self.cap_blocks * w.d, dtype=torch.int16,
                                        device=self.device) if bf16 else None)
        self.n_cells = torch.zeros(w.n_seq, dtype=torch.int32, device=self.device)

    @classmethod
    def clone_of(cls, other: "Layer") -> "Layer":
        """A second copy of the same caches at new addresses (a replica)."""
        obj = cls.__new__(cls)
        obj.w, obj.dims, obj.device = other.w, other.dims, other.device
        obj.cap_blocks = other.cap_blocks
        for name in ("kidx", "k", "v", "pooled", "pooled_bf16", "n_cells"):
            t = getattr(other, name)
            setattr(obj, name, None if t is None else t.clone())
        return obj

    def seqs(self, n_cells: Optional[torch.Tensor] = None) -> qsa.Seqs:
        return qsa.Seqs(self.w.n_seq, self.w.cap_cells,
                        self.n_cells if n_cells is None else n_cells)

    def set_n_cells(self, n: np.ndarray) -> None:
        self.n_cells.copy_(torch.from_numpy(np.asarray(n, dtype=np.int32)))

    def rebuild(self, n_cells: np.ndarray) -> None:
        """Recompute every present block (the resume path)."""
        self.set_n_cells(n_cells)
        pairs = [(s, b) for s in range(self.w.n_seq)
                 for b in range(-(-int(n_cells[s]) // self.w.r))]
        dl = torch.tensor(pairs, dtype=torch.int32, device=self.device).reshape(-1)
        qsa.update_pooled_keys(self.dims, self.seqs(), self.kidx, dl, len(pairs), self.pooled,
                               self.pooled_bf16)

    def pooled_rows(self) -> torch.Tensor:
        return untile_pooled(self.pooled, self.w.n_seq, self.cap_blocks, self.w.d)


class StepBuffers:
    """Outputs and workspaces of one step for n_q queries."""

    def __init__(self, dims: qsa.Dims, n_q: int, nb_max: int, device, prefill: bool = False):
        dev = torch.device(device)
        self.n_q, self.nb_max = n_q, nb_max
        self.ld = (nb_max + 63) // 64 * 64
        self.scores = torch.empty(n_q, self.ld, dtype=torch.float32, device=dev)
        self.sel_blocks = torch.empty(n_q, dims.n_blocks_keep, dtype=torch.int32, device=dev)
        self.sel_cells = torch.empty(n_q, dims.ld_cells, dtype=torch.int32, device=dev)
        self.n_sel = torch.empty(n_q, dtype=torch.int32, device=dev)
        self.out = torch.empty(n_q, dims.n_head, dims.head_dim, dtype=torch.float32, device=dev)
        op = qsa.OP_ATTN_PREFILL if prefill else qsa.OP_ATTN_DECODE
        self.ws_attn_bytes = qsa.workspace_size(dims, op, n_q)
        self.ws_attn = torch.empty(max(self.ws_attn_bytes, 16), dtype=torch.uint8, device=dev)
        self.ws_score_bytes = qsa.workspace_size(dims, qsa.OP_SCORE_BF16, n_q)
        self.ws_score = torch.empty(max(self.ws_score_bytes, 16), dtype=torch.uint8, device=dev)
        self.ws_fused_bytes = qsa.workspace_size(dims, qsa.OP_SCORE_SELECT, n_q, nb_max)
        self.ws_fused = torch.empty(max(self.ws_fused_bytes, 16), dtype=torch.uint8, device=dev)
        self.ws_pf_bytes = (qsa.workspace_size(dims, qsa.OP_SCORE_SELECT_PREFILL, n_q, nb_max)
                            if prefill else 0)
        self.ws_pf = torch.empty(max(self.ws_pf_bytes, 16), dtype=torch.uint8, device=dev)


PATHS = ("attend", "indexer", "general")
SEL_ATTN_MAX_BLOCKS = 1 << 16  # nb_max limit of qsa_decode_select_attend


def run_step(layer: Layer, bufs: StepBuffers, q_idx, q, q_seq, q_pos, dirty, n_dirty: int,
             mode: int = qsa.SCORE_F32, prefill: bool = False, path: str = "attend",
             stream=None) -> StepOut:
    """update -> score -> select -> attend, all enqueued on one stream, by one
    of three call sequences with the same results:
      attend:  qsa_decode_score_candidates, then qsa_decode_select_attend
               (decode, fp32 scores, contexts up to 65536 blocks);
      indexer: qsa_score_select_decode (fp32 scores) or, for bf16 scores,
               qsa_score_select_prefill (exact in order T; bufs built with
               prefill=True), then the attention call;
      general: update, score, select and attention as four calls (with bf16
               scores the selection follows the matrix-core sums, which match
               T's to within a bound, not bit for bit)."""
    assert path in PATHS, path
    d, sq = layer.dims, layer.seqs()
    n_q = bufs.n_q
    if path == "attend" and (prefill or mode != qsa.SCORE_F32 or bufs.nb_max > SEL_ATTN_MAX_BLOCKS):
        path = "indexer"
    if path == "indexer" and mode == qsa.SCORE_BF16:
        qsa.score_select_prefill(d, sq, layer.kidx, dirty, n_dirty, layer.pooled,
                                 layer.pooled_bf16, q_idx, q_seq, q_pos, n_q, bufs.nb_max,
                                 bufs.sel_blocks, bufs.sel_cells, bufs.n_sel, bufs.ws_pf,
                                 bufs.ws_pf_bytes, stream=stream)
        attn = qsa.sparse_attn_prefill if prefill else qsa.sparse_attn_decode
        attn(d, sq, q, q_seq, n_q, layer.k, layer.v, bufs.sel_cells, bufs.n_sel, bufs.out,
             bufs.ws_attn, bufs.ws_attn_bytes, stream=stream)
        return StepOut(None, bufs.sel_blocks, bufs.sel_cells, bufs.n_sel, bufs.out)
    if path == "attend":
        qsa.decode_score_candidates(d, sq, layer.kidx, dirty, n_dirty, layer.pooled,
                                    layer.pooled_bf16, q_idx, q_seq, q_pos, n_q, bufs.nb_max,
                                    bufs.scores, bufs.ld, bufs.ws_fused, bufs.ws_fused_bytes,
                                    stream=stream)
        qsa.decode_select_attend(d, sq, q_seq, q_pos, n_q, bufs.nb_max, bufs.scores, bufs.ld,
                                 bufs.sel_blocks, bufs.sel_cells, bufs.n_sel, bufs.ws_fused,
                                 bufs.ws_fused_bytes, q, layer.k, layer.v, bufs.out,
                                 bufs.ws_attn, bufs.ws_attn_bytes, stream=stream)
        return StepOut(bufs.scores, bufs.sel_blocks, bufs.sel_cells, bufs.n_sel, bufs.out)
    if path == "indexer":
        qsa.score_select_decode(d, sq, layer.kidx, dirty, n_dirty, layer.pooled,
                                layer.pooled_bf16, q_idx, q_seq, q_pos, n_q, bufs.nb_max,
                                bufs.scores, bufs.ld, bufs.sel_blocks, bufs.sel_cells,
                                bufs.n_sel, bufs.ws_fused, bufs.ws_fused_bytes, stream=stream)
    else:
        if n_dirty:
            qsa.update_pooled_keys(d, sq, layer.kidx, dirty, n_dirty, layer.pooled,
                                   layer.pooled_bf16, stream=stream)
        qsa.score_blocks(d, sq, q_idx, q_seq, q_pos, n_q, layer.pooled, layer.pooled_bf16,
                         bufs.nb_max, bufs.scores, bufs.ld, mode, bufs.ws_score,
                         bufs.ws_score_bytes, stream=stream)
        qsa.select_topk_blocks(d, sq, bufs.scores, bufs.ld, q_seq, q_pos, n_q, bufs.nb_max,
                               bufs.sel_blocks, bufs.sel_cells, bufs.n_sel, stream=stream)
    attn = qsa.sparse_attn_prefill if prefill else qsa.sparse_attn_decode
    attn(d, sq, q, q_seq, n_q, layer.k, layer.v, bufs.sel_cells, bufs.n_sel, bufs.out,
         bufs.ws_attn, bufs.ws_attn_bytes, stream=stream)
    return StepOut(bufs.scores, bufs.sel_blocks, bufs.sel_cells, bufs.n_sel, bufs.out)
