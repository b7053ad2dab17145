"""ctypes binding of libqsa (include/qsa.h).

Argument marshalling only: every function passes device pointers of torch
tensors, sizes and the current HIP stream straight to the C ABI of the same
name and raises on a non-zero return code.  Nothing here computes any part of
the step, and there is no fallback: if libqsa.so is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqsa.so")

QSA_OK, QSA_EINVAL, QSA_ENOTSUP, QSA_EWS, QSA_EHIP = 0, -1, -2, -3, -4
KV_F32, KV_Q8_0, KV_F16 = 0, 1, 2
KIDX_F32, KIDX_BF16 = 0, 1
SCORE_F32, SCORE_BF16 = 0, 1
OP_SELECT, OP_ATTN_DECODE, OP_ATTN_PREFILL, OP_SCORE_BF16, OP_SCORE_SELECT = 0, 1, 2, 3, 4
OP_SCORE_SELECT_PREFILL = 5
OP_ATTN_DECODE_UNION = 6  # the nb_max argument of workspace_size carries t_group
TILE = 64

EXPORTS = ("qsa_version", "qsa_last_error", "qsa_workspace_size",
           "qsa_update_pooled_keys", "qsa_score_blocks", "qsa_select_topk_blocks",
           "qsa_score_select_decode", "qsa_decode_score_candidates",
           "qsa_decode_select_candidates", "qsa_sparse_attn_decode", "qsa_sparse_attn_prefill",
           "qsa_decode_select_attend", "qsa_score_select_prefill", "qsa_detect_dirty_blocks",
           "qsa_sparse_attn_decode_noalloc", "qsa_sparse_attn_decode_union",
           # memory-traffic probes (include/qsa_probe.h)
           "qsa_probe_stream_read", "qsa_probe_gather_prefill")


class QsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libqsa error {code}: {msg}")
        self.code = code


class _Dims(ctypes.Structure):
    _fields_ = [("n_head", ctypes.c_int32), ("n_head_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_idx", ctypes.c_int32),
                ("r", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("kv_type", ctypes.c_int32), ("kq_scale", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("idx_norm_w_dev", ctypes.c_void_p), ("kidx_type", ctypes.c_int32)]


class _Seqs(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("cap_cells", ctypes.c_int64),
                ("n_cells_dev", ctypes.c_void_p), ("cell_rows_dev", ctypes.c_void_p),
                ("n_rows", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqsa.so (built by top_sparse_attention_pooled_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime with the same soname as the system one;
    # loading torch first makes libqsa bind to that single runtime, so torch's
    # streams and allocations are valid handles for the library.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m top_sparse_attention_pooled_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D, S = ctypes.POINTER(_Dims), ctypes.POINTER(_Seqs)
    lib.qsa_version.restype = ctypes.c_int
    lib.qsa_version.argtypes = []
    lib.qsa_last_error.restype = ctypes.c_char_p
    lib.qsa_last_error.argtypes = []
    lib.qsa_workspace_size.restype = ctypes.c_int
    lib.qsa_workspace_size.argtypes = [D, i32, i32, i32, ctypes.POINTER(sz)]
    lib.qsa_update_pooled_keys.restype = ctypes.c_int
    lib.qsa_update_pooled_keys.argtypes = [D, S, vp, vp, i32, vp, vp, vp]
    lib.qsa_detect_dirty_blocks.restype = ctypes.c_int
    lib.qsa_detect_dirty_blocks.argtypes = [D, S, vp, vp, i32, vp, vp]
    lib.qsa_score_blocks.restype = ctypes.c_int
    lib.qsa_score_blocks.argtypes = [D, S, vp, vp, vp, i32, vp, vp, i32, vp, i64, i32, vp, sz, vp]
    lib.qsa_select_topk_blocks.restype = ctypes.c_int
    lib.qsa_select_topk_blocks.argtypes = [D, S, vp, i64, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.qsa_score_select_decode.restype = ctypes.c_int
    lib.qsa_score_select_decode.argtypes = [D, S, vp, vp, i32, vp, vp, vp, vp, vp, i32, i32,
                                            vp, i64, vp, vp, vp, vp, sz, vp]
    lib.qsa_decode_score_candidates.restype = ctypes.c_int
    lib.qsa_decode_score_candidates.argtypes = [D, S, vp, vp, i32, vp, vp, vp, vp, vp, i32, i32,
                                                vp, i64, vp, sz, vp]
    lib.qsa_decode_select_candidates.restype = ctypes.c_int
    lib.qsa_decode_select_candidates.argtypes = [D, S, vp, vp, i32, i32, vp, i64, vp, vp, vp, vp,
                                                 sz, vp]
    for name in ("qsa_sparse_attn_decode", "qsa_sparse_attn_prefill"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [D, S, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.qsa_sparse_attn_decode_union.restype = ctypes.c_int
    lib.qsa_sparse_attn_decode_union.argtypes = [D, S, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp,
                                                 sz, vp]
    lib.qsa_sparse_attn_decode_noalloc.restype = ctypes.c_int
    lib.qsa_sparse_attn_decode_noalloc.argtypes = [D, S, vp, vp, i32, vp, vp, vp, vp, vp, vp]
    lib.qsa_score_select_prefill.restype = ctypes.c_int
    lib.qsa_score_select_prefill.argtypes = [D, S, vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, vp,
                                             vp, vp, vp, sz, vp]
    lib.qsa_decode_select_attend.restype = ctypes.c_int
    lib.qsa_decode_select_attend.argtypes = [D, S, vp, vp, i32, i32, vp, i64, vp, vp, vp, vp, sz,
                                             vp, vp, vp, vp, vp, sz, vp]
    lib.qsa_probe_stream_read.restype = ctypes.c_int
    lib.qsa_probe_stream_read.argtypes = [vp, sz, i32, vp, i32, vp]
    lib.qsa_probe_gather_prefill.restype = ctypes.c_int
    lib.qsa_probe_gather_prefill.argtypes = [D, S, vp, i32, vp, vp, vp, vp, vp, i32, vp]
    _lib = lib
    return lib


@dataclass
class Dims:
    n_head: int = 16
    n_head_kv: int = 2
    head_dim: int = 256
    d_idx: int = 128
    r: int = 4
    top_k: int = 2048
    kv_type: int = KV_Q8_0
    kq_scale: float = 0.0
    rope_theta: float = 1.0e4
    rms_eps: float = 1.0e-6
    idx_norm_w: Optional[object] = None  # device float32 tensor [d_idx] or None
    kidx_type: int = KIDX_F32

    def c(self) -> _Dims:
        return _Dims(self.n_head, self.n_head_kv, self.head_dim, self.d_idx, self.r,
                     self.top_k, self.kv_type, self.kq_scale, self.rope_theta,
                     self.rms_eps, _ptr(self.idx_norm_w), self.kidx_type)

    @property
    def ld_cells(self) -> int:
        return self.top_k + self.r - 1

    @property
    def n_blocks_keep(self) -> int:
        return self.top_k // self.r


@dataclass
class Seqs:
    n_seq: int
    cap_cells: int
    n_cells: object  # device int32 tensor [n_seq]
    cell_rows: Optional[object] = None  # device int32 [n_seq][cap_cells] or None
    n_rows: int = 0

    def c(self) -> _Seqs:
        return _Seqs(self.n_seq, self.cap_cells, _ptr(self.n_cells), _ptr(self.cell_rows),
                     self.n_rows)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _rc(rc: int) -> None:
    if rc != QSA_OK:
        raise QsaError(rc, load().qsa_last_error().decode())


def version() -> int:
    return load().qsa_version()


def workspace_size(dims: Dims, op: int, n_q: int, nb_max: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _rc(load().qsa_workspace_size(ctypes.byref(dims.c()), op, n_q, nb_max, ctypes.byref(out)))
    return out.value


def detect_dirty_blocks(dims: Dims, seqs: Seqs, snapshot, dirty, max_dirty: int, n_found,
                        stream=None) -> None:
    _rc(load().qsa_detect_dirty_blocks(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                       _ptr(snapshot), _ptr(dirty), max_dirty, _ptr(n_found),
                                       _stream(stream)))


def update_pooled_keys(dims: Dims, seqs: Seqs, kidx, dirty, n_dirty: int, pooled,
                       pooled_bf16=None, stream=None) -> None:
    _rc(load().qsa_update_pooled_keys(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                      _ptr(kidx), _ptr(dirty), n_dirty, _ptr(pooled),
                                      _ptr(pooled_bf16), _stream(stream)))


def score_blocks(dims: Dims, seqs: Seqs, q_idx, q_seq, q_pos, n_q: int, pooled,
                 pooled_bf16, nb_max: int, scores, ld_scores: int, mode: int = SCORE_F32,
                 ws=None, ws_bytes: int = 0, stream=None) -> None:
    _rc(load().qsa_score_blocks(ctypes.byref(dims.c()), ctypes.byref(seqs.c()), _ptr(q_idx),
                                _ptr(q_seq), _ptr(q_pos), n_q, _ptr(pooled), _ptr(pooled_bf16),
                                nb_max, _ptr(scores), ld_scores, mode, _ptr(ws), ws_bytes,
                                _stream(stream)))


def select_topk_blocks(dims: Dims, seqs: Seqs, scores, ld_scores: int, q_seq, q_pos, n_q: int,
                       nb_max: int, sel_blocks, sel_cells, n_sel, ws=None, ws_bytes: int = 0,
                       stream=None) -> None:
    _rc(load().qsa_select_topk_blocks(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                      _ptr(scores), ld_scores, _ptr(q_seq), _ptr(q_pos), n_q,
                                      nb_max, _ptr(sel_blocks), _ptr(sel_cells), _ptr(n_sel),
                                      _ptr(ws), ws_bytes, _stream(stream)))


def score_select_decode(dims: Dims, seqs: Seqs, kidx, dirty, n_dirty: int, pooled, pooled_bf16,
                        q_idx, q_seq, q_pos, n_q: int, nb_max: int, scores, ld_scores: int,
                        sel_blocks, sel_cells, n_sel, ws, ws_bytes: int, stream=None) -> None:
    _rc(load().qsa_score_select_decode(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                       _ptr(kidx), _ptr(dirty), n_dirty, _ptr(pooled),
                                       _ptr(pooled_bf16), _ptr(q_idx), _ptr(q_seq), _ptr(q_pos),
                                       n_q, nb_max, _ptr(scores), ld_scores, _ptr(sel_blocks),
                                       _ptr(sel_cells), _ptr(n_sel), _ptr(ws), ws_bytes,
                                       _stream(stream)))


def decode_score_candidates(dims: Dims, seqs: Seqs, kidx, dirty, n_dirty: int, pooled,
                            pooled_bf16, q_idx, q_seq, q_pos, n_q: int, nb_max: int, scores,
                            ld_scores: int, ws, ws_bytes: int, stream=None) -> None:
    _rc(load().qsa_decode_score_candidates(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                           _ptr(kidx), _ptr(dirty), n_dirty, _ptr(pooled),
                                           _ptr(pooled_bf16), _ptr(q_idx), _ptr(q_seq),
                                           _ptr(q_pos), n_q, nb_max, _ptr(scores), ld_scores,
                                           _ptr(ws), ws_bytes, _stream(stream)))


def decode_select_candidates(dims: Dims, seqs: Seqs, q_seq, q_pos, n_q: int, nb_max: int,
                             scores, ld_scores: int, sel_blocks, sel_cells, n_sel, ws,
                             ws_bytes: int, stream=None) -> None:
    _rc(load().qsa_decode_select_candidates(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                            _ptr(q_seq), _ptr(q_pos), n_q, nb_max, _ptr(scores),
                                            ld_scores, _ptr(sel_blocks), _ptr(sel_cells),
                                            _ptr(n_sel), _ptr(ws), ws_bytes, _stream(stream)))


def score_select_prefill(dims: Dims, seqs: Seqs, kidx, dirty, n_dirty: int, pooled, pooled_bf16,
                         q_idx, q_seq, q_pos, n_q: int, nb_max: int, sel_blocks, sel_cells,
                         n_sel, ws, ws_bytes: int, stream=None) -> None:
    _rc(load().qsa_score_select_prefill(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                        _ptr(kidx), _ptr(dirty), n_dirty, _ptr(pooled),
                                        _ptr(pooled_bf16), _ptr(q_idx), _ptr(q_seq), _ptr(q_pos),
                                        n_q, nb_max, _ptr(sel_blocks), _ptr(sel_cells),
                                        _ptr(n_sel), _ptr(ws), ws_bytes, _stream(stream)))


def decode_select_attend(dims: Dims, seqs: Seqs, q_seq, q_pos, n_q: int, nb_max: int, scores,
                         ld_scores: int, sel_blocks, sel_cells, n_sel, ws_idx, ws_idx_bytes: int,
                         q, k_cache, v_cache, out, ws_attn, ws_attn_bytes: int,
                         stream=None) -> None:
    _rc(load().qsa_decode_select_attend(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                        _ptr(q_seq), _ptr(q_pos), n_q, nb_max, _ptr(scores),
                                        ld_scores, _ptr(sel_blocks), _ptr(sel_cells), _ptr(n_sel),
                                        _ptr(ws_idx), ws_idx_bytes, _ptr(q), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(out), _ptr(ws_attn), ws_attn_bytes,
                                        _stream(stream)))


def sparse_attn_decode(dims: Dims, seqs: Seqs, q, q_seq, n_q: int, k_cache, v_cache, sel_cells,
                       n_sel, out, ws, ws_bytes: int, stream=None) -> None:
    _rc(load().qsa_sparse_attn_decode(ctypes.byref(dims.c()), ctypes.byref(seqs.c()), _ptr(q),
                                      _ptr(q_seq), n_q, _ptr(k_cache), _ptr(v_cache),
                                      _ptr(sel_cells), _ptr(n_sel), _ptr(out), _ptr(ws),
                                      ws_bytes, _stream(stream)))


def sparse_attn_decode_noalloc(dims: Dims, seqs: Seqs, q, q_seq, n_q: int, k_cache, v_cache,
                               sel_cells, n_sel, out, stream=None) -> None:
    _rc(load().qsa_sparse_attn_decode_noalloc(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                              _ptr(q), _ptr(q_seq), n_q, _ptr(k_cache),
                                              _ptr(v_cache), _ptr(sel_cells), _ptr(n_sel),
                                              _ptr(out), _stream(stream)))


def sparse_attn_prefill(dims: Dims, seqs: Seqs, q, q_seq, n_q: int, k_cache, v_cache, sel_cells,
                        n_sel, out, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _rc(load().qsa_sparse_attn_prefill(ctypes.byref(dims.c()), ctypes.byref(seqs.c()), _ptr(q),
                                       _ptr(q_seq), n_q, _ptr(k_cache), _ptr(v_cache),
                                       _ptr(sel_cells), _ptr(n_sel), _ptr(out), _ptr(ws),
                                       ws_bytes, _stream(stream)))


def sparse_attn_decode_union(dims: Dims, seqs: Seqs, q, q_seq, n_q: int, t_group: int,
                             k_cache, v_cache, sel_cells, n_sel, out, ws=None, ws_bytes: int = 0,
                             stream=None) -> None:
    """Decode attention of queries in groups of t_group over the union of
    each group's cell lists (include/qsa.h)."""
    _rc(load().qsa_sparse_attn_decode_union(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                            _ptr(q), _ptr(q_seq), n_q, t_group, _ptr(k_cache),
                                            _ptr(v_cache), _ptr(sel_cells), _ptr(n_sel),
                                            _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def probe_stream_read(src, n_bytes: int, sink, n_sink: int, nontemporal: bool = True,
                      stream=None) -> None:
    """Memory-traffic probe: read n_bytes of src once (include/qsa_probe.h)."""
    _rc(load().qsa_probe_stream_read(_ptr(src), n_bytes, int(nontemporal), _ptr(sink), n_sink,
                                     _stream(stream)))


def probe_gather_prefill(dims: Dims, seqs: Seqs, q_seq, n_q: int, k_cache, v_cache, sel_cells,
                         n_sel, sink, n_sink: int, stream=None) -> None:
    """Memory-traffic probe: the K/V row gather of sparse_attn_prefill alone."""
    _rc(load().qsa_probe_gather_prefill(ctypes.byref(dims.c()), ctypes.byref(seqs.c()),
                                        _ptr(q_seq), n_q, _ptr(k_cache), _ptr(v_cache),
                                        _ptr(sel_cells), _ptr(n_sel), _ptr(sink), n_sink,
                                        _stream(stream)))


def pooled_numel(n_seq: int, cap_cells: int, r: int, d_idx: int = 128) -> int:
    """Float count of the tiled pooled-key buffer."""
    return n_seq * (cap_cells // r) * d_idx
