"""Host-side checks of the C ABI: the library loads, exports every entry point
include/qsa.h declares, sizes workspaces, and rejects bad arguments before any
device work (so these run without a GPU: every call below fails validation).
"""
import ctypes
import os
import re

import pytest

from top_sparse_attention_pooled_amd import qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 64 KiB-aligned non-null address; never dereferenced here


def _declared():
    """Every qsa_* function the headers under include/ declare."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            with open(os.path.join(inc, h)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            names |= set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = qsa.load()
    names = _declared()
    assert set(names) == set(qsa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_error_string():
    assert qsa.version() == 3
    assert isinstance(qsa.load().qsa_last_error(), bytes)


def test_workspace_sizes():
    d = qsa.Dims()
    assert qsa.workspace_size(d, qsa.OP_SELECT, 5) == 0
    assert qsa.workspace_size(d, qsa.OP_SCORE_BF16, 512) == 512 * 128 * 2
    runs = -(-d.ld_cells // 32)  # 32-cell runs
    assert qsa.workspace_size(d, qsa.OP_ATTN_DECODE, 5) == 5 * runs * 16 * 258 * 4
    # decode score+select, sized for the calls whose queries overflow the fused
    # grid: per 64-block group 6 kept + 1 dropped
    n_grp = -(-62070 // 256) * 4
    assert qsa.workspace_size(d, qsa.OP_SCORE_SELECT, 5, 62070) == 5 * n_grp * 7 * 8
    # shorter contexts keep more keys per group: 16 for 196 groups (12,420 blocks)
    n_grp = -(-12420 // 256) * 4
    assert qsa.workspace_size(d, qsa.OP_SCORE_SELECT, 1, 12420) == n_grp * 17 * 8
    n_grp = -(-30000 // 256) * 4  # 472 groups: 8 kept
    assert qsa.workspace_size(d, qsa.OP_SCORE_SELECT, 1, 30000) == n_grp * 9 * 8
    with pytest.raises(qsa.QsaError) as e:
        qsa.workspace_size(d, 99, 1)
    assert e.value.code == qsa.QSA_EINVAL


def _seqs(cap=4096 * 4, n_cells=FAKE):
    return qsa.Seqs(1, cap, n_cells)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 128, qsa.QSA_ENOTSUP),
    ("d_idx", 64, qsa.QSA_ENOTSUP),
    ("n_head", 12, qsa.QSA_ENOTSUP),     # 12/2 = 6 heads per KV head
    ("n_head", 3, qsa.QSA_EINVAL),       # not a multiple of 2
    ("top_k", 2050, qsa.QSA_EINVAL),     # not a multiple of r
    ("top_k", 4 * 4097, qsa.QSA_ENOTSUP),
    ("r", 0, qsa.QSA_ENOTSUP),
    ("kv_type", 7, qsa.QSA_EINVAL),
    ("kidx_type", 2, qsa.QSA_EINVAL),
    ("rope_theta", 0.5, qsa.QSA_EINVAL),
])
def test_bad_dims_rejected(field, value, code):
    d = qsa.Dims()
    setattr(d, field, value)
    with pytest.raises(qsa.QsaError) as e:
        qsa.update_pooled_keys(d, _seqs(), FAKE, FAKE, 4, FAKE, None, stream=0)
    assert e.value.code == code


def test_kidx_alignment_follows_its_type():
    """f32 keys need 4-byte alignment, bf16 keys 2 (a 2-byte offset is
    rejected for f32 only)."""
    d = qsa.Dims()
    with pytest.raises(qsa.QsaError) as e:
        qsa.update_pooled_keys(d, _seqs(), FAKE + 2, FAKE, 4, FAKE, None, stream=0)
    assert e.value.code == qsa.QSA_EINVAL
    assert "kidx" in str(e.value)
    d.kidx_type = qsa.KIDX_BF16
    with pytest.raises(qsa.QsaError) as e:
        qsa.update_pooled_keys(d, _seqs(), FAKE + 1, FAKE, 4, FAKE, None, stream=0)
    assert "kidx" in str(e.value)


def test_bad_geometry_and_pointers_rejected():
    d = qsa.Dims()
    cases = [
        # cap_cells not a multiple of 64*r
        lambda: qsa.update_pooled_keys(d, _seqs(cap=1000), FAKE, FAKE, 4, FAKE, None, stream=0),
        # pooled not 16-byte aligned
        lambda: qsa.update_pooled_keys(d, _seqs(), FAKE, FAKE, 4, FAKE + 8, None, stream=0),
        # null n_cells
        lambda: qsa.update_pooled_keys(d, qsa.Seqs(1, 4096, None), FAKE, FAKE, 4, FAKE, None,
                                       stream=0),
        # nb_max beyond the capacity in blocks
        lambda: qsa.score_blocks(d, _seqs(), FAKE, FAKE, FAKE, 1, FAKE, FAKE, 4097, FAKE, 5000,
                                 stream=0),
        # ld below nb_max
        lambda: qsa.select_topk_blocks(d, _seqs(), FAKE, 10, FAKE, FAKE, 1, 64, FAKE, FAKE, FAKE,
                                       stream=0),
        # a score row is required whenever blocks compete (nb_max > 0); with
        # nb_max = 0 the row is never read and may be NULL (GPU test)
        lambda: qsa.select_topk_blocks(d, _seqs(), None, 64, FAKE, FAKE, 1, 64, FAKE, FAKE,
                                       FAKE, stream=0),
        # unknown score mode
        lambda: qsa.score_blocks(d, _seqs(), FAKE, FAKE, FAKE, 1, FAKE, FAKE, 64, FAKE, 64,
                                 mode=5, stream=0),
        # misaligned attention query
        lambda: qsa.sparse_attn_decode(d, _seqs(), FAKE + 4, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, 1 << 30, stream=0),
    ]
    for fn in cases:
        with pytest.raises(qsa.QsaError) as e:
            fn()
        assert e.value.code == qsa.QSA_EINVAL, qsa.load().qsa_last_error()


def test_workspace_too_small_rejected():
    d = qsa.Dims()
    with pytest.raises(qsa.QsaError) as e:
        qsa.sparse_attn_decode(d, _seqs(), FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                               stream=0)
    assert e.value.code == qsa.QSA_EWS
    with pytest.raises(qsa.QsaError) as e:
        qsa.score_blocks(d, _seqs(), FAKE, FAKE, FAKE, 4, FAKE, FAKE, 64, FAKE, 64,
                         mode=qsa.SCORE_BF16, ws=None, ws_bytes=0, stream=0)
    assert e.value.code == qsa.QSA_EWS


def test_empty_calls_are_noops():
    d = qsa.Dims()
    qsa.update_pooled_keys(d, _seqs(), FAKE, FAKE, 0, FAKE, None, stream=0)
    qsa.score_blocks(d, _seqs(), FAKE, FAKE, FAKE, 0, FAKE, FAKE, 64, FAKE, 64, stream=0)
    qsa.select_topk_blocks(d, _seqs(), FAKE, 64, FAKE, FAKE, 0, 64, FAKE, FAKE, FAKE, stream=0)
    assert qsa.load().qsa_last_error() == b""


def test_fused_select_attend_limits():
    d = qsa.Dims()
    big = 70000  # blocks: above the 65536 the fused selection holds on chip
    with pytest.raises(qsa.QsaError) as e:
        qsa.decode_select_attend(d, _seqs(cap=280064), FAKE, FAKE, 1, big, FAKE, big, FAKE, FAKE,
                                 FAKE, FAKE, 1 << 30, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                 stream=0)
    assert e.value.code == qsa.QSA_ENOTSUP
    need = qsa.workspace_size(d, qsa.OP_SCORE_SELECT, 1, 4000)
    with pytest.raises(qsa.QsaError) as e:  # candidate workspace too small
        qsa.decode_select_attend(d, _seqs(), FAKE, FAKE, 1, 4000, FAKE, 4000, FAKE, FAKE, FAKE,
                                 FAKE, need - 8, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0)
    assert e.value.code == qsa.QSA_EWS
    with pytest.raises(qsa.QsaError) as e:  # attention workspace too small
        qsa.decode_select_attend(d, _seqs(), FAKE, FAKE, 1, 4000, FAKE, 4000, FAKE, FAKE, FAKE,
                                 FAKE, need, FAKE, FAKE, FAKE, FAKE, FAKE, 16, stream=0)
    assert e.value.code == qsa.QSA_EWS
    qsa.decode_select_attend(d, _seqs(), FAKE, FAKE, 0, 4000, FAKE, 4000, FAKE, FAKE, FAKE,
                             FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, stream=0)  # n_q = 0: no-op


def test_prefill_indexer_workspace_and_limits():
    d = qsa.Dims()
    a256 = lambda x: -(-x // 256) * 256
    n_grp = -(-49785 // 256) * 4  # 64-block groups, 4 per 256 blocks
    # subgroup maxima (4 per group), thresholds, group masks, roped queries,
    # Delta, each query's (sequence, causal blocks)
    want = (a256(512 * n_grp * 4 * 4) + a256(512 * 4) + a256(512 * n_grp * 8)
            + a256(512 * 128 * 2) + a256(512 * 4) + a256(512 * 8))
    assert qsa.workspace_size(d, qsa.OP_SCORE_SELECT_PREFILL, 512, 49785) == want
    assert qsa.workspace_size(d, qsa.OP_SCORE_SELECT_PREFILL, 0, 49785) == 0
    big = 131073  # blocks: above what the selection's bitmap holds
    seqs = _seqs(cap=4 * 131328)
    with pytest.raises(qsa.QsaError) as e:
        qsa.score_select_prefill(d, seqs, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1, big,
                                 FAKE, FAKE, FAKE, FAKE, 1 << 40, stream=0)
    assert e.value.code == qsa.QSA_ENOTSUP
    need = qsa.workspace_size(d, qsa.OP_SCORE_SELECT_PREFILL, 8, 4000)
    with pytest.raises(qsa.QsaError) as e:
        qsa.score_select_prefill(d, _seqs(), FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 4000,
                                 FAKE, FAKE, FAKE, FAKE, need - 16, stream=0)
    assert e.value.code == qsa.QSA_EWS
    with pytest.raises(qsa.QsaError) as e:  # the bf16 key copy is required here
        qsa.score_select_prefill(d, _seqs(), FAKE, FAKE, 4, FAKE, None, FAKE, FAKE, FAKE, 8, 4000,
                                 FAKE, FAKE, FAKE, FAKE, need, stream=0)
    assert e.value.code == qsa.QSA_EINVAL
    qsa.score_select_prefill(d, _seqs(), FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4000,
                             FAKE, FAKE, FAKE, FAKE, 0, stream=0)  # nothing to do: no-op


def test_no_kernel_spills_to_scratch():
    """Every kernel keeps its register arrays in registers: a spilled key or
    tile array would turn the register-resident loops into memory traffic."""
    import json
    import os
    from top_sparse_attention_pooled_amd import build
    if not os.path.exists(build.RESOURCES):
        pytest.skip("library not built")
    res = json.load(open(build.RESOURCES))
    assert res, "no kernel resource report"
    spilled = {k: v["scratch"] for k, v in res.items() if v.get("scratch", 0) > 0}
    assert not spilled, spilled


def test_bf16_key_storage_helpers():
    """The bf16 per-cell key storage used by the tests: round to nearest even
    (as torch rounds) and an exact widening back."""
    import numpy as np
    import torch
    from top_sparse_attention_pooled_amd import synth
    x = np.random.default_rng(3).standard_normal(50000).astype(np.float32) * 7
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties go to even
    bits = synth.to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)
    assert np.array_equal(synth.widen_kidx(bits),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_noalloc_decode_attention_rejects_oversize_before_any_device_work():
    """The allocation-free entry point holds 8 MiB of partial states per GPU:
    64 queries of 16 heads over 2051-cell lists need more, and the call says
    so before touching the device (no GPU needed for this check)."""
    d = qsa.Dims()
    with pytest.raises(qsa.QsaError) as e:
        qsa.sparse_attn_decode_noalloc(d, _seqs(), FAKE, FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       stream=0)
    assert e.value.code == qsa.QSA_EWS
    assert "scratch" in str(e.value)


def test_probes_reject_bad_arguments_before_any_device_work():
    """The memory-traffic probes validate like the other calls: a source that
    is not whole 16-byte words, a misaligned source, an empty sink, and the
    gather probe on a cache type its q8_0 kernel does not read."""
    for src, n, n_sink in ((FAKE, 24, 1), (FAKE + 8, 32, 1), (FAKE, 32, 0), (None, 32, 1)):
        with pytest.raises(qsa.QsaError) as e:
            qsa.probe_stream_read(src, n, FAKE, n_sink, stream=0)
        assert e.value.code == qsa.QSA_EINVAL
    d = qsa.Dims(kv_type=qsa.KV_F16)
    with pytest.raises(qsa.QsaError) as e:
        qsa.probe_gather_prefill(d, _seqs(), FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1, stream=0)
    assert e.value.code == qsa.QSA_ENOTSUP
    with pytest.raises(qsa.QsaError) as e:
        qsa.probe_gather_prefill(qsa.Dims(), _seqs(), FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                                 stream=0)
    assert e.value.code == qsa.QSA_EINVAL


def test_union_decode_attention_validates_before_any_device_work():
    """qsa_sparse_attn_decode_union: t_group outside 1..8, a cache type or
    head layout it does not read, too many entries per group, a short
    workspace -- all rejected on the host; its workspace is the union lists
    plus the per-run partial states."""
    d = qsa.Dims()
    ld = d.ld_cells
    args = (FAKE, FAKE, 5)
    for t, code in ((0, qsa.QSA_EINVAL), (9, qsa.QSA_EINVAL)):
        with pytest.raises(qsa.QsaError) as e:
            qsa.sparse_attn_decode_union(d, _seqs(), *args, t, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         1 << 30, stream=0)
        assert e.value.code == code
    for dd in (qsa.Dims(kv_type=qsa.KV_F16), qsa.Dims(n_head_kv=8), qsa.Dims(top_k=4096)):
        with pytest.raises(qsa.QsaError) as e:
            qsa.sparse_attn_decode_union(dd, _seqs(), *args, 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, 1 << 30, stream=0)
        assert e.value.code == qsa.QSA_ENOTSUP
    need = qsa.workspace_size(d, qsa.OP_ATTN_DECODE_UNION, 5, 5)
    cap = 5 * ld
    runs = -(-cap // 64)
    rnd = lambda x: -(-x // 256) * 256
    assert need == rnd(cap * 4) + rnd(cap) + rnd(4) + rnd(2 * runs * 5 * 8 * 258 * 4)
    with pytest.raises(qsa.QsaError) as e:
        qsa.sparse_attn_decode_union(d, _seqs(), *args, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     need - 16, stream=0)
    assert e.value.code == qsa.QSA_EWS
