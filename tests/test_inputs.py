"""The seeded input recipes (no GPU): the AR(1) indexer queries of the
prefill variant follow their recursion and have the stated correlation."""
import numpy as np

from top_sparse_attention_pooled_amd import synth


def test_ar1_rows_recursion_and_moments():
    x = synth.normal((512, 128), 4, 0, synth.T_QIDX)
    rho = 0.9
    y = synth.ar1_rows(x, rho).astype(np.float64)
    assert np.array_equal(y[0], x[0].astype(np.float64))
    # the recursion, up to the float32 rounding of each row
    c = np.sqrt(1 - rho * rho)
    assert np.allclose(y[1:], rho * y[:-1] + c * x[1:], atol=1e-5)
    # unit variance and lag-1 correlation rho (512 x 128 samples)
    assert abs(y.var() - 1.0) < 0.1
    lag1 = np.mean(y[1:] * y[:-1]) / np.mean(y * y)
    assert abs(lag1 - rho) < 0.02
    # an independent series has no such correlation
    assert abs(np.mean(x[1:] * x[:-1])) < 0.02


def test_prefill_ar1_workload_changes_only_the_indexer_queries():
    a, b = synth.WORKLOADS["prefill"], synth.WORKLOADS["prefill_ar1"]
    qa = synth.make_queries(a, 0)
    qb = synth.make_queries(b, 0)
    assert np.array_equal(qb[0], synth.ar1_rows(qa[0], 0.9))
    for u, v in zip(qa[1:], qb[1:]):
        assert np.array_equal(u, v)
