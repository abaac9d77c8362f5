"""The seeded input generator: determinism, sub-range regeneration, rounding and the shape of
the distributions the workloads ask for."""
import numpy as np
from scipy import stats

import synth
from synth import workloads as W


def test_same_seed_same_bits_and_subranges():
    a = synth.normal(7, 1, 0, 100000)
    b = synth.normal(7, 1, 0, 100000)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = synth.normal(7, 1, 31337, 1000)
    assert np.array_equal(a[31337:32337].view(np.uint32), c.view(np.uint32))
    assert not np.array_equal(a[:1000], synth.normal(7, 2, 0, 1000))
    assert not np.array_equal(a[:1000], synth.normal(8, 1, 0, 1000))


def test_bf16_is_rne_of_fp32():
    f = synth.normal(3, 2, 0, 50000, 0.0, 3.0)
    h = synth.normal_bf16_bits(3, 2, 0, 50000, 0.0, 3.0)
    u = f.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(h, want)
    g = synth.normal(3, 2, 0, 50000, 0.0, 3.0, bf16=True)
    assert np.array_equal(g.view(np.uint32), h.astype(np.uint32) << 16)


def test_normal_distribution_shape():
    x = synth.normal(11, 4, 0, 1_000_000).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    assert abs(stats.kurtosis(x)) < 0.03 and abs(stats.skew(x)) < 0.02
    assert stats.kstest(x[:200000], "norm").pvalue > 1e-4
    y = synth.normal(11, 4, 0, 100000, 0.0, 2.0).astype(np.float64)
    assert abs(y.std() - 2) < 0.03


def test_uniform_range():
    u = synth.uniform(5, 6, 0, 200000)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 5e-3


def test_spike_basis_is_orthonormal():
    U = synth.spike_basis(1002, 9, 4, 128)
    np.testing.assert_allclose(U @ U.T, np.eye(4), atol=1e-13)


def test_index_keys_rows_regenerate():
    U = synth.spike_basis(1, 9, 4, 16)
    full = synth.index_keys(1, 7, 8, 0, 50, 16, U, 8.0, True)
    part = synth.index_keys(1, 7, 8, 20, 5, 16, U, 8.0, True)
    assert np.array_equal(full[20:25], part)
    # The spike makes the keys low-rank-dominated: the top 4 singular values carry most energy.
    raw = synth.index_keys(1, 7, 8, 0, 4000, 16, U, 8.0, False).astype(np.float64)
    sv = np.linalg.svd(raw, compute_uv=False)
    assert (sv[:4] ** 2).sum() / (sv ** 2).sum() > 0.7


def test_workload_shapes():
    wl = W.workload(4)
    assert int(wl.cu_groups(wl.layers[0])[-1]) == 262144
    wl5 = W.workload(5)
    assert wl5.batch == 64
    assert all(190000 <= n <= 210000 for n in wl5.lengths)
    assert len(set(n % 4 for n in wl5.lengths)) > 1          # groups end mid-window
    assert int(W.workload(3).cu_groups(W.workload(3).layers[0])[-1]) == 4 * 8192


def test_topk_score_variants():
    wl = W.workload(4)
    s = W.topk_scores(wl, "normal")
    d = W.topk_scores(wl, "dup10")
    n = wl.topk_len
    changed = np.flatnonzero(s != d)
    assert len(changed) <= n // 10
    vals, counts = np.unique(d, return_counts=True)
    assert (counts > 1).sum() > n // 20
    t = W.topk_scores(wl, "tie64")
    tau = np.sort(s)[::-1][511]
    assert (t == tau).sum() >= 64
