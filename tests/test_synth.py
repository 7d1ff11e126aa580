"""The seeded input generator: determinism, shapes and the stated distributions."""
import numpy as np


def test_deterministic_and_counter_based(syn):
    base = syn.config_seed(2)
    a, _, _ = syn.mixture_keys(base, 3, 200, 64, 8, 0.3, 4, 10.0, syn.BF16)
    b, _, _ = syn.mixture_keys(base, 3, 200, 64, 8, 0.3, 4, 10.0, syn.BF16)
    assert a.tobytes() == b.tobytes()
    # tokens 150..199 drawn on their own equal rows 150..199 of the full draw
    c, _, _ = syn.mixture_keys(base, 3, 50, 64, 8, 0.3, 4, 10.0, syn.BF16, i0=150)
    assert np.array_equal(c, a[:, 150:])
    assert not np.array_equal(a, syn.mixture_keys(syn.config_seed(3), 3, 200, 64, 8, 0.3, 4, 10.0, syn.BF16)[0])


def test_mixture_statistics(syn, orc):
    base = syn.config_seed(4)
    K, comp, means = syn.mixture_keys(base, 2, 20000, 128, 16, 0.3, 4, 10.0, syn.F32, want_comp=True,
                                      want_means=True)
    for h in range(2):
        counts = np.bincount(comp[h], minlength=16)
        assert counts.min() > 20000 / 16 * 0.85
        scale = np.abs(means[h]).mean(axis=0)
        out = np.argsort(scale)[-4:]
        assert np.all(scale[out] > 4 * np.median(scale))  # four channels scaled by 10
        resid = K[h] - means[h][comp[h]]
        s = resid.std(axis=0)
        np.testing.assert_allclose(np.sort(s)[:124], 0.3, rtol=0.05)
        np.testing.assert_allclose(np.sort(s)[124:], 3.0, rtol=0.05)
    v = syn.values(base, 2, 5000, 128, syn.F32)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01


def test_init_idx_and_queries(syn):
    base = syn.config_seed(5)
    idx = syn.init_idx(base, 4, 1000, 400)
    for h in range(4):
        assert len(set(idx[h].tolist())) == 400 and idx[h].min() >= 0 and idx[h].max() < 1000
    assert not np.array_equal(idx[0], idx[1])
    K, _, means = syn.mixture_keys(base, 2, 300, 128, 8, 0.3, 4, 10.0, syn.BF16, want_means=True)
    q = syn.queries_noisy_key(base, 0, 2, 1, K, 300, 0.1)
    assert q.shape == (2, 128) and q.dtype == np.uint16
    qm = syn.queries_mixture(base, 3, 8, 4, means, 0.2)
    assert qm.shape == (8, 128)
    assert not np.array_equal(qm, syn.queries_mixture(base, 4, 8, 4, means, 0.2))


def test_drifting_queries(syn):
    """Drifting mixture queries: deterministic; with no change events (p = 0)
    and no noise every step gives the same query; with a change at every step
    (p = 1) consecutive queries differ; fresh noise alone keeps the mean part."""
    base = syn.config_seed(4)
    _, _, means = syn.mixture_keys(base, 2, 64, 16, 16, 0.3, 0, 1.0, syn.F32, want_means=True)
    q = lambda s, sig, p: syn.queries_drift(base, s, 4, 2, means, sig, p, syn.F32)
    assert np.array_equal(q(5, 0.2, 0.1), q(5, 0.2, 0.1))
    assert all(np.array_equal(q(0, 0.0, 0.0), q(s, 0.0, 0.0)) for s in (1, 7, 30))
    assert not np.array_equal(q(3, 0.0, 1.0), q(4, 0.0, 1.0))
    assert not np.array_equal(q(3, 0.2, 0.0), q(4, 0.2, 0.0))
