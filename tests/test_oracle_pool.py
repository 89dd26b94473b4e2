"""Pins for the oracle's score pooling (CPU only)."""
import numpy as np
import scipy.ndimage

from oracle import score


def test_kernel_one_is_identity():
    s = np.random.default_rng(1).random(50)
    for mode in ("max", "avg"):
        np.testing.assert_array_equal(score.pool_scores(s, 1, mode), s)


def test_max_pool_matches_library_filter():
    # replicating the edge value adds no new value to a max, so the cut window
    # equals scipy's 'nearest' mode
    rng = np.random.default_rng(2)
    for k in (3, 5, 7, 63):
        s = rng.random(500)
        np.testing.assert_array_equal(score.pool_scores(s, k, "max"),
                                      scipy.ndimage.maximum_filter1d(s, k, mode="nearest"))


def test_avg_pool_interior_matches_library_and_edges_are_cut_means():
    rng = np.random.default_rng(3)
    k, T = 7, 300
    s = rng.random(T)
    got = score.pool_scores(s, k, "avg")
    lib = scipy.ndimage.uniform_filter1d(s, k, mode="constant")
    np.testing.assert_allclose(got[3:-3], lib[3:-3], rtol=1e-12)
    assert got[0] == s[:4].mean() and got[1] == s[:5].mean() and got[-1] == s[-4:].mean()


def test_spike_spreads_to_a_plateau_and_constants_stay():
    s = np.zeros(40)
    s[20] = 5.0
    m = score.pool_scores(s, 5, "max")
    np.testing.assert_array_equal(np.flatnonzero(m), np.arange(18, 23))
    a = score.pool_scores(s, 5, "avg")
    np.testing.assert_allclose(a[18:23], 1.0)
    np.testing.assert_allclose(score.pool_scores(np.full(9, 2.5), 7, "avg"), 2.5)
