"""Pins for the oracle's H2O cumulative-attention scoring and eviction (CPU only)."""
import itertools

import numpy as np
import scipy.special

from oracle import decode, h2o


def test_mass_sums_to_group_size_and_matches_library_softmax():
    rng = np.random.default_rng(1)
    for G, n, d in [(1, 7, 16), (4, 300, 64), (7, 33, 128)]:
        q = rng.standard_normal((G, d))
        K = rng.standard_normal((n, d)) * 3
        m = h2o.attention_mass(q, K)
        assert m.shape == (n,) and np.all(m >= 0)
        np.testing.assert_allclose(m.sum(), G, rtol=1e-12)
        lib = scipy.special.softmax(K @ q.T / np.sqrt(d), axis=0).sum(axis=1)
        np.testing.assert_allclose(m, lib, rtol=1e-12, atol=1e-15)


def test_equal_keys_share_the_mass_evenly():
    rng = np.random.default_rng(2)
    G, n, d = 4, 50, 32
    K = np.tile(rng.standard_normal(d), (n, 1))
    m = h2o.attention_mass(rng.standard_normal((G, d)), K)
    np.testing.assert_allclose(m, np.full(n, G / n), rtol=1e-12)


def test_mass_equals_decode_weights_read_through_identity_values():
    # decode_head's output with V = I (one unit vector per key) is the weight
    # vector itself: the two oracles agree head by head.
    rng = np.random.default_rng(3)
    G, n, d = 3, 20, 32
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((n, d))
    V = np.eye(n, d)
    w = sum(decode.decode_head(q[g], K, V)[0][:n] for g in range(G))
    np.testing.assert_allclose(h2o.attention_mass(q, K), w, rtol=1e-12, atol=1e-15)


def test_eviction_is_the_best_subset_by_brute_force():
    # distinct totals: the kept set is the size-B superset of the protected
    # slots with the largest total, found here by enumerating all subsets
    rng = np.random.default_rng(4)
    T, B = 11, 6
    for trial in range(20):
        acc = rng.random(T) * 5
        tags = rng.integers(0, 3, T)
        bonus = np.array([[0.0], [2.0], [0.5]])
        floor = np.array([[0], [0], [trial % 2]])
        kept = h2o.evict(acc, tags, bonus, floor, 0, 1, 2, B)
        total = acc + bonus[tags, 0]
        prot = set([0, T - 2, T - 1]) | {j for j in range(T) if floor[tags[j], 0]}
        if len(prot) >= B:
            assert set(kept) == prot
            continue
        best = max((c for c in itertools.combinations(range(T), B) if prot <= set(c)),
                   key=lambda c: sum(total[list(c)]))
        np.testing.assert_array_equal(kept, np.array(sorted(best)))


def test_heavy_hitter_and_foresight_survive_churn_and_mass_is_conserved():
    """A key aligned with every query (a heavy hitter) and a tagged span with a
    bonus above any attainable cumulative score stay resident through many
    evictions; every step adds exactly G to the resident plus evicted scores."""
    rng = np.random.default_rng(5)
    G, d, B, E, steps = 4, 32, 24, 8, 64
    heavy_dir = rng.standard_normal(d)
    K = rng.standard_normal((B, d))
    K[3] = heavy_dir * 2.0
    acc = np.zeros(B)
    tags = np.zeros(B, np.int64)
    tags[10:14] = 1
    ident = np.arange(B)                      # which original token each slot holds
    bonus = np.array([[0.0], [1e3]])
    floor = np.zeros((2, 1), np.uint8)
    evicted = 0.0
    next_id = B
    for t in range(steps):
        K = np.vstack([K, rng.standard_normal(d)])
        acc = np.append(acc, 0.0)
        tags = np.append(tags, 0)
        ident = np.append(ident, next_id)
        next_id += 1
        q = heavy_dir / np.linalg.norm(heavy_dir) * 2 + 0.3 * rng.standard_normal((G, d))
        before = acc.sum()
        acc = h2o.accumulate(acc, q, K)
        np.testing.assert_allclose(acc.sum() - before, G, rtol=1e-12)
        if (t + 1) % E == 0:
            kept = h2o.evict(acc, tags, bonus, floor, 0, 2, 4, B)
            assert kept.size == B and np.all(np.diff(kept) > 0)
            assert {0, 1} <= set(kept) and set(range(acc.size - 4, acc.size)) <= set(kept)
            evicted += acc.sum() - acc[kept].sum()
            K, acc, tags, ident = K[kept], acc[kept], tags[kept], ident[kept]
            assert 3 in ident and set(range(10, 14)) <= set(ident)
    np.testing.assert_allclose(acc.sum() + evicted, G * steps, rtol=1e-12)
    assert acc[list(ident).index(3)] > 0.5 * G * steps     # the heavy hitter took most of the mass
