"""Pins for the oracle's score, bonus/floor policy and top-B selection (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import policy, score, select

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_row(rng, T, G, W, d):
    return rng.standard_normal((T, d)), rng.standard_normal((G, W, d))


@pytest.mark.parametrize("T,G,W,d", [(64, 4, 16, 64), (300, 2, 5, 32), (37, 7, 3, 16)])
def test_score_mass_is_window_times_group(T, G, W, d):
    rng = np.random.default_rng(T)
    K, Q = _rand_row(rng, T, G, W, d)
    s = score.obs_window_score(K, Q, W)
    assert s.sum() == pytest.approx(W * G, rel=1e-12)
    assert np.all(s >= 0)


def test_score_zero_queries_closed_form():
    # q = 0: every visible key gets 1/(pos+1) from a query at position pos.
    T, G, W, d = 50, 3, 8, 16
    K = np.random.default_rng(0).standard_normal((T, d))
    s = score.obs_window_score(K, np.zeros((G, W, d)), W)
    j = np.arange(T)
    exp = np.zeros(T)
    for w in range(W):
        pos = T - W + w
        exp += G * (j <= pos) / (pos + 1)
    np.testing.assert_allclose(s, exp, rtol=1e-13)


def test_score_single_query_is_torch_softmax():
    # W = G = 1: the one query sits at the last position and sees every key.
    rng = np.random.default_rng(5)
    T, d = 200, 64
    K, Q = _rand_row(rng, T, 1, 1, d)
    ref = torch.softmax(torch.from_numpy(Q[0, 0] @ K.T / np.sqrt(d)), dim=0).numpy()
    np.testing.assert_allclose(score.obs_window_score(K, Q, 1), ref, rtol=1e-13)


def test_score_causal_window():
    # The last key is seen only by the last window query; with q = 0 for all but that
    # query, its score is exactly that query's weight.
    T, W, d = 40, 4, 8
    rng = np.random.default_rng(6)
    K = rng.standard_normal((T, d))
    Q = np.zeros((1, W, d))
    Q[0, W - 1] = rng.standard_normal(d)
    s = score.obs_window_score(K, Q, W)
    logits = K @ Q[0, W - 1] / np.sqrt(d)
    last = np.exp(logits[-1]) / np.exp(logits).sum()
    assert s[-1] == pytest.approx(last, rel=1e-12)
    # key T-2 is seen by queries at T-2 and T-1 (window slots W-2, W-1)
    mid = np.exp(logits[-2]) / np.exp(logits).sum() + 1.0 / (T - 1)
    assert s[-2] == pytest.approx(mid, rel=1e-12)


def test_score_groups_add():
    rng = np.random.default_rng(7)
    T, G, W, d = 90, 4, 6, 32
    K, Q = _rand_row(rng, T, G, W, d)
    total = score.obs_window_score(K, Q, W)
    parts = sum(score.obs_window_score(K, Q[g:g + 1], W) for g in range(G))
    np.testing.assert_allclose(total, parts, rtol=1e-13)


def test_score_dominant_key():
    # A key aligned with every query and far larger than the rest takes ~all the mass.
    T, G, W, d = 64, 2, 4, 32
    rng = np.random.default_rng(8)
    K = rng.standard_normal((T, d)) * 0.01
    u = rng.standard_normal(d)
    K[10] = 50 * u
    Q = np.broadcast_to(u, (G, W, d)).copy()
    s = score.obs_window_score(K, Q, W)
    assert s[10] == pytest.approx(G * W, rel=1e-6)


def test_layer_groups_reproduce_pask_examples():
    g = json.load(open(os.path.join(GOLDEN, "pask_layer_groups.json")))
    for case in g["cases"]:
        got = policy.group_ranges(case["n_layers"], g["n_groups"])
        assert [list(r) for r in got] == case["ranges"], case["model"]


def test_layer_groups_four_way():
    assert policy.group_ranges(32, 4) == [(0, 7), (8, 15), (16, 23), (24, 31)]
    assert policy.group_ranges(36, 1) == [(0, 35)]


def test_foresight_bonus_floor_and_order():
    g = json.load(open(os.path.join(GOLDEN, "pace_foresight.json")))
    sig, lam = g["sigma"], g["lambda"]
    vals = [policy.foresight_bonus(sig, lam, k) for k in range(60)]
    assert vals[0] == sig                                # needed now: full scale
    assert all(a > b for a, b in zip(vals, vals[1:]))    # soonest-needed ranks highest
    assert vals[-1] > g["floor"] > g["max_observed_score"]
    assert vals[-1] == pytest.approx(g["floor"], rel=1e-8)
    assert policy.foresight_bonus(sig, lam, 10**6) == g["floor"]   # the limit is the floor
    assert policy.foresight_bonus(sig, lam, None) == 0.0


def test_protection_masks():
    T = 20
    tags = np.zeros(T, np.int64)
    tags[7] = 2
    bonus = np.array([[0.0, 0.0], [5.0, 6.0], [1.0, 2.0]])
    floor = np.array([[0, 0], [0, 0], [0, 1]])
    s = np.linspace(0, 1, T)
    tot, prot = policy.totals_and_protection(s, tags, bonus, floor, 1, 3, 4)
    assert tot[7] == pytest.approx(s[7] + 2.0)
    assert tot[6] == s[6]
    assert list(np.flatnonzero(prot)) == [0, 1, 2, 7, 16, 17, 18, 19]
    _, prot0 = policy.totals_and_protection(s, tags, bonus, floor, 0, 3, 4)
    assert 7 not in np.flatnonzero(prot0)


def _brute_force_keep(total, protected, B):
    """Enumerate every B-subset containing the protected set; keep the one with the
    largest total mass (unique for distinct totals)."""
    T = len(total)
    P = set(np.flatnonzero(protected))
    best, best_sum = None, -np.inf
    for S in itertools.combinations(range(T), B):
        if not P.issubset(S):
            continue
        v = sum(total[i] for i in S)
        if v > best_sum:
            best, best_sum = S, v
    return list(best)


def test_select_brute_force_small():
    rng = np.random.default_rng(9)
    for trial in range(40):
        T = rng.integers(4, 11)
        B = rng.integers(1, T)
        total = rng.standard_normal(T)
        prot = rng.random(T) < 0.2
        if prot.sum() > B:
            continue
        kept, excess = select.select_top_b(total, prot, B)
        assert not excess
        assert list(kept) == _brute_force_keep(total, prot, B)


def test_select_ties_go_to_earlier_position():
    total = np.array([1.0, 3.0, 2.0, 2.0, 2.0, 0.5, 2.0])
    kept, _ = select.select_top_b(total, np.zeros(7, bool), 3)
    assert list(kept) == [1, 2, 3]


def test_select_invariants_and_edge_cases():
    rng = np.random.default_rng(10)
    T, B = 500, 64
    total = np.round(rng.standard_normal(T), 1)          # many ties
    prot = np.zeros(T, bool)
    prot[:4] = True
    prot[-16:] = True
    kept, excess = select.select_top_b(total, prot, B)
    assert not excess and kept.size == B
    assert np.all(np.diff(kept) > 0)
    assert set(np.flatnonzero(prot)).issubset(kept)
    free_kept = np.setdiff1d(kept, np.flatnonzero(prot))
    dropped = np.setdiff1d(np.arange(T), kept)
    thr = total[free_kept].min()
    assert total[dropped].max() <= thr
    # every dropped token tied with the threshold comes after every kept tied one
    tied_kept = free_kept[total[free_kept] == thr]
    tied_drop = dropped[total[dropped] == thr]
    if tied_drop.size:
        assert tied_kept.max() < tied_drop.min()
    # T <= B keeps all; floor excess keeps every protected token
    k2, e2 = select.select_top_b(total[:50], prot[:50], 64)
    assert list(k2) == list(range(50)) and not e2
    allp = np.ones(T, bool)
    k3, e3 = select.select_top_b(total, allp, B)
    assert e3 and k3.size == T
