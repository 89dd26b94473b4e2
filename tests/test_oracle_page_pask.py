"""Pins for the oracle's CommitKV page effects and PASK controller (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import page_effect as pe
from oracle import pask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_deletion_effect_equals_eq6_renormalisation():
    # CommitKV Eq. 6: o^{\E} = (o - sum_{i in E} a_i v_i) / (1 - sum_{i in E} a_i).
    rng = np.random.default_rng(20)
    Hkv, Hq, T, P, d = 2, 6, 96, 5, 16
    K = rng.standard_normal((Hkv, T, d))
    V = rng.standard_normal((Hkv, T, d))
    Q = rng.standard_normal((Hq, P, d))
    q_pos = np.arange(T - P, T)
    E = np.arange(32, 48)
    rel, ab = pe.deletion_effect(K, V, Q, q_pos, E)
    best_rel, best_abs = 0.0, 0.0
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        s = Q[h] @ K[kv].T / np.sqrt(d)
        s = np.where(np.arange(T)[None, :] <= q_pos[:, None], s, -np.inf)
        a = np.exp(s - s.max(1, keepdims=True))
        a /= a.sum(1, keepdims=True)
        o = a @ V[kv]
        aE = a[:, E]
        o_del = (o - aE @ V[kv][E]) / (1 - aE.sum(1, keepdims=True))
        diff = np.linalg.norm(o - o_del, axis=1)
        best_rel = max(best_rel, np.max(diff / np.linalg.norm(o, axis=1)))
        best_abs = max(best_abs, np.max(diff))
    assert rel == pytest.approx(best_rel, rel=1e-10)
    assert ab == pytest.approx(best_abs, rel=1e-10)


def test_deletion_effect_uniform_attention_closed_form():
    # q = 0: uniform attention, so o is the mean of visible values and o^{\E} the mean of
    # the rest.
    rng = np.random.default_rng(21)
    T, d = 64, 8
    K = rng.standard_normal((1, T, d))
    V = rng.standard_normal((1, T, d))
    Q = np.zeros((1, 1, d))
    E = np.arange(16, 32)
    rel, ab = pe.deletion_effect(K, V, Q, np.array([T - 1]), E)
    keep = np.setdiff1d(np.arange(T), E)
    o, o_del = V[0].mean(0), V[0][keep].mean(0)
    assert ab == pytest.approx(np.linalg.norm(o - o_del), rel=1e-12)
    assert rel == pytest.approx(np.linalg.norm(o - o_del) / np.linalg.norm(o), rel=1e-12)


def test_deletion_effect_empty_set_and_everything():
    rng = np.random.default_rng(22)
    K = rng.standard_normal((1, 20, 4))
    V = rng.standard_normal((1, 20, 4))
    Q = rng.standard_normal((2, 3, 4))
    assert pe.deletion_effect(K, V, Q, np.array([17, 18, 19]), []) == (0.0, 0.0)
    assert pe.deletion_effect(K, V, Q, np.array([17, 18, 19]), np.arange(20))[0] == np.inf


def test_deletion_effect_invisible_page_is_zero():
    rng = np.random.default_rng(23)
    K = rng.standard_normal((1, 40, 4))
    V = rng.standard_normal((1, 40, 4))
    Q = rng.standard_normal((1, 2, 4))
    # queries at positions 10, 11 never see tokens 20..35
    assert pe.deletion_effect(K, V, Q, np.array([10, 11]), np.arange(20, 36)) == (0.0, 0.0)


def test_percentiles_and_states():
    R = np.array([0.5, 0.1, 0.1, 0.9, 0.0])
    np.testing.assert_allclose(pe.percentile_ranks(R), [3 / 4, 1 / 4, 1 / 4, 4 / 4, 0])
    c = json.load(open(os.path.join(GOLDEN, "commitkv_constants.json")))
    # 5 pages: before/after effects chosen to land in each state of Eq. 10
    Rm = np.array([0.30, 0.001, 0.0005, 0.40, 0.02])
    Rp = np.array([0.0008, 0.0009, 0.50, 0.60, 0.02])
    st = pe.lifecycle_states(Rm, Rp, c["tau_use"], c["tau_dead"], c["rho_use"], c["rho_dead"])
    names = [pe.STATES[s] for s in st]
    assert names == ["completion_candidate", "dormant", "newly_active", "still_active", "uncertain"]


def test_candidate_order_and_greedy():
    Rm = np.array([0.5, 0.9, 0.9, 0.2])
    Rp = np.array([0.001, 0.001, 0.001, 0.0001])
    st = np.array([1, 1, 1, 0])
    assert list(pe.candidate_order(Rm, Rp, st)) == [1, 2, 0]
    # additive joint effect: accept while the running sum stays within tau
    w = {0: 0.5, 1: 0.5, 2: 0.25, 3: 0.25}          # exact binary fractions
    D = pe.greedy_retire([1, 2, 0, 3], lambda S: sum(w[e] for e in S), 1.0)
    assert D == [1, 2, 3]
    assert pe.greedy_retire(list(range(100)), lambda S: 0.0, 1.0) == list(range(64))


def test_page_scores_hand_built():
    # 3 rows (layers x heads), T = 10, pages of 4: the tail tokens 8, 9 lie outside both pages
    rows = np.array([[1, 0, 0, 0, 2, 0, 0, 0, 9, 9],
                     [0, 1, 0, 0, 0, 0, 3, 0, 9, 9],
                     [0, 0, 0, 1, 0, 0, 0, 4, 9, 9]], dtype=float)
    np.testing.assert_array_equal(pe.page_scores(rows, 4, 2), [3.0, 9.0])


def test_page_scores_pool_every_row_closed_form():
    # window scores of a row sum to G*W (each query's weights sum to 1); pooled over
    # R rows and pages that tile the cache, the page scores sum to R*G*W
    from oracle import score as o_score
    rng = np.random.default_rng(3)
    R, T, d, G, W = 5, 96, 16, 3, 4
    rows = [o_score.obs_window_score(rng.standard_normal((T, d)), rng.standard_normal((G, W, d)), W)
            for _ in range(R)]
    ps = pe.page_scores(np.stack(rows), 8, T // 8)
    assert ps.sum() == pytest.approx(R * G * W, rel=1e-12)
    assert np.all(ps > 0)


def test_event_pages_cut_every_event_into_pages_of_at_most_G():
    # CommitKV §3.1: events of 37, 5, 16 and 17 tokens with G = 16
    first, length = pe.event_pages([37, 5, 16, 17], 16)
    np.testing.assert_array_equal(length, [16, 16, 5, 5, 16, 16, 1])
    np.testing.assert_array_equal(first, [0, 16, 32, 37, 42, 58, 74])
    # invariants on random events: the pages tile the events in order, none
    # longer than G, none crossing an event boundary
    rng = np.random.default_rng(3)
    ev = rng.integers(1, 90, 40)
    for G in (1, 7, 16, 64):
        first, length = pe.event_pages(ev, G, start=11)
        assert first[0] == 11 and first[-1] + length[-1] == 11 + ev.sum()
        np.testing.assert_array_equal(first[1:], first[:-1] + length[:-1])
        assert length.min() >= 1 and length.max() <= G
        bounds = 11 + np.concatenate([[0], np.cumsum(ev)])
        ev_of_first = np.searchsorted(bounds, first, side="right") - 1
        ev_of_last = np.searchsorted(bounds, first + length - 1, side="right") - 1
        np.testing.assert_array_equal(ev_of_first, ev_of_last)
        assert len(first) == sum(-(-int(n) // G) for n in ev)


def test_page_scores_spans_and_retained_tokens():
    S = np.arange(2 * 12, dtype=np.float64).reshape(2, 12)   # per-token sums 12, 14, ..., 34
    first, length = np.array([0, 3, 5, 10]), np.array([3, 2, 5, 2])
    np.testing.assert_array_equal(pe.page_scores_spans(S, first, length),
                                  [12 + 14 + 16, 18 + 20, 22 + 24 + 26 + 28 + 30, 32 + 34])
    # uniform spans reduce to page_scores
    rng = np.random.default_rng(4)
    R = rng.random((5, 96))
    np.testing.assert_allclose(pe.page_scores_spans(R, np.arange(6) * 16, np.full(6, 16)),
                               pe.page_scores(R, 16, 6), rtol=1e-15)
    np.testing.assert_array_equal(pe.retained_tokens(first, length, [3, 0, 2]),
                                  [10, 11, 0, 1, 2, 5, 6, 7, 8, 9])
    assert pe.retained_tokens(first, length, []).size == 0


def test_retained_pages_hand_built_and_brute_force():
    assert list(pe.retained_pages([5, 1, 5, 3, 7], {4}, 2)) == [0, 2]     # 7 retired; tie to the lower index
    assert list(pe.retained_pages([5, 1, 5, 3, 7], {4}, 4)) == [0, 1, 2, 3]
    assert list(pe.retained_pages([5, 1, 5, 3, 7], set(), 1)) == [4]
    assert list(pe.retained_pages([1, 2, 3], {2}, 3)) == [0, 1, 2]       # no more pages than the budget
    rng = np.random.default_rng(8)
    for _ in range(200):
        n = int(rng.integers(2, 12))
        sc = rng.integers(0, 4, n).astype(float)                          # many ties
        ret = set(rng.choice(n, int(rng.integers(0, n)), replace=False).tolist())
        k = int(rng.integers(1, n))
        kept = set(pe.retained_pages(sc, ret, k).tolist())
        assert len(kept) == k
        eff = np.where(np.isin(np.arange(n), list(ret)), -np.inf, sc)
        for a in kept:                                                    # every kept page outranks every dropped one
            for b in set(range(n)) - kept:
                assert (eff[a], -a) > (eff[b], -b)



def test_retained_pages_budget_hand_built():
    """Event pages under a token budget (CommitKV §3.3 Eq. 13, |I| <= B): the
    longest prefix of the (score desc, index asc) ranking that fits."""
    sc, ln = [5, 9, 9, 1, 7], [3, 4, 2, 5, 6]       # ranking: 1, 2, 4, 0, 3
    k, used = pe.retained_pages_budget(sc, ln, (), 12)
    assert list(k) == [1, 2, 4] and used == 12
    # page 4 does not fit after 1 and 2: the prefix ends there even though page 0 would fit
    k, used = pe.retained_pages_budget(sc, ln, (), 9)
    assert list(k) == [1, 2] and used == 6
    # equal scores go to the lower index first: page 1 (4 tokens) fits, page 2 then does not
    k, used = pe.retained_pages_budget(sc, ln, (), 5)
    assert list(k) == [1] and used == 4
    assert list(pe.retained_pages_budget(sc, ln, (), 100)[0]) == [0, 1, 2, 3, 4]
    assert pe.retained_pages_budget(sc, ln, (), 0)[0].size == 0
    # a retired page ranks last
    k, used = pe.retained_pages_budget(sc, ln, {1}, 9)
    assert list(k) == [2, 4] and used == 8
    k, used = pe.retained_pages_budget(sc, ln, {1}, 20)
    assert list(k) == [0, 1, 2, 3, 4] and used == 20
    # NaN below -inf; a zero-length page after the first misfit stays out
    assert list(pe.retained_pages_budget([np.nan, 1.0, -np.inf], [1, 1, 1], (), 2)[0]) == [1, 2]
    assert list(pe.retained_pages_budget([3.0, 2.0, 1.0], [2, 5, 0], (), 4)[0]) == [0]
    assert list(pe.retained_pages_budget([3.0, 2.0, 1.0], [2, 0, 5], (), 4)[0]) == [0, 1]


def test_retained_pages_budget_reduces_to_page_count_and_matches_subset_search():
    """Equal lengths G and a budget of k*G keep retained_pages' k pages; on
    tiny cases the kept set is the only subset that fits, contains every page
    ranked above any of its members, and cannot take the best page left."""
    rng = np.random.default_rng(31)
    for _ in range(100):
        n = int(rng.integers(2, 14))
        sc = rng.integers(0, 5, n).astype(float)
        ret = set(rng.choice(n, int(rng.integers(0, n)), replace=False).tolist())
        k, G = int(rng.integers(1, n)), int(rng.integers(1, 17))
        got, used = pe.retained_pages_budget(sc, np.full(n, G), ret, k * G + int(rng.integers(0, G)))
        assert list(got) == list(pe.retained_pages(sc, ret, k)) and used == k * G

    def above(s, a, b):          # page a ranks above page b
        if np.isnan(s[b]):
            return not np.isnan(s[a]) or a < b
        if np.isnan(s[a]):
            return False
        return s[a] > s[b] or (s[a] == s[b] and a < b)

    for _ in range(300):
        n = int(rng.integers(1, 8))
        sc = rng.integers(0, 4, n).astype(float)
        sc[rng.random(n) < 0.15] = np.nan
        ln = rng.integers(0, 6, n)
        ret = set(rng.choice(n, int(rng.integers(0, n + 1)), replace=False).tolist())
        B = int(rng.integers(0, ln.sum() + 2))
        eff = sc.copy()
        eff[list(ret)] = -np.inf
        fits = []
        for mask in range(1 << n):
            S = [e for e in range(n) if mask >> e & 1]
            rest = [e for e in range(n) if not mask >> e & 1]
            if ln[S].sum() > B:
                continue
            if any(above(eff, a, b) for b in S for a in rest):
                continue
            best = [e for e in rest if not any(above(eff, a, e) for a in rest if a != e)]
            if best and ln[S].sum() + ln[best[0]] <= B:
                continue
            fits.append(S)
        assert len(fits) == 1
        got, used = pe.retained_pages_budget(sc, ln, ret, B)
        assert list(got) == fits[0] and used == ln[fits[0]].sum()


# ---------------------------------------------------------------- PASK controller

def _rand_table(rng, n_tags, C):
    a0 = rng.integers(0, 3, (n_tags, C))
    amin = np.minimum(a0, rng.integers(0, 3, (n_tags, C)))
    prio = rng.random((n_tags, C, 2))
    crit = rng.random(n_tags) < 0.3
    return a0, amin, prio, crit


def test_payload_costs_eq13_14():
    c = pask.group_costs([8, 8, 8, 8], 8, 128)
    assert c[0][2] == 16 * 2 * 8 * 8 * 128          # m(H) = 16 n_c
    assert c[0][1] == 8 * 2 * 8 * 8 * 128 + 16 * 2 * 8 * 8
    assert c[0][0] == 0
    c4 = pask.group_costs([1], 1, 6, low_bits=4)    # PASK's INT4 form
    assert c4[0][1] == 4 * 12 + 16 * 2


def test_controller_floors_ledger_and_fallback():
    rng = np.random.default_rng(30)
    costs = pask.group_costs([8, 8, 8, 8], 8, 128)
    a0, amin, prio, crit = _rand_table(rng, 8, 4)
    tags = rng.integers(0, 8, 500)
    acts, ledger = pask.control_sequence(tags, a0, amin, prio, crit, costs, 1 / 3)
    assert np.all(acts >= amin[tags])                           # floors never violated
    b = costs[:, 2].sum() / 3
    M = np.array([pask.cost(a, costs) for a in acts])
    t = np.arange(1, len(tags) + 2)
    np.testing.assert_allclose(ledger, t * b - np.concatenate([[0], np.cumsum(M)]), rtol=1e-12)
    # all-high fallback: B_D = 1 and base actions all H keep every token H
    allH = np.full_like(a0, 2)
    acts2, _ = pask.control_sequence(tags, allH, np.zeros_like(amin), prio, crit, costs, 1.0)
    assert np.all(acts2 == 2)


def test_controller_step_brute_force_properties():
    rng = np.random.default_rng(31)
    costs = pask.group_costs([3, 2, 4], 2, 16)
    for trial in range(300):
        a0 = rng.integers(0, 3, 3)
        amin = np.minimum(a0, rng.integers(0, 3, 3))
        prio = rng.random((3, 2))
        crit = bool(rng.random() < 0.5)
        R_t = rng.uniform(-0.2, 1.2) * costs[:, 2].sum()
        a, M = pask.control_token(a0, amin, prio, crit, R_t, costs)
        B_t = max(R_t, 0.0)
        start = np.maximum(a0, amin)
        assert np.all(np.array(a) >= amin)
        if not crit:
            assert np.all(np.array(a) <= start)
            if M > B_t:
                assert list(a) == list(amin)              # only floors remain
            # demotion stops as soon as the cost fits: undoing the last step (one of
            # the demoted groups) no longer fits
            undo = []
            for c in range(3):
                if a[c] < start[c]:
                    up = list(a)
                    up[c] += 1
                    undo.append(pask.cost(up, costs) > B_t)
            assert not undo or any(undo)
        # brute force over all 3^3 action vectors: the result is one of the vectors
        # between the floor and H; with non-critical tags it never exceeds the start
        space = [v for v in itertools.product(range(3), repeat=3)
                 if all(v[c] >= amin[c] for c in range(3))]
        assert tuple(a) in space


def test_protection_budget_and_prefix_rule_commitkv_eq12():
    # CommitKV §3.3 Eq. 12 with the setup's eta = 0.125 and at most 16 pages:
    # B = 4096 gives B_N = 512 tokens; 16-token pages hit the 16-page cap first,
    # 48-token pages the token bound after 10 pages.
    Rm = np.linspace(1.0, 0.1, 30)
    np.testing.assert_array_equal(pe.protect_pending(Rm, np.full(30, 16), 4096, 0.125), np.arange(16))
    np.testing.assert_array_equal(pe.protect_pending(Rm, np.full(30, 48), 4096, 0.125), np.arange(10))
    # the largest effect does not fit: nothing after it is taken either
    tok = np.full(30, 16)
    tok[0] = 600
    assert pe.protect_pending(Rm, tok, 4096, 0.125).size == 0
    assert pe.protect_pending(Rm, np.full(30, 16), 4096, 0.0).size == 0


def test_retained_pages_keep_protected_and_drop_retired_eq13():
    score = np.array([5.0, 1.0, 4.0, 3.0, 2.0, 0.5])
    # keep 3: page 5 protected (lowest score), page 0 retired (highest)
    np.testing.assert_array_equal(pe.retained_pages(score, [0], 3, protected=[5]), [2, 3, 5])
    np.testing.assert_array_equal(pe.retained_pages(score, [], 3, protected=[]), [0, 2, 3])
    np.testing.assert_array_equal(pe.retained_pages(score, [0, 2], 2, protected=[1]), [1, 3])


# ---- PASK §3.5, Algorithm 2 (Demote, then Promote for critical tags): the order ----
# Demotion takes eligible adjacent steps in ascending stored priority; promotion
# takes them in descending priority and stops at the first step that does not fit.
# Demoting H->L undoes the upgrade L->H, so it carries that upgrade's stored
# priority (index 1); demoting L->R carries that of R->L (index 0).

_FLAT = np.array([[0.0, 5.0, 10.0]] * 4)      # m(R), m(L), m(H) per group


def test_demotion_takes_the_lowest_stored_priority_first():
    # two groups at H, a budget that allows exactly one demotion
    prio = [[0.5, 0.9], [0.5, 0.1]]            # group 1's L->H upgrade ranks lowest
    a, M = pask.control_token([2, 2], [0, 0], prio, False, 15.0, _FLAT[:2])
    assert a == [2, 1] and M == 15.0
    prio = [[0.5, 0.1], [0.5, 0.9]]
    a, _ = pask.control_token([2, 2], [0, 0], prio, False, 15.0, _FLAT[:2])
    assert a == [1, 2]


def test_demotion_uses_the_priority_of_the_upgrade_it_undoes():
    # H->L is priced by the L->H priority, not by R->L's
    prio = [[0.1, 0.9], [0.8, 0.2]]
    a, _ = pask.control_token([2, 2], [0, 0], prio, False, 15.0, _FLAT[:2])
    assert a == [2, 1]
    # L->R is priced by the R->L priority, not by L->H's
    prio = [[0.3, 0.9], [0.7, 0.1]]
    a, _ = pask.control_token([1, 1], [0, 0], prio, False, 5.0, _FLAT[:2])
    assert a == [0, 1]


def test_demotion_sequence_over_several_steps():
    # three groups at H, cost 30, budget 15: three demotions, each the cheapest
    # eligible step at its turn. Step 1: H->L of group 1 (0.2); step 2: H->L of
    # group 0 (0.5 < 0.8, group 1's L->R is 0.9); step 3: L->R of group 0 (0.3).
    prio = [[0.3, 0.5], [0.9, 0.2], [0.1, 0.8]]
    a, M = pask.control_token([2, 2, 2], [0, 0, 0], prio, False, 15.0, _FLAT[:3])
    assert a == [0, 1, 2] and M == 15.0


def test_demotion_skips_floored_groups_and_ties_go_to_the_lower_group():
    prio = [[0.5, 0.9], [0.5, 0.1]]
    # group 1 is floored at H: group 0 is demoted although its priority is higher
    a, _ = pask.control_token([2, 2], [0, 2], prio, False, 15.0, _FLAT[:2])
    assert a == [1, 2]
    # equal priorities: the lower group index goes first
    a, _ = pask.control_token([2, 2], [0, 0], [[0.4, 0.4], [0.4, 0.4]], False, 15.0, _FLAT[:2])
    assert a == [1, 2]


def test_promotion_takes_the_highest_priority_first_and_stops_at_the_first_misfit():
    costs = np.array([[0.0, 1.0, 2.0], [0.0, 5.0, 10.0], [0.0, 5.0, 10.0]])
    prio = [[0.4, 0.0], [0.6, 0.0], [0.0, 0.9]]
    # start [R, R, L], cost 5, budget 12. Promote L->H of group 2 (0.9): cost 10.
    # Next is R->L of group 1 (0.6): 15 > 12, so promotion stops there, although
    # group 0's cheaper step (0.4, +1) would still fit.
    a, M = pask.control_token([0, 0, 1], [0, 0, 0], prio, True, 12.0, costs)
    assert a == [0, 0, 2] and M == 10.0
    # the same table for a non-critical tag: no promotion at all
    a, _ = pask.control_token([0, 0, 1], [0, 0, 0], prio, False, 12.0, costs)
    assert a == [0, 0, 1]


def _chain_walk(steps_per_group, key):
    """Every interleaving of per-group step chains (each group's steps in their
    fixed order); returns the interleaving whose sequence of keys is
    lexicographically smallest, as a list of (group, step index)."""
    best = None
    counts = [len(s) for s in steps_per_group]
    groups = [c for c in range(len(counts)) for _ in range(counts[c])]
    for perm in set(itertools.permutations(groups)):
        seen = [0] * len(counts)
        seq = []
        for c in perm:
            seq.append((key(steps_per_group[c][seen[c]], c), c, seen[c]))
            seen[c] += 1
        cand = [k for k, _, _ in seq]
        if best is None or cand < best[0]:
            best = (cand, [(c, i) for _, c, i in seq])
    return best[1]


def _brute_force_token(a0, amin, prio, crit, R_t, costs):
    """Algorithm 2 restated as a search over step orders: the demotion order is
    the interleaving of the groups' demotion chains whose priorities read
    smallest first (ties by group index), walked until the cost fits; the
    promotion order is the interleaving whose priorities read largest first,
    walked while the cost still fits."""
    C = len(a0)
    a = [max(int(a0[c]), int(amin[c])) for c in range(C)]
    B = max(R_t, 0.0)
    cost = lambda v: sum(costs[c][v[c]] for c in range(C))
    # demotion chain of group c: a[c] -> a[c]-1 -> ... -> amin[c]; the step from
    # level k to k-1 carries the priority of the upgrade k-1 -> k
    chains = [[prio[c][k - 1] for k in range(a[c], int(amin[c]), -1)] for c in range(C)]
    for c, _ in _chain_walk(chains, lambda p, c: (p, c)):
        if cost(a) <= B:
            break
        a[c] -= 1
    if crit:
        chains = [[prio[c][k] for k in range(a[c], 2)] for c in range(C)]
        for c, _ in _chain_walk(chains, lambda p, c: (-p, c)):
            up = list(a)
            up[c] += 1
            if cost(up) > B:
                break
            a = up
    return a


def test_controller_matches_the_order_derived_by_search_over_all_step_orders():
    rng = np.random.default_rng(32)
    for trial in range(400):
        C = int(rng.integers(2, 4))
        costs = np.array([[0.0, float(rng.integers(1, 6)), 0.0] for _ in range(C)])
        costs[:, 2] = costs[:, 1] + rng.integers(1, 6, C)
        a0 = rng.integers(0, 3, C)
        amin = np.minimum(a0, rng.integers(0, 3, C))
        prio = rng.random((C, 2)).round(1)          # coarse values make ties common
        crit = bool(rng.random() < 0.5)
        R_t = float(rng.uniform(-0.1, 1.1) * costs[:, 2].sum())
        a, _ = pask.control_token(a0, amin, prio, crit, R_t, costs)
        assert a == _brute_force_token(a0, amin, prio, crit, R_t, costs), (trial, a0, amin, prio, crit, R_t)


def test_row_actions_broadcast_groups_and_keep_the_recent_window_high():
    # 5 layers in 2 groups (layers 0-2 -> group 0, 3-4 -> group 1 by the
    # ceil(c*L/n_groups) boundaries), 2 KV heads, 6 generated tokens, recent 2
    from oracle.policy import layer_group
    assert [layer_group(l, 5, 2) for l in range(5)] == [0, 0, 0, 1, 1]
    acts = np.array([[[0, 1], [1, 2], [2, 0], [0, 0], [1, 1], [0, 2]]], np.uint8)
    ra = pask.row_actions(acts, 5, 2, 2)
    assert ra.shape == (1, 5, 2, 6)
    np.testing.assert_array_equal(ra[0, 0, 0], [0, 1, 2, 0, 2, 2])
    np.testing.assert_array_equal(ra[0, 4, 1], [1, 2, 0, 0, 2, 2])
    assert (ra[0, :3] == ra[0, 0, 0]).all() and (ra[0, 3:] == ra[0, 4, 1]).all()
    # recent 0 leaves the schedule as it is; a window longer than the stream makes all H
    np.testing.assert_array_equal(pask.row_actions(acts, 5, 2, 0)[0, 3, 0], acts[0, :, 1])
    assert (pask.row_actions(acts, 5, 2, 9) == pask.H_ACT).all()
