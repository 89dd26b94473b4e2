"""Host-side serial control in libkvc (PASK controller, CommitKV candidate
order) against the oracle. Plain host code: runs without a GPU."""
import numpy as np
import pytest

from budgeted_retention_amd import kvc
from oracle import page_effect as o_pe
from oracle import pask as o_pask


def test_pask_costs_match_oracle():
    got = kvc.kvc_host_pask_costs([8, 8, 8, 8], 8, 128, 8)
    np.testing.assert_array_equal(got, o_pask.group_costs([8, 8, 8, 8], 8, 128))
    got4 = kvc.kvc_host_pask_costs([12, 12, 12], 8, 128, 4)
    np.testing.assert_array_equal(got4, o_pask.group_costs([12, 12, 12], 8, 128, low_bits=4))


@pytest.mark.parametrize("seed,B_D", [(1, 1 / 3), (2, 0.5), (3, 0.1), (4, 1.0)])
def test_pask_control_matches_oracle(seed, B_D):
    rng = np.random.default_rng(seed)
    n_tags, C, n_seq, n_tok = 8, 4, 3, 700
    a0 = rng.integers(0, 3, (n_tags, C)).astype(np.uint8)
    amin = np.minimum(a0, rng.integers(0, 3, (n_tags, C))).astype(np.uint8)
    prio = rng.random((n_tags, C, 2)).astype(np.float32)
    crit = (rng.random(n_tags) < 0.3).astype(np.uint8)
    costs = o_pask.group_costs([8, 8, 8, 8], 8, 128)
    tags = rng.integers(0, n_tags, (n_seq, n_tok)).astype(np.uint8)
    acts, ledger = kvc.kvc_host_pask_control(a0, amin, prio, crit, costs, B_D, tags)
    for n in range(n_seq):
        o_acts, o_ledger = o_pask.control_sequence(tags[n], a0.astype(np.int64), amin.astype(np.int64),
                                                   prio.astype(np.float64), crit, costs, B_D)
        np.testing.assert_array_equal(acts[n], o_acts)
        np.testing.assert_allclose(ledger[n], o_ledger, rtol=1e-12, atol=1e-6)


@pytest.mark.parametrize("n_layers,n_groups,recent", [(32, 4, 16), (5, 2, 0), (7, 3, 40), (3, 3, 1)])
def test_pask_row_actions_match_oracle(n_layers, n_groups, recent):
    rng = np.random.default_rng(n_layers * 10 + recent)
    n_seq, n_tok, Hkv = 2, 37, 3
    acts = rng.integers(0, 3, (n_seq, n_tok, n_groups)).astype(np.uint8)
    got = kvc.kvc_host_pask_row_actions(acts, n_layers, Hkv, recent)
    np.testing.assert_array_equal(got, o_pask.row_actions(acts, n_layers, Hkv, recent))


def test_commit_candidates_match_oracle():
    rng = np.random.default_rng(5)
    n = 500
    Rm = (10.0 ** rng.uniform(-5, 0, n)).astype(np.float32)
    Rp = (10.0 ** rng.uniform(-5, 0, n)).astype(np.float32)
    Rp[:40] = Rp[0]                       # ties in R+ exercise the secondary key
    c = dict(tau_use=0.05, tau_dead=1e-3, rho_use=0.75, rho_dead=0.25)
    state, order, n_order = kvc.kvc_host_commit_candidates(Rm, Rp, max_scan=64, **c)
    o_state = o_pe.lifecycle_states(Rm.astype(np.float64), Rp.astype(np.float64), c["tau_use"],
                                    np.float32(c["tau_dead"]), c["rho_use"], c["rho_dead"])
    np.testing.assert_array_equal(state, o_state)
    o_order = o_pe.candidate_order(Rm.astype(np.float64), Rp.astype(np.float64), o_state)[:64]
    assert n_order == o_order.size
    np.testing.assert_array_equal(order[:n_order], o_order)
    assert np.all(order[n_order:] == -1)


@pytest.mark.parametrize("G,start,max_ev", [(16, 0, 40), (1, 7, 5), (64, 100, 300), (9, 0, 9)])
def test_event_pages_match_oracle(G, start, max_ev):
    rng = np.random.default_rng(G * 1000 + max_ev)
    ev = rng.integers(1, max_ev + 1, 400)
    first, length = kvc.kvc_host_event_pages(ev, G, start)
    o_first, o_len = o_pe.event_pages(ev, G, start)
    np.testing.assert_array_equal(first, o_first)
    np.testing.assert_array_equal(length, o_len)


def test_event_pages_beyond_the_cap_report_the_count_and_write_only_cap():
    import ctypes
    from budgeted_retention_amd import _lib
    ev = np.array([5, 3, 9], np.int32)                  # pages of 4: [4, 1], [3], [4, 4, 1]
    first = np.full(4, -7, np.int32)
    length = np.full(4, -7, np.int32)
    n = ctypes.c_int32(0)
    st = _lib.load().kvc_host_event_pages(ev.ctypes.data, 3, 4, 0, first.ctypes.data, length.ctypes.data, 2,
                                          ctypes.byref(n))
    assert st != 0 and n.value == 6
    assert list(first) == [0, 4, -7, -7] and list(length) == [4, 1, -7, -7]


def test_host_helpers_reject_bad_arguments():
    from budgeted_retention_amd import _lib
    with pytest.raises(_lib.KvcError):
        kvc.kvc_host_pask_costs([8, -1], 8, 128)
    with pytest.raises(_lib.KvcError):
        tags = np.full((1, 4), 9, np.uint8)        # tag outside the 8-row table
        z = np.zeros((8, 2), np.uint8)
        kvc.kvc_host_pask_control(z, z, np.zeros((8, 2, 2), np.float32), np.zeros(8, np.uint8),
                                  np.zeros((2, 3)), 0.5, tags)
    with pytest.raises(_lib.KvcError):
        kvc.kvc_host_pask_row_actions(np.zeros((1, 4, 2), np.uint8), 0, 8, 2)   # no layers
    with pytest.raises(_lib.KvcError):
        kvc.kvc_host_pask_row_actions(np.zeros((1, 4, 2), np.uint8), 4, 8, -1)  # negative window
    with pytest.raises(_lib.KvcError):
        kvc.kvc_host_event_pages([3, 0, 2], 4)                                   # an empty event
    with pytest.raises(_lib.KvcError):
        kvc.kvc_host_event_pages([3, 2], 0)                                      # G = 0
    with pytest.raises(_lib.KvcError):
        kvc.kvc_host_event_pages([2 ** 30, 2 ** 30], 64, 2 ** 30)                 # tokens past 2^31 - 1


def test_commit_protection_matches_oracle_and_the_page_budget():
    from oracle import page_effect as o_pe
    rng = np.random.default_rng(3)
    for trial in range(50):
        n = int(rng.integers(0, 40))
        Rm = rng.gamma(0.5, 0.05, n).astype(np.float32)
        if n > 4:
            Rm[1] = Rm[3]                                   # a tie: the lower index first
        tok = np.where(rng.random(n) < 0.8, 16, rng.integers(1, 64, n)).astype(np.int32)
        B = int(rng.integers(256, 8192))
        eta = float(rng.choice([0.0, 0.0625, 0.125, 0.5, 1.0]))
        got, k = kvc.kvc_host_commit_protect(Rm, tok, B, eta, 16)
        want = o_pe.protect_pending(Rm.astype(np.float64), tok, B, eta, 16)
        np.testing.assert_array_equal(np.flatnonzero(got), want)
        assert k == want.size <= 16 and tok[want].sum() <= int(np.floor(eta * B))


def test_pace_renumber_matches_oracle_and_keeps_positions_below_the_limit():
    from oracle import positions
    rng = np.random.default_rng(8)
    for _ in range(200):
        L = int(rng.choice([4096, 8192, 16384]))
        H = int(rng.integers(0, 4097))
        bmax = int(rng.integers(1, max(2, L - H)))
        if not positions.admissible(L, bmax, H):
            with pytest.raises(RuntimeError):
                kvc.kvc_host_pace_renumber(10, 0, 1, L, H, bmax)
            continue
        res = int(rng.integers(0, bmax + 1))
        shift = int(rng.integers(0, 10 ** 6))
        m = shift + int(rng.integers(res, L + 1))
        assert kvc.kvc_host_pace_renumber(m, shift, res, L, H, bmax) == positions.after_eviction(m, shift, res, L, H)
    # a session driven by the native rule never writes a position >= L
    shift, m, top = 0, 0, -1
    while m < 300_000:
        top = max(top, m + 2000 - 1 - shift)
        m += 2000
        ren, shift = kvc.kvc_host_pace_renumber(m, shift, 2048, 8192, 4096, 2048 + 64)
    assert top < 8192
