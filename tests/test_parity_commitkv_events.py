"""GPU parity of the CommitKV-style commit on event pages (CommitKV §3.1:
every event is cut into contiguous pages of at most G tokens), through the C
ABI: the pages cut on the host (kvc_host_event_pages), page deletion effects
in both windows, lifecycle labels and candidate order, greedy joint
retirement, checkpoint page scores over token spans, the pages kept under the
token budget (kvc_page_select, Eq. 13), their token list (kvc_page_tokens),
the compaction by that list and decode over the compacted pool and through
the original storage.

At the small shape the float64 oracle runs the whole commit on its own page
cut (oracle.page_effect.event_pages) for every page and row. At the full
shape (16 x 28 x 4 rows, 33,312 tokens, 2,905 event pages per trajectory) it
checks sampled outputs one by one and what the planted completion events fix.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from budgeted_retention_amd import synth
from oracle import decode as o_decode, numfmt, page_effect as o_pe, score as o_score
import kvc_testlib as tl

pytestmark = pytest.mark.gpu

EFF_RTOL, EFF_ATOL = 1e-2, 1e-7


def run_commit(w, inp, taus):
    from budgeted_retention_amd import pipelines
    res = pipelines.run_commit(w, inp, taus)
    torch.cuda.synchronize()
    for k in ("Rm", "Rp", "pscore", "kept", "n_kept", "n_h", "lse1", "lse2", "page_first", "page_len", "tokens",
              "n_tokens"):
        res[k] = res[k].cpu().numpy()
    res["retire"] = [(a.cpu().numpy(), j.cpu().numpy()) for a, j in res["retire"]]
    res["o1"], res["o2"] = tl.f64(res["o1"]), tl.f64(res["o2"])
    return res


def _oracle_pages(w, inp, n):
    """The oracle's cut of trajectory n: (first, length) of every page and the
    number lying wholly before the pre-commit window."""
    first, length = o_pe.event_pages(inp.events[n], w.page_size)
    return first, length, int(np.count_nonzero(first + length <= w.q_first_pre))


def _toks(first, length, pages):
    return np.concatenate([np.arange(first[e], first[e] + length[e]) for e in pages])


def _effects(K, V, Q, q_first, W, first, length, pages, mapper):
    q_pos = q_first + np.arange(W)
    return np.array(list(mapper(
        lambda e: o_pe.deletion_effect(K, V, Q, q_pos, np.arange(first[e], first[e] + length[e]))[0], pages)))


def _joint(K, V, Q, q_first, W, first, length, pages):
    return o_pe.deletion_effect(K, V, Q, q_first + np.arange(W), _toks(first, length, pages))[0]


def _layer_f64(inp, n, layer):
    return (tl.f64(inp.K[n, layer]), tl.f64(inp.V[n, layer]), tl.f64(inp.Q_pre[n, layer]),
            tl.f64(inp.Q_post[n, layer]))


def _oracle_scores(inp, n, W, first, length, mapper):
    L, Hkv = inp.K.shape[1], inp.K.shape[2]
    G = inp.Q_post.shape[2] // Hkv

    def row(lh):
        l, h = lh
        return o_score.obs_window_score(tl.f64(inp.K[n, l, h]), tl.f64(inp.Q_post[n, l, h * G:(h + 1) * G]), W)
    rows = np.stack(list(mapper(row, [(l, h) for l in range(L) for h in range(Hkv)])))
    return rows, o_pe.page_scores_spans(rows, first, length)


def _check_kept(res, n, o_kept, o_ps, length, retired, B):
    """Kept pages equal except swaps among pages whose oracle score lies within
    1e-3 relative of the last kept page's; never a retired page; the kept
    token count fits the budget."""
    g = res["kept"][n][: res["n_kept"][n]].astype(np.int64)
    assert np.all(np.diff(g) > 0) and not set(g.tolist()) & set(retired)
    assert res["n_tokens"][n] == length[g].sum() <= B
    diff = np.setxor1d(g, o_kept)
    if diff.size:
        thr = o_ps[o_kept].min()
        assert np.all(np.abs(o_ps[diff] - thr) <= 1e-3 * abs(thr)), (diff, o_ps[diff], thr)
    return diff.size


def _check_rows(res, inp, w, rows_sel, first, length):
    L, Hkv = w.n_layers, w.n_kv_heads
    for r in rows_sel:
        n, l, h = r // (L * Hkv), (r // Hkv) % L, r % Hkv
        pages = res["kept"][n][: res["n_kept"][n]].astype(np.int64)
        toks = o_pe.retained_tokens(first, length, pages)
        assert res["n_h"][r] == toks.size == res["n_tokens"][n]
        np.testing.assert_array_equal(res["tokens"][n][: toks.size], toks)
        tl.check_compaction(tl.bits(res["Ko"][r]), tl.bits(res["Vo"][r]), res["pos"][r].cpu().numpy(),
                            tl.bits(inp.K[n, l, h]), tl.bits(inp.V[n, l, h]), np.arange(w.n_tokens), toks,
                            -1, 1e6)


def _check_decode(res, inp, w, n, heads, toks, exact_set):
    G = w.n_q_heads // w.n_kv_heads
    for l, hq in heads:
        h = hq // G
        K, V = tl.f64(inp.K[n, l, h])[toks], tl.f64(inp.V[n, l, h])[toks]
        o, lse = o_decode.decode_partitions(tl.f64(inp.q_dec[n, l, hq]), [(K, V)])
        for g_o, g_lse in ((res["o1"], res["lse1"]), (res["o2"], res["lse2"])):
            np.testing.assert_allclose(g_o[n, l, hq], numfmt.round_bf16(o), rtol=1e-2, atol=2e-2)
            if exact_set:
                np.testing.assert_allclose(g_o[n, l, hq], o, rtol=8e-3, atol=1e-3)
                assert g_lse[n, l, hq] == pytest.approx(lse, rel=1e-5, abs=1e-5)


def _planted_pages(inp, n, first):
    return np.array([int(np.flatnonzero(first == f)[0]) for f, _ in inp.planted[n]])


def test_commitkv_events_small_end_to_end():
    """Every page and row against the oracle's own run of the commit."""
    w = synth.COMMIT_WORKLOADS["commitkv_events_small"]
    inp = synth.make_commit_inputs(w, "cpu")
    W, B = w.window, w.budget
    oracle = []
    for n in range(w.n_seq):
        first, length, n_el = _oracle_pages(w, inp, n)
        K, V, Qm, Qp = _layer_f64(inp, n, w.layer)
        Rm = _effects(K, V, Qm, w.q_first_pre, W, first, length, range(n_el), map)
        Rp = _effects(K, V, Qp, w.q_first_post, W, first, length, range(n_el), map)
        st = o_pe.lifecycle_states(Rm, Rp, w.tau_use, np.float32(w.tau_dead), w.rho_use, w.rho_dead)
        order = o_pe.candidate_order(Rm, Rp, st)[: w.max_scan]
        oracle.append(dict(first=first, length=length, n_el=n_el, K=K, V=V, Qp=Qp, Rm=Rm, Rp=Rp, st=st,
                           order=order))
        assert set(order.tolist()) == set(_planted_pages(inp, n, first).tolist())
    inp.K, inp.V, inp.Q_pre, inp.Q_post, inp.q_dec = (t.cuda() for t in (inp.K, inp.V, inp.Q_pre, inp.Q_post,
                                                                         inp.q_dec))
    # a bound between the joint effects of the first two and first three candidates of trajectory 0
    o = oracle[0]
    j2 = _joint(o["K"], o["V"], o["Qp"], w.q_first_post, W, o["first"], o["length"], o["order"][:2])
    j3 = _joint(o["K"], o["V"], o["Qp"], w.q_first_post, W, o["first"], o["length"], o["order"][:3])
    assert j3 > 1.05 * j2
    tau = float(np.sqrt(j2 * j3))
    res = run_commit(w, inp, [tau])
    acc, jr = res["retire"][0]
    for n, o in enumerate(oracle):
        P = o["first"].size
        np.testing.assert_array_equal(res["page_first"][n], o["first"])
        np.testing.assert_array_equal(res["page_len"][n], o["length"])
        assert res["n_eligible"] == o["n_el"]
        np.testing.assert_allclose(res["Rm"][n], o["Rm"], rtol=EFF_RTOL, atol=EFF_ATOL)
        np.testing.assert_allclose(res["Rp"][n], o["Rp"], rtol=EFF_RTOL, atol=EFF_ATOL)
        np.testing.assert_array_equal(res["states"][n], o["st"])
        assert res["n_order"][n] == o["order"].size
        np.testing.assert_array_equal(res["order"][n][: o["order"].size], o["order"])
        D = []
        for c, e in enumerate(o["order"].tolist()):
            j = _joint(o["K"], o["V"], o["Qp"], w.q_first_post, W, o["first"], o["length"], D + [e])
            assert jr[n, c] == pytest.approx(j, rel=EFF_RTOL, abs=EFF_ATOL)
            if abs(j - tau) <= 1e-3 * tau:
                break
            assert bool(acc[n, c]) == (j <= tau), (n, c, j, tau)
            if j <= tau:
                D.append(e)
        if n == 0:
            assert 0 < acc[n].sum() < o["order"].size
        retired = [int(res["order"][n][c]) for c in range(w.max_scan) if acc[n, c]]
        rows, o_ps = _oracle_scores(inp, n, W, o["first"], o["length"], map)
        g_rows = res["scores"][n].reshape(-1, w.n_tokens).cpu().numpy()
        for r in range(rows.shape[0]):
            tl.check_scores(g_rows[r], rows[r])
        keep = np.ones(P, bool)
        keep[retired] = False
        tl.check_scores(res["pscore"][n][keep], o_ps[keep])
        assert np.all(np.isneginf(res["pscore"][n][~keep]))
        o_kept, used = o_pe.retained_pages_budget(o_ps, o["length"], retired, B)
        assert B - w.page_size < used <= B
        swaps = _check_kept(res, n, o_kept, o_ps, o["length"], retired, B)
        toks = o_pe.retained_tokens(o["first"], o["length"], o_kept)
        _check_decode(res, inp, w, n, [(l, hq) for l in range(w.n_layers) for hq in range(w.n_q_heads)], toks,
                      swaps == 0)
        _check_rows(res, inp, w, range(n * w.n_layers * w.n_kv_heads, (n + 1) * w.n_layers * w.n_kv_heads),
                    o["first"], o["length"])


def test_commitkv_events_full_size_sampled():
    """16 trajectories x 28 layers x 4 KV heads, 33,312 tokens in event pages of
    at most 16 tokens; a second run is bit-identical."""
    w = synth.COMMIT_WORKLOADS["commitkv_events"]
    inp = synth.make_commit_inputs(w, "cuda")
    W, B = w.window, w.budget
    executor = ThreadPoolExecutor(8)
    pool = executor.map
    first, length, n_el = _oracle_pages(w, inp, 0)
    K, V, Qm, Qp = _layer_f64(inp, 0, w.layer)
    planted0 = _planted_pages(inp, 0, first)
    j_all = _joint(K, V, Qp, w.q_first_post, W, first, length, planted0)
    res = run_commit(w, inp, [w.tau_joint, 0.5 * j_all])
    assert res["n_eligible"] == n_el
    for n in range(w.n_seq):
        f_n, l_n, _ = _oracle_pages(w, inp, n)
        np.testing.assert_array_equal(res["page_first"][n], f_n)
        np.testing.assert_array_equal(res["page_len"][n], l_n)
    # effects at sampled pages: planted ones, one-token pages and others
    rng = np.random.default_rng(2)
    short = np.flatnonzero(length[:n_el] == 1)[:2]
    others = rng.choice(np.setdiff1d(np.arange(n_el), planted0), 3, replace=False)
    sample = np.concatenate([planted0[[0, 31, 63]], short, others])
    np.testing.assert_allclose(res["Rm"][0][sample],
                               _effects(K, V, Qm, w.q_first_pre, W, first, length, sample, pool),
                               rtol=EFF_RTOL, atol=EFF_ATOL)
    np.testing.assert_allclose(res["Rp"][0][sample],
                               _effects(K, V, Qp, w.q_first_post, W, first, length, sample, pool),
                               rtol=EFF_RTOL, atol=EFF_ATOL)
    # every trajectory: the completion candidates are exactly the planted event pages, each
    # effect further from its threshold than twice the effect tolerance
    lo, hi = 1 - 2 * EFF_RTOL, 1 + 2 * EFF_RTOL
    for n in range(w.n_seq):
        pl = _planted_pages(inp, n, res["page_first"][n])
        assert res["Rm"][n][pl].min() > hi * w.tau_use and res["Rp"][n][pl].max() < lo * w.tau_dead
        o_st = o_pe.lifecycle_states(res["Rm"][n].astype(np.float64), res["Rp"][n].astype(np.float64),
                                     w.tau_use, np.float32(w.tau_dead), w.rho_use, w.rho_dead)
        np.testing.assert_array_equal(res["states"][n], o_st)
        o_order = o_pe.candidate_order(res["Rm"][n].astype(np.float64), res["Rp"][n].astype(np.float64), o_st)
        assert set(o_order.tolist()) == set(pl.tolist()) and res["n_order"][n] == w.n_planted
        np.testing.assert_array_equal(res["order"][n], o_order[: w.max_scan])
    acc, jr = res["retire"][0]
    assert acc.all()
    assert jr[0, -1] == pytest.approx(j_all, rel=EFF_RTOL, abs=EFF_ATOL)
    order0 = res["order"][0].tolist()
    acc2, jr2 = res["retire"][1]
    tau2 = 0.5 * j_all
    first_rej = int(np.flatnonzero(acc2[0] == 0)[0])
    for c in sorted({0, 1, first_rej, first_rej + 1, w.max_scan - 1}):
        D = [order0[i] for i in range(c) if acc2[0, i]]
        j = _joint(K, V, Qp, w.q_first_post, W, first, length, D + [order0[c]])
        assert jr2[0, c] == pytest.approx(j, rel=EFF_RTOL, abs=EFF_ATOL), c
        if abs(j - tau2) > 1e-3 * tau2:
            assert bool(acc2[0, c]) == (j <= tau2), (c, j, tau2)
    # checkpoint of trajectory 0: every row's window score, the span page scores and the pages
    # kept under the token budget
    rows, o_ps = _oracle_scores(inp, 0, W, first, length, pool)
    g_rows = res["scores"][0].reshape(-1, w.n_tokens).cpu().numpy()
    for r in range(rows.shape[0]):
        tl.check_scores(g_rows[r], rows[r])
    keep = np.ones(first.size, bool)
    keep[planted0] = False
    tl.check_scores(res["pscore"][0][keep], o_ps[keep])
    assert np.all(np.isneginf(res["pscore"][0][planted0]))
    o_kept, used = o_pe.retained_pages_budget(o_ps, length, planted0, B)
    assert B - w.page_size < used <= B
    swaps = _check_kept(res, 0, o_kept, o_ps, length, planted0, B)
    assert swaps <= 2
    for n in range(1, w.n_seq):
        g = res["kept"][n][: res["n_kept"][n]]
        assert np.all(np.diff(g) > 0) and 0 < res["n_tokens"][n] <= B
        assert not set(g.tolist()) & set(_planted_pages(inp, n, res["page_first"][n]).tolist())
    L, Hkv = w.n_layers, w.n_kv_heads
    _check_rows(res, inp, w, [0, (0 * L + 27) * Hkv + 3, (0 * L + 13) * Hkv + 1], first, length)
    f15, l15, _ = _oracle_pages(w, inp, 15)
    _check_rows(res, inp, w, [(15 * L + 20) * Hkv + 2, w.rows - 1], f15, l15)
    _check_decode(res, inp, w, 0, [(0, 0), (13, 9), (27, 27), (27, 6)], o_pe.retained_tokens(first, length, o_kept),
                  swaps == 0)
    np.testing.assert_allclose(res["o1"], res["o2"], rtol=8e-3, atol=1e-3)
    executor.shutdown()
    tl.assert_same_bits(res, run_commit(w, inp, [w.tau_joint, 0.5 * j_all]))
