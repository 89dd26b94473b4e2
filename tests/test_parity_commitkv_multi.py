"""GPU parity of successive CommitKV commits with pending-page protection
(CommitKV §3.2-3.4: Eq. 7-11 per commit, Eq. 12 protection of pages awaiting
their post-commit measurement, Eq. 13 retained set, Eq. 4 one index set),
through the C ABI and the host routines.

At the small shape the float64 oracle runs every commit of every trajectory
on its own state: pre- and post-commit effects (1e-2 relative, the page
effect bar), protected pages, page scores, retained pages (swaps only within
1e-3 relative of the last kept score), lifecycle order and greedy retirement
(a decision within 1e-3 of tau_joint may go either way). A trajectory whose
GPU and oracle decisions part by such an allowed difference has different
caches from then on; its later commits are not compared (the test counts
them). At the full shape (16 x 28 x 4 rows, 5,664 tokens per commit) sampled
effects are checked one by one, and every commit against the properties that
hold at any size.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from budgeted_retention_amd import synth
from oracle import numfmt, page_effect as o_pe, score as o_score
import kvc_testlib as tl

pytestmark = pytest.mark.gpu

EFF_RTOL, EFF_ATOL = 1e-2, 1e-7


def _run(w, inp):
    from budgeted_retention_amd import pipelines
    res = pipelines.run_commit_multi(w, inp, record=True)
    torch.cuda.synchronize()
    return res


def _effects(K, V, Q, q_first, W, pages, ps, mapper):
    q_pos = q_first + np.arange(W)
    return np.array(list(mapper(
        lambda e: o_pe.deletion_effect(K, V, Q, q_pos, o_pe.page_tokens(e * ps, ps))[0], pages)))


def _joint(K, V, Q, q_first, W, pages, ps):
    toks = np.concatenate([o_pe.page_tokens(e * ps, ps) for e in pages])
    return o_pe.deletion_effect(K, V, Q, q_first + np.arange(W), toks)[0]


def _oracle_trajectory(w, inp, n, rec, mapper):
    """The oracle's commits of trajectory n, compared commit by commit with
    the GPU's record. Returns the number of commits compared in full."""
    L, Hkv, d, W, ps, B = w.n_layers, w.n_kv_heads, w.head_dim, w.window, w.page_size, w.budget
    G = w.n_q_heads // Hkv
    Ta, Tb = w.t_pre, w.t_post
    n_el, Pa, n_keep = (Ta - W) // ps, Ta // ps, B // ps
    first_turn = Tb // ps
    Kb, Vb = tl.bits(inp.K0[n]), tl.bits(inp.V0[n])                # [L][Hkv][Tb][d]
    pos = np.arange(Tb)
    next_pos = Tb
    retired = []
    for c in range(w.commits):
        g = rec[c]
        Ka = np.concatenate([Kb, tl.bits(inp.K_call[c, n])], axis=2)
        Va = np.concatenate([Vb, tl.bits(inp.V_call[c, n])], axis=2)
        pa = np.concatenate([pos, np.arange(next_pos, next_pos + w.n_call)])
        next_pos += w.n_call
        Kl, Vl = numfmt.bf16_bits_to_f64(Ka[w.layer]), numfmt.bf16_bits_to_f64(Va[w.layer])
        Qm = tl.f64(inp.Q_pre[c, n, w.layer])
        Rm = _effects(Kl, Vl, Qm, Ta - W, W, range(n_el), ps, mapper)
        np.testing.assert_allclose(g["Rm"][n], Rm, rtol=EFF_RTOL, atol=EFF_ATOL)
        pend = np.arange(first_turn, n_el)
        prot = pend[o_pe.protect_pending(Rm[pend], np.full(pend.size, ps), B, w.eta, w.max_protect)]
        if not np.array_equal(np.flatnonzero(g["tags"][n]), prot):
            return c
        rows = np.stack([o_score.obs_window_score(numfmt.bf16_bits_to_f64(Ka[l, h]),
                                                  tl.f64(inp.Q_pre[c, n, l, h * G:(h + 1) * G]), W)
                         for l in range(L) for h in range(Hkv)])
        ps_o = o_pe.page_scores(rows, ps, Pa)
        live = np.setdiff1d(np.arange(Pa), retired)
        np.testing.assert_allclose(g["pscore"][n][live], ps_o[live], rtol=1e-4)
        assert np.all(np.isneginf(g["pscore"][n][retired]))
        kept = o_pe.retained_pages(ps_o, retired, n_keep, protected=prot)
        gk = g["kept"][n][: g["n_kept"][n]].astype(np.int64)
        assert g["n_kept"][n] == n_keep and set(prot) <= set(gk) and not set(retired) & set(gk)
        if not np.array_equal(gk, kept):
            thr = ps_o[kept].min()
            diff = np.setxor1d(gk, kept)
            assert np.all(np.abs(ps_o[diff] - thr) <= 1e-3 * abs(thr)), (diff, ps_o[diff], thr)
            return c
        toks = (kept[:, None] * ps + np.arange(ps)[None, :]).reshape(-1)
        Kb = np.concatenate([Ka[:, :, toks], tl.bits(inp.K_obs[c, n])], axis=2)
        Vb = np.concatenate([Va[:, :, toks], tl.bits(inp.V_obs[c, n])], axis=2)
        pos = np.concatenate([pa[toks], np.arange(next_pos, next_pos + w.n_obs + W)])
        next_pos += w.n_obs + W
        np.testing.assert_array_equal(g["pos"][n].reshape(-1, Tb), np.tile(pos, (L * Hkv, 1)))
        ev = np.flatnonzero(kept < n_el)
        Kl, Vl = numfmt.bf16_bits_to_f64(Kb[w.layer]), numfmt.bf16_bits_to_f64(Vb[w.layer])
        Qp = tl.f64(inp.Q_post[c, n, w.layer])
        Rp = _effects(Kl, Vl, Qp, Tb - W, W, ev, ps, mapper)
        np.testing.assert_allclose(g["Rp"][n][ev], Rp, rtol=EFF_RTOL, atol=EFF_ATOL)
        st = o_pe.lifecycle_states(Rm[kept[ev]], Rp, w.tau_use, w.tau_dead, w.rho_use, w.rho_dead)
        order = ev[o_pe.candidate_order(Rm[kept[ev]], Rp, st)][: w.max_scan]
        if not np.array_equal(g["order"][n][: g["n_order"][n]], order):
            return c
        D = o_pe.greedy_retire(order, lambda pages: _joint(Kl, Vl, Qp, Tb - W, W, pages, ps), w.tau_joint,
                               w.max_scan)
        g_D = g["order"][n][: g["n_order"][n]][g["accepted"][n][: g["n_order"][n]] == 1]
        if sorted(g_D.tolist()) != sorted(D):
            for E in np.setxor1d(g_D, D):      # only decisions at the bound may differ
                prev = [x for x in order[: list(order).index(E)] if x in D]
                assert abs(_joint(Kl, Vl, Qp, Tb - W, W, prev + [int(E)], ps) - w.tau_joint) <= 1e-3 * w.tau_joint
            return c
        retired = sorted(D)
    return w.commits


def test_commitkv_multi_small_every_trajectory():
    w = synth.COMMIT_MULTI_WORKLOADS["commitkv_multi_small"]
    inp = synth.make_commit_multi_inputs(w, "cuda")
    res = _run(w, inp)
    rec = res["commits"]
    with ThreadPoolExecutor(8) as ex:
        done = [_oracle_trajectory(w, inp, n, rec, ex.map) for n in range(w.n_seq)]
    assert sum(d == w.commits for d in done) >= w.n_seq - 1, done
    # the lifecycle ran: pending pages were protected and completion pages retired
    assert all(r["tags"].sum() > 0 for r in rec)
    assert sum(int(r["accepted"].sum()) for r in rec) > 0


def test_commitkv_multi_full_size_properties_and_sampled_effects():
    """16 trajectories x 28 layers x 4 KV heads, four commits of 1,024-token
    turns with 512-token observations, B = 4,096, eta = 0.125."""
    w = synth.COMMIT_MULTI_WORKLOADS["commitkv_multi"]
    inp = synth.make_commit_multi_inputs(w, "cuda")
    res = _run(w, inp)
    rec = res["commits"]
    ps, W, B = w.page_size, w.window, w.budget
    n_el, n_keep, first_turn = (w.t_pre - W) // ps, B // ps, w.t_post // ps
    B_N = int(np.floor(w.eta * B))
    prev_retired = [np.zeros(0, np.int64)] * w.n_seq
    planted_hits = 0
    for c, g in enumerate(rec):
        for n in range(w.n_seq):
            prot = np.flatnonzero(g["tags"][n])
            assert prot.size <= w.max_protect and prot.size * ps <= B_N
            assert np.all((prot >= first_turn) & (prot < n_el))
            kept = g["kept"][n][: g["n_kept"][n]]
            assert g["n_kept"][n] == n_keep and np.all(np.diff(kept) > 0)
            assert set(prot) <= set(kept.tolist())
            assert not set(prev_retired[n].tolist()) & set(kept.tolist())
            # protection takes the largest pre-commit effects among the turn's pages
            pend = np.arange(first_turn, n_el)
            rest = np.setdiff1d(pend, prot)
            if prot.size and rest.size:
                assert g["Rm"][n][prot].min() >= g["Rm"][n][rest].max()
            # the turn's planted completion pages are protected, then retired
            planted = first_turn + inp.planted[c, n]
            assert set(planted.tolist()) <= set(prot.tolist())
            no = g["n_order"][n]
            D = g["order"][n][:no][g["accepted"][n][:no] == 1]
            retired_src = kept[D]                              # retired pages in the commit's numbering
            planted_hits += len(set(retired_src.tolist()) & set(planted.tolist()))
            prev_retired[n] = D.astype(np.int64)
            # positions stay absolute and ascending in every row
            pos = g["pos"][n][0, 0]
            assert np.all(np.diff(pos) > 0)
    assert planted_hits >= 0.75 * w.commits * w.n_seq * w.n_plant
    # sampled effects of trajectory 3 at the first commit, one by one
    n, c = 3, 0
    Ka = torch.cat([inp.K0[n], inp.K_call[c, n]], dim=2)
    Va = torch.cat([inp.V0[n], inp.V_call[c, n]], dim=2)
    Kl, Vl = tl.f64(Ka[w.layer]), tl.f64(Va[w.layer])
    Qm = tl.f64(inp.Q_pre[c, n, w.layer])
    pages = [0, first_turn + int(inp.planted[c, n, 0]), n_el - 1]
    Rm = _effects(Kl, Vl, Qm, w.t_pre - W, W, pages, ps, map)
    np.testing.assert_allclose(rec[c]["Rm"][n][pages], Rm, rtol=EFF_RTOL, atol=EFF_ATOL)
