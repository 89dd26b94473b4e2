"""GPU parity of the page calls on event pages (CommitKV §3.1: every event is
cut into contiguous pages of at most G tokens, so page lengths vary), through
the C ABI, against the float64 oracle: deletion effects recomputed from
scratch (oracle.page_effect.deletion_effect on each page's token set), the
greedy joint retirement, checkpoint page scores over token spans, and the
retained token set that the compaction then gathers."""
import numpy as np
import pytest
import torch

from budgeted_retention_amd import synth
from oracle import page_effect as o_pe
import kvc_testlib as tl

pytestmark = pytest.mark.gpu


def _event_pages(rng, N, T, G, max_event=40):
    """Per sequence: events of 1..max_event tokens from token 0, cut into pages
    of at most G tokens; the first n_pages pages of every sequence (the
    shortest count) as int32 [N][n_pages] first / length."""
    firsts, lens = [], []
    for _ in range(N):
        ev = rng.integers(1, max_event + 1, T)
        ev = ev[: np.searchsorted(np.cumsum(ev), T, side="right")]
        f, ln = o_pe.event_pages(ev, G)
        firsts.append(f)
        lens.append(ln)
    n_pages = min(f.size for f in firsts)
    first = np.stack([f[:n_pages] for f in firsts]).astype(np.int32)
    length = np.stack([ln[:n_pages] for ln in lens]).astype(np.int32)
    return first, length, n_pages


@pytest.mark.parametrize("N,L,layer,Hkv,Hq,d,T,W,q_first,G,shuffle", [
    (2, 2, 1, 2, 6, 128, 700, 8, 600, 16, False),   # window inside the cache, keys after it unseen
    (1, 1, 0, 1, 4, 64, 333, 5, 328, 64, False),    # pages up to the 64-key tile, d = 64
    (2, 1, 0, 2, 8, 128, 520, 16, 504, 9, True),    # a page length that divides nothing; pages out of order
])
def test_event_page_effect_matches_recomputation(N, L, layer, Hkv, Hq, d, T, W, q_first, G, shuffle):
    from budgeted_retention_amd import kvc
    rng = np.random.default_rng(T + G)
    K, V, Q = synth.small_case(T, Hkv, Hq, d, W, L, N, seed=T + d)
    first, length, n_pages = _event_pages(rng, N, T, G)
    if shuffle:
        perm = rng.permutation(n_pages)
        first, length = first[:, perm].copy(), length[:, perm].copy()
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    ws = kvc.page_workspace(dims, W, q_first)
    rel = torch.empty((N, n_pages), dtype=torch.float32, device="cuda")
    ab = torch.empty_like(rel)
    kvc.kvc_page_effect(dims, layer, K.cuda(), V.cuda(), Q.cuda(), W, q_first, G, n_pages, rel, ws, ab,
                        page_first=torch.from_numpy(first).cuda(), page_len=torch.from_numpy(length).cuda())
    torch.cuda.synchronize()
    rel, ab = rel.cpu().numpy(), ab.cpu().numpy()
    Kf, Vf, Qf = tl.f64(K), tl.f64(V), tl.f64(Q)
    q_pos = q_first + np.arange(W)
    for n in range(N):
        for e in range(n_pages):
            toks = np.arange(first[n, e], first[n, e] + length[n, e])
            r_o, a_o = o_pe.deletion_effect(Kf[n, layer], Vf[n, layer], Qf[n, layer], q_pos, toks)
            assert rel[n, e] == pytest.approx(r_o, rel=1e-2, abs=1e-5), (n, e, first[n, e], length[n, e])
            assert ab[n, e] == pytest.approx(a_o, rel=1e-2, abs=1e-5), (n, e)


def test_event_pages_equal_to_uniform_pages_give_the_same_bits():
    """Event pages that happen to be uniform reproduce the uniform-page call."""
    from budgeted_retention_amd import kvc
    N, L, Hkv, Hq, d, T, W, ps, n_pages = 2, 1, 2, 8, 128, 600, 8, 16, 36
    K, V, Q = synth.small_case(T, Hkv, Hq, d, W, L, N, seed=5)
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    ws = kvc.page_workspace(dims, W, T - W)
    first = torch.from_numpy(np.tile(np.arange(n_pages, dtype=np.int32) * ps, (N, 1))).cuda()
    length = torch.full((N, n_pages), ps, dtype=torch.int32, device="cuda")
    a = torch.empty((N, n_pages), dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    kvc.kvc_page_effect(dims, 0, K.cuda(), V.cuda(), Q.cuda(), W, T - W, ps, n_pages, a, ws)
    kvc.kvc_page_effect(dims, 0, K.cuda(), V.cuda(), Q.cuda(), W, T - W, ps, n_pages, b, ws,
                        page_first=first, page_len=length)
    torch.cuda.synchronize()
    np.testing.assert_allclose(b.cpu().numpy(), a.cpu().numpy(), rtol=2e-6, atol=1e-7)


def test_event_page_retire_greedy_matches_oracle():
    from budgeted_retention_amd import kvc
    N, L, layer, Hkv, Hq, d, T, W, G = 2, 2, 0, 2, 6, 128, 520, 8, 16
    q_first = T - W
    rng = np.random.default_rng(99)
    K, V, Q = synth.small_case(T, Hkv, Hq, d, W, L, N, seed=99)
    first, length, n_pages = _event_pages(rng, N, T, G, max_event=24)
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    Kf, Vf, Qf = tl.f64(K), tl.f64(V), tl.f64(Q)
    q_pos = q_first + np.arange(W)
    toks_of = lambda n, e: np.arange(first[n, e], first[n, e] + length[n, e])
    orders, taus = [], []
    for n in range(N):
        single = np.array([o_pe.deletion_effect(Kf[n, layer], Vf[n, layer], Qf[n, layer], q_pos,
                                                toks_of(n, e))[0] for e in range(n_pages)])
        orders.append(np.argsort(single)[:12])
        taus.append(float(np.sort(single)[5] * 2.0))
    order = torch.from_numpy(np.stack(orders).astype(np.int32))
    order[1, 3] = -1
    tau = taus[0]
    ws = kvc.page_workspace(dims, W, q_first)
    acc = torch.zeros((N, 12), dtype=torch.uint8, device="cuda")
    jr = torch.zeros((N, 12), dtype=torch.float32, device="cuda")
    kvc.kvc_page_retire(dims, layer, K.cuda(), V.cuda(), Q.cuda(), W, q_first, G, n_pages, order.cuda(), tau,
                        acc, ws, jr, page_first=torch.from_numpy(first).cuda(),
                        page_len=torch.from_numpy(length).cuda())
    torch.cuda.synchronize()
    acc, jr = acc.cpu().numpy(), jr.cpu().numpy()
    for n in range(N):
        D = []
        for c, e in enumerate(order[n].tolist()):
            if e < 0:
                assert acc[n, c] == 0 and jr[n, c] == -1
                continue
            toks = np.concatenate([toks_of(n, x) for x in D + [e]])
            j, _ = o_pe.deletion_effect(Kf[n, layer], Vf[n, layer], Qf[n, layer], q_pos, toks)
            assert jr[n, c] == pytest.approx(j, rel=1e-2, abs=1e-6)
            if abs(j - tau) <= 1e-3 * tau:
                break                     # a decision this close to the bound may go either way
            assert bool(acc[n, c]) == (j <= tau), (n, c, j, tau)
            if j <= tau:
                D.append(e)
        assert acc[n].sum() >= 1


@pytest.mark.parametrize("G,shuffle", [(16, False), (64, False), (16, True), (1000, False)])
def test_event_page_scores_pool_rows_and_exclude_retired(G, shuffle):
    """Staged runs (pages in order within 1024 tokens) and per-page sums
    (shuffled pages, or pages of up to 1000 tokens) give the oracle's sums."""
    from budgeted_retention_amd import kvc
    rng = np.random.default_rng(G + shuffle)
    N, L, Hkv, T = 3, 2, 2, 4000
    scores = rng.gamma(0.5, 1.0, (N, L, Hkv, T)).astype(np.float32)
    first, length, n_pages = _event_pages(rng, N, T, G, max_event=3 * G)
    if shuffle:
        perm = rng.permutation(n_pages)
        first, length = first[:, perm].copy(), length[:, perm].copy()
    n_cand = min(6, n_pages)
    order = np.stack([rng.choice(n_pages, n_cand, replace=False) for _ in range(N)]).astype(np.int32)
    order[0, 1] = -1
    acc = np.ones((N, n_cand), np.uint8)
    acc[:, -1] = 0
    dims = kvc.make_dims(N, L, Hkv, 8, 64, T)
    pf, pl = torch.from_numpy(first).cuda(), torch.from_numpy(length).cuda()
    out = torch.empty((N, n_pages), dtype=torch.float32, device="cuda")
    plain = torch.empty_like(out)
    sc = torch.from_numpy(scores).cuda()
    kvc.kvc_page_scores(dims, sc, G, n_pages, out, torch.from_numpy(order).cuda(), torch.from_numpy(acc).cuda(),
                        page_first=pf, page_len=pl)
    kvc.kvc_page_scores(dims, sc, G, n_pages, plain, page_first=pf, page_len=pl)
    torch.cuda.synchronize()
    out, plain = out.cpu().numpy(), plain.cpu().numpy()
    for n in range(N):
        ref = o_pe.page_scores_spans(scores[n].reshape(L * Hkv, T).astype(np.float64), first[n], length[n])
        np.testing.assert_allclose(plain[n], ref, rtol=1e-5, atol=1e-5)
        retired = {int(e) for e, a in zip(order[n], acc[n]) if a and 0 <= e < n_pages}
        mask = np.zeros(n_pages, bool)
        mask[list(retired)] = True
        assert np.all(np.isneginf(out[n][mask]))
        np.testing.assert_array_equal(out[n][~mask], plain[n][~mask])


def test_event_pages_select_expand_and_compact():
    """The checkpoint on event pages: page scores -> kvc_select over pages ->
    kvc_page_tokens (the retained token set) -> kvc_compact_rerotate with one
    token per list entry. Token lists are exact; K, V and positions are the
    gathered rows bit for bit."""
    from budgeted_retention_amd import kvc
    rng = np.random.default_rng(12)
    N, L, Hkv, d, T, G, Bp = 2, 2, 2, 128, 3000, 16, 64
    rows = N * L * Hkv
    K, V, _ = synth.small_case(T, Hkv, 2 * Hkv, d, 4, L, N, seed=12)
    first, length, n_pages = _event_pages(rng, N, T, G)
    scores = rng.gamma(0.5, 1.0, (N, L, Hkv, T)).astype(np.float32)
    dims = kvc.make_dims(N, L, Hkv, 2 * Hkv, d, T)
    pf, pl = torch.from_numpy(first).cuda(), torch.from_numpy(length).cuda()
    pscore = torch.empty((N, n_pages), dtype=torch.float32, device="cuda")
    kvc.kvc_page_scores(dims, torch.from_numpy(scores).cuda(), G, n_pages, pscore, page_first=pf, page_len=pl)
    pol = kvc.Policy(0, 0, Bp, 1, 1, 0, 1, None, torch.zeros((1, 1), dtype=torch.float32, device="cuda"))
    kept = torch.full((N, Bp), -1, dtype=torch.int32, device="cuda")
    nk = torch.zeros(N, dtype=torch.int32, device="cuda")
    kvc.kvc_select(kvc.make_dims(N, 1, 1, 1, 64, n_pages), pscore, pol, kept, Bp, nk)
    cap = Bp * G
    tokens = torch.full((N, cap), -1, dtype=torch.int32, device="cuda")
    n_tok = torch.zeros(N, dtype=torch.int32, device="cuda")
    kvc.kvc_page_tokens(dims, G, n_pages, kept, nk, tokens, n_tok, page_first=pf, page_len=pl)
    pos = np.tile((np.arange(T, dtype=np.int32) * 3 + 1), (rows, 1))
    Ko = torch.zeros((rows, cap, d), dtype=torch.bfloat16, device="cuda")
    Vo = torch.zeros_like(Ko)
    po = torch.full((rows, cap), -1, dtype=torch.int32, device="cuda")
    nh = torch.zeros(rows, dtype=torch.int32, device="cuda")
    kvc.kvc_compact_rerotate(dims, K.cuda(), V.cuda(), torch.from_numpy(pos).cuda(), tokens, cap, n_tok, -1, 1e6,
                             kvc.CompactOut(cap, Ko, Vo, po, nh, kept_page=1))
    torch.cuda.synchronize()
    ps_h = pscore.cpu().numpy()
    Kb, Vb = tl.bits(K).reshape(rows, T, d), tl.bits(V).reshape(rows, T, d)
    gK, gV, gpos = tl.bits(Ko), tl.bits(Vo), po.cpu().numpy()
    for n in range(N):
        ref_ps = o_pe.page_scores_spans(scores[n].reshape(L * Hkv, T).astype(np.float64), first[n], length[n])
        np.testing.assert_allclose(ps_h[n], ref_ps, rtol=1e-5, atol=1e-5)
        # the kept pages are the best Bp by the fp32 page scores the kernel formed
        kp = kept[n].cpu().numpy()[: int(nk[n])]
        np.testing.assert_array_equal(kp, o_pe.retained_pages(ps_h[n].astype(np.float64), (), Bp))
        want = o_pe.retained_tokens(first[n], length[n], kp)
        assert int(n_tok[n]) == want.size
        np.testing.assert_array_equal(tokens[n].cpu().numpy()[: want.size], want.astype(np.int32))
        for r in range(n * L * Hkv, (n + 1) * L * Hkv):
            assert nh[r].item() == want.size
            np.testing.assert_array_equal(gK[r][: want.size], Kb[r][want])
            np.testing.assert_array_equal(gV[r][: want.size], Vb[r][want])
            np.testing.assert_array_equal(gpos[r][: want.size], pos[r][want])


def test_page_tokens_skips_bad_entries_and_truncates():
    from budgeted_retention_amd import kvc
    N, T, G = 2, 100, 8
    first = np.array([[0, 5, 13, 20, 28], [50, 58, 66, 74, 90]], np.int32)
    length = np.array([[5, 8, 7, 8, 3], [8, 8, 8, 8, 20]], np.int32)   # the last page is clamped to G
    pages = np.array([[4, -1, 1, 9, 0], [0, 4, 2, 3, 1]], np.int32)
    n_listed = np.array([5, 3], np.int32)
    dims = kvc.make_dims(N, 1, 1, 1, 64, T)
    tokens = torch.full((N, 12), -7, dtype=torch.int32, device="cuda")
    n_tok = torch.zeros(N, dtype=torch.int32, device="cuda")
    kvc.kvc_page_tokens(dims, G, 5, torch.from_numpy(pages).cuda(), torch.from_numpy(n_listed).cuda(), tokens,
                        n_tok, page_first=torch.from_numpy(first).cuda(), page_len=torch.from_numpy(length).cuda())
    torch.cuda.synchronize()
    clamp = np.minimum(length, G)
    for n in range(N):
        listed = [e for e in pages[n][: n_listed[n]] if 0 <= e < 5]
        want = o_pe.retained_tokens(first[n], clamp[n], listed)
        assert int(n_tok[n]) == want.size
        got = tokens[n].cpu().numpy()
        np.testing.assert_array_equal(got[: min(12, want.size)], want[:12].astype(np.int32))
        assert np.all(got[want.size:] == -7)


def _page_select(n_seq, T, G, scores, first=None, length=None, budget=0, stride=None):
    from budgeted_retention_amd import kvc
    n_pages = scores.shape[1]
    dims = kvc.make_dims(n_seq, 1, 1, 1, 64, T)
    stride = stride or n_pages
    kept = torch.full((n_seq, stride), -1, dtype=torch.int32, device="cuda")
    nk = torch.full((n_seq,), -1, dtype=torch.int32, device="cuda")
    ntok = torch.full((n_seq,), -1, dtype=torch.int32, device="cuda")
    pf = None if first is None else torch.from_numpy(first).cuda()
    pl = None if length is None else torch.from_numpy(length).cuda()
    kvc.kvc_page_select(dims, torch.from_numpy(scores).cuda(), G, n_pages, budget, kept, nk, ntok,
                        page_first=pf, page_len=pl)
    torch.cuda.synchronize()
    return kept.cpu().numpy(), nk.cpu().numpy(), ntok.cpu().numpy()


@pytest.mark.parametrize("n_pages", [1, 700, 1023, 1024, 1025, 3000])
@pytest.mark.parametrize("dist", ["ties", "gamma_inf_nan"])
def test_page_select_under_a_token_budget_matches_the_oracle(n_pages, dist):
    """kvc_page_select against oracle.page_effect.retained_pages_budget: the
    longest prefix of the (score desc, index asc) ranking whose page lengths
    fit the budget. Index work: exact."""
    rng = np.random.default_rng(n_pages * 7 + len(dist))
    N, G = 3, 16
    first, length, P = _event_pages(rng, N, 60 * n_pages, G, max_event=30)
    first, length = first[:, :n_pages].copy(), length[:, :n_pages].copy()
    T = int((first + length).max())
    if dist == "ties":
        sc = rng.integers(0, 4, (N, n_pages)).astype(np.float32)
    else:
        sc = rng.gamma(0.5, 1.0, (N, n_pages)).astype(np.float32)
        sc[rng.random((N, n_pages)) < 0.05] = -np.inf
        sc[rng.random((N, n_pages)) < 0.02] = np.nan
    tot = length.astype(np.int64).sum(axis=1)
    for budget in sorted({0, 1, int(tot.min()) // 3, int(tot.min()) - 1, int(tot.min()), int(tot.max()) + 5}):
        budget = max(budget, 0)
        kept, nk, ntok = _page_select(N, T, G, sc, first, length, budget)
        for n in range(N):
            want, used = o_pe.retained_pages_budget(sc[n].astype(np.float64), length[n], (), budget)
            assert nk[n] == want.size and ntok[n] == used, (n, budget)
            np.testing.assert_array_equal(kept[n][: want.size], want.astype(np.int32))


def test_page_select_uniform_pages_equal_the_top_k_select():
    """Uniform pages and a budget of k pages' tokens: kvc_select's top-k."""
    from budgeted_retention_amd import kvc
    rng = np.random.default_rng(4)
    N, G, P, k = 4, 16, 2500, 300
    sc = rng.integers(0, 50, (N, P)).astype(np.float32)                 # many ties
    sc[:, ::97] = -np.inf
    kept, nk, ntok = _page_select(N, P * G, G, sc, budget=k * G + G - 1)
    pol = kvc.Policy(0, 0, k, 1, 1, 0, 1, None, torch.zeros((1, 1), dtype=torch.float32, device="cuda"))
    kept2 = torch.full((N, k), -1, dtype=torch.int32, device="cuda")
    nk2 = torch.zeros(N, dtype=torch.int32, device="cuda")
    kvc.kvc_select(kvc.make_dims(N, 1, 1, 1, 64, P), torch.from_numpy(sc).cuda(), pol, kept2, k, nk2)
    torch.cuda.synchronize()
    assert np.all(nk == k) and np.all(ntok == k * G)
    np.testing.assert_array_equal(kept[:, :k], kept2.cpu().numpy())
    for n in range(N):
        np.testing.assert_array_equal(kept[n][:k], o_pe.retained_pages(sc[n].astype(np.float64), (), k))


def test_page_select_short_list_clamped_pages_and_the_largest_size():
    """A kept list shorter than the kept count holds its first entries;
    clamped page spans (past the cache, negative, longer than page_size) count
    their clamped lengths; 2^20 - 1 pages of 4096 tokens stay within 32-bit
    sums."""
    rng = np.random.default_rng(9)
    N, G, P, T = 2, 16, 2000, 20000
    first = np.sort(rng.integers(-40, T + 40, (N, P))).astype(np.int32)
    length = rng.integers(-3, 24, (N, P)).astype(np.int32)
    sc = rng.gamma(1.0, 1.0, (N, P)).astype(np.float32)
    clamped = np.clip(length, 0, G)
    f = np.clip(first, 0, T)
    clamped = np.minimum(clamped, T - f)
    kept, nk, ntok = _page_select(N, T, G, sc, first, length, 5000, stride=64)
    for n in range(N):
        want, used = o_pe.retained_pages_budget(sc[n].astype(np.float64), clamped[n], (), 5000)
        assert nk[n] == want.size > 64 and ntok[n] == used
        np.testing.assert_array_equal(kept[n], want[:64].astype(np.int32))
    # the largest call: every page 4096 tokens, a budget just under the 2^31 limit
    P = (1 << 20) - 1
    G = 4096
    sc = rng.random((1, P)).astype(np.float32)
    first = np.zeros((1, P), np.int32)
    length = np.full((1, P), G, np.int32)
    budget = (1 << 31) - 1
    kept, nk, ntok = _page_select(1, G, G, sc, first, length, budget)
    n_fit = budget // G
    want = np.sort(np.lexsort((np.arange(P), -sc[0].astype(np.float64)))[:n_fit])
    assert nk[0] == n_fit and ntok[0] == n_fit * G
    np.testing.assert_array_equal(kept[0][:n_fit], want.astype(np.int32))
