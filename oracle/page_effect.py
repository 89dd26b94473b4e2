"""CommitKV page deletion effects and lifecycle decisions (test infrastructure).

CommitKV §3.2: for one attention layer and query head, a query p pays
attention a_pi to resident token i and produces o_p. Deleting an event page
E (a contiguous span of at most G tokens) and renormalising the remaining
weights gives o_p^{\\E}; Eq. 6 writes that renormalisation in closed form.
This oracle uses the plain definition instead -- attention recomputed over
the visible tokens not in E -- which Eq. 6 reaches exactly.

    R_h(E; Q) = max_{p in Q} ||o_p - o_p^{\\E}||_2 / ||o_p||_2     (Eq. 7)
    R(E; Q)   = max_h R_h(E; Q)

Eq. 8 evaluates it on the pre-commit window Q^- and the post-commit window
Q^+ (Eq. 5). Eq. 9 labels a page high (R >= tau_use and percentile >=
rho_use) or low (R <= tau_dead and percentile <= rho_dead); Eq. 10 names the
states; §3.3 (Eq. 11) retires completion candidates greedily, in the order
(R^+ ascending, R^- descending), while the joint effect of the retired set
stays within tau_joint. The page's setup section fixes tau_use = 0.05,
rho_use = 0.75, rho_dead = 0.25 and a scan of at most 64 pages.

Readings where the page is silent:
* percentile rank = fraction of the other comparison pages with a strictly
  smaller effect: #{E' : R(E') < R(E)} / (|E_c| - 1);
* remaining ties in the greedy order go to the lower page index;
* deleting every visible token leaves no output: the effect is +inf and such
  a page is never accepted.

Checkpoint retention (§3.3, Eq. 13, with Eq. 4's single index set): a page's
score pools the window score of its tokens over every layer and KV head of
the sequence; retired pages are excluded; the best n_keep pages are kept.
With event pages of unequal length the budget counts tokens instead
(retained_pages_budget).

Parity status: the effect itself is pinned (Eq. 6 identity, brute force,
closed forms); the page score and the retained set by hand-built cases and
brute force; the labels and the greedy loop only by invariants and
hand-built cases -- the workload they run on in the benchmark is synthetic,
so beyond those invariants they are "parity unpinned".
"""
import numpy as np

STATES = ("uncertain", "completion_candidate", "dormant", "newly_active", "still_active")


def head_outputs(K, V, Q, q_pos, k_pos=None, drop=None):
    """Attention outputs of one query head over one KV head.

    K, V: [T, d]; Q: [P, d]; q_pos: [P]; k_pos: [T] (default 0..T-1);
    drop: boolean [T] of tokens removed before the softmax (default none).
    Returns [P, d] float64; rows with no remaining visible key are NaN.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Q = np.asarray(Q, np.float64)
    T, d = K.shape
    if k_pos is None:
        k_pos = np.arange(T)
    vis = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    if drop is not None:
        vis &= ~np.asarray(drop, bool)[None, :]
    s = np.where(vis, (Q @ K.T) / np.sqrt(d), -np.inf)
    m = s.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.exp(s - m)
        e = np.where(vis, e, 0.0)
        return (e @ V) / e.sum(axis=1, keepdims=True)


def deletion_effect(K, V, Q, q_pos, tokens, k_pos=None):
    """R(E; Q) and its absolute numerator for the token set ``tokens``.

    K, V: [Hkv, T, d]; Q: [Hq, P, d] (Hq a multiple of Hkv, query head h reads
    KV head h // (Hq/Hkv)); q_pos: [P]. Returns (R_rel, R_abs) with
    R_rel = max_h max_p ||o - o^{\\E}|| / ||o|| and
    R_abs = max_h max_p ||o - o^{\\E}||.
    """
    Hkv, T, _ = np.shape(K)
    Hq = np.shape(Q)[0]
    G = Hq // Hkv
    drop = np.zeros(T, bool)
    drop[np.asarray(tokens, dtype=np.int64)] = True
    rel = 0.0
    ab = 0.0
    for h in range(Hq):
        kv = h // G
        o = head_outputs(K[kv], V[kv], Q[h], q_pos, k_pos)
        o_del = head_outputs(K[kv], V[kv], Q[h], q_pos, k_pos, drop)
        if np.isnan(o_del).any():
            return np.inf, np.inf
        diff = np.linalg.norm(o - o_del, axis=1)
        rel = max(rel, float(np.max(diff / np.linalg.norm(o, axis=1))))
        ab = max(ab, float(np.max(diff)))
    return rel, ab


def page_tokens(first, page_size):
    return np.arange(first, first + page_size, dtype=np.int64)


def event_pages(event_lengths, G, start=0):
    """Event pages (CommitKV §3.1, "Agent events and commit transitions"):
    every event is partitioned into contiguous pages of at most G tokens, so no
    page spans two events. Reading: an event is cut from its first token into
    pages of G tokens, the last one shorter. Events follow each other from
    token ``start``. Returns (first, length), int64, in token order.
    """
    first, length = [], []
    t = int(start)
    for n_ev in event_lengths:
        off = 0
        while off < n_ev:
            ln = min(int(G), int(n_ev) - off)
            first.append(t + off)
            length.append(ln)
            off += ln
        t += int(n_ev)
    return np.asarray(first, np.int64), np.asarray(length, np.int64)


def page_scores_spans(row_scores, first, length):
    """page_scores for pages given as token spans [first[e], first[e] + length[e])."""
    per_token = np.asarray(row_scores, np.float64).sum(axis=0)
    return np.array([per_token[f:f + ln].sum() for f, ln in zip(np.asarray(first), np.asarray(length))])


def retained_tokens(first, length, pages):
    """The index set of the listed pages (Eq. 13 applied through Eq. 4's single
    index set): each page's tokens in order, pages in list order."""
    parts = [np.arange(first[e], first[e] + length[e], dtype=np.int64) for e in pages]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def percentile_ranks(R):
    """P(E) = #{E' != E : R(E') < R(E)} / (n - 1)."""
    R = np.asarray(R, np.float64)
    n = R.size
    if n <= 1:
        return np.zeros(n)
    less = (R[None, :] < R[:, None]).sum(axis=1)
    return less / (n - 1)


def lifecycle_states(R_minus, R_plus, tau_use, tau_dead, rho_use, rho_dead):
    """Eq. 9-10 labels per page; returns an int array indexing STATES."""
    Pm, Pp = percentile_ranks(R_minus), percentile_ranks(R_plus)
    Rm, Rp = np.asarray(R_minus), np.asarray(R_plus)
    Hm = (Rm >= tau_use) & (Pm >= rho_use)
    Lm = (Rm <= tau_dead) & (Pm <= rho_dead)
    Hp = (Rp >= tau_use) & (Pp >= rho_use)
    Lp = (Rp <= tau_dead) & (Pp <= rho_dead)
    st = np.zeros(Rm.size, np.int64)
    st[Hm & Lp] = 1
    st[Lm & Lp] = 2
    st[Lm & Hp] = 3
    st[Hm & Hp] = 4
    return st


def candidate_order(R_minus, R_plus, states):
    """Completion candidates sorted by (R^+ asc, R^- desc, index asc)."""
    idx = np.flatnonzero(np.asarray(states) == 1)
    Rm, Rp = np.asarray(R_minus), np.asarray(R_plus)
    order = np.lexsort((idx, -Rm[idx], Rp[idx]))
    return idx[order]


def page_scores(row_scores, page_size, n_pages):
    """Checkpoint page score of one sequence (CommitKV §3.3 with Eq. 4: one
    index set for every layer and head, so the score is pooled over them):
    the window score of every token, summed over the sequence's rows
    (layers x KV heads) and over the page's tokens.

    row_scores: [R, T] float64 (R = layers x KV heads). Returns [n_pages].
    """
    S = np.asarray(row_scores, np.float64)
    per_token = S.sum(axis=0)
    return np.array([per_token[e * page_size:(e + 1) * page_size].sum() for e in range(n_pages)])


def retained_pages(score, retired, n_keep, protected=()):
    """Pages kept at the checkpoint (CommitKV §3.3, Eq. 13): the protected
    pending pages N are kept, retired pages are excluded (scored -inf), the
    rest ranked by (score descending, page index ascending) fill the budget
    to n_keep; returned in ascending order. Retired pages are used only when
    fewer than n_keep others exist.
    """
    score = np.asarray(score, np.float64).copy()
    score[np.asarray(list(retired), dtype=np.int64)] = -np.inf
    if score.size <= n_keep:
        return np.arange(score.size, dtype=np.int64)
    prot = np.asarray(sorted(set(int(e) for e in protected)), dtype=np.int64)
    if prot.size >= n_keep:
        return prot
    rest = np.setdiff1d(np.arange(score.size), prot)
    order = rest[np.lexsort((rest, -score[rest]))]
    return np.sort(np.concatenate([prot, order[: n_keep - prot.size]])).astype(np.int64)


def retained_pages_budget(score, length, retired, budget):
    """Pages kept at the checkpoint when pages differ in length (event pages,
    CommitKV §3.1) and the budget counts tokens (§3.3, Eq. 13: |I| <= B).

    Reading: retired pages are scored -inf, as in retained_pages; pages are
    ranked by (score descending, page index ascending), a NaN score below
    every other; the kept pages are the longest prefix of that ranking whose
    lengths sum to at most the budget, so the first page that does not fit
    ends the prefix. Returns (kept pages ascending, kept token count).
    """
    s = np.asarray(score, np.float64).copy()
    ln = np.asarray(length, np.int64)
    ret = np.asarray(sorted(set(int(e) for e in retired)), dtype=np.int64)
    s[ret] = -np.inf
    ranked = sorted(range(s.size), key=lambda e: (1, 0.0, e) if np.isnan(s[e]) else (0, -s[e], e))
    kept, used = [], 0
    for e in ranked:
        if used + ln[e] > budget:
            break
        used += int(ln[e])
        kept.append(e)
    return np.sort(np.asarray(kept, np.int64)), used


def protect_pending(R_minus, page_tokens, budget, eta, max_pages=16):
    """Pending pages protected at a checkpoint (CommitKV §3.3 "Protecting
    incomplete transitions", Eq. 12): pages awaiting their post-commit
    measurement are protected in order of decreasing pre-commit effect
    (ties: lower index) while their tokens total at most B_N = floor(eta * B)
    and at most max_pages pages are protected (the setup section protects at
    most 16). Reading: the protected set is a prefix of that order -- the
    first page that does not fit ends it. Returns the protected indices
    (positions in R_minus), ascending.
    """
    Rm = np.asarray(R_minus, np.float64)
    tok = np.asarray(page_tokens, np.int64)
    B_N = int(np.floor(eta * budget))
    order = np.lexsort((np.arange(Rm.size), -Rm))
    out, used = [], 0
    for e in order:
        if len(out) >= max_pages or used + tok[e] > B_N:
            break
        out.append(int(e))
        used += int(tok[e])
    return np.sort(np.asarray(out, np.int64))


def greedy_retire(order, joint_effect, tau_joint, max_scan=64):
    """Eq. 11: walk ``order`` (at most max_scan entries) and accept E iff
    joint_effect(D + [E]) <= tau_joint. Returns the accepted page list D."""
    D = []
    for E in list(order)[:max_scan]:
        if joint_effect(D + [int(E)]) <= tau_joint:
            D.append(int(E))
    return D
