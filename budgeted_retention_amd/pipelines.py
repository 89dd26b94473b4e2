"""Whole-workload runs through the C ABI: the mixed-precision (PASK-style) and
page-lifecycle (CommitKV-style) workloads, call by call.

Each run takes an optional `timer`: a callable returning a context manager per
call name. bench.py passes one that brackets every GPU call with HIP events on
the current stream and every host step with the wall clock; the parity tests
pass none. Argument marshalling only: every step runs in libkvc.
"""
import contextlib
import statistics
import time

import numpy as np
import torch

from . import kvc


def _null_timer(name):
    return contextlib.nullcontext()


class CallTimer:
    """Per-call timing: HIP events around GPU calls (on the current stream),
    wall clock around host steps (names starting with 'host:')."""

    def __init__(self):
        self.events = []     # (name, start event, end event)
        self.host = {}       # name -> seconds

    @contextlib.contextmanager
    def __call__(self, name):
        if name.startswith("host:"):
            torch.cuda.synchronize()   # time the host step alone, not the GPU work queued before it
            t0 = time.perf_counter()
            yield
            self.host[name] = self.host.get(name, 0.0) + time.perf_counter() - t0
            return
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        yield
        b.record()
        self.events.append((name, a, b))

    def totals_ms(self):
        """Sum of event-timed milliseconds per call name (synchronises)."""
        torch.cuda.synchronize()
        out = {}
        for name, a, b in self.events:
            out[name] = out.get(name, 0.0) + a.elapsed_time(b)
        return out

    def median_step_ms(self, steps):
        """Per call name, the median over `steps` equal runs of that run's summed
        milliseconds (the events split into `steps` groups of the same calls), so
        that one run delayed on the host does not move the figures."""
        torch.cuda.synchronize()
        n = len(self.events)
        if steps < 1 or n % steps:
            raise ValueError(f"{n} timed calls do not split into {steps} equal runs")
        per = n // steps
        runs = []
        for i in range(steps):
            tot = {}
            for name, a, b in self.events[i * per:(i + 1) * per]:
                tot[name] = tot.get(name, 0.0) + a.elapsed_time(b)
            runs.append(tot)
        names = runs[0].keys()
        if any(r.keys() != names for r in runs):
            raise ValueError("the timed runs made different calls")
        return {k: statistics.median(r[k] for r in runs) for k in names}


def run_pask(w, inp, timer=None):
    """The mixed-precision workload: the prompt of every row scored by its
    observation window, compacted to B tokens with positions kept; the
    generated tokens' tags drive the per-token controller, each row takes its
    layer group's action (the last gen_recent tokens stay bf16) and its tokens
    are appended to the bf16 pool, quantised into the int8 pool or released;
    decode attention at the next position runs over both pools."""
    t = timer or _null_timer
    N, L, Hkv, Hq, d, Tp, Tg, W, B = (w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim,
                                      w.n_prompt, w.n_gen, w.window, w.budget)
    dev = inp.K.device
    rows = N * L * Hkv
    S = B + Tg                                         # pool capacity: kept prompt + every generated token
    dims_p = kvc.make_dims(N, L, Hkv, Hq, d, Tp)
    scores = torch.empty((N, L, Hkv, Tp), dtype=torch.float32, device=dev)
    ws = kvc.workspace(kvc.KVC_OP_SCORE, dims_p, W, 0, dev)
    with t("kvc_score"):
        kvc.kvc_score(dims_p, inp.K, inp.Q_obs, W, scores, ws)
    pol = kvc.Policy(w.n_sink, w.n_recent, B, 1, 1, 0, L, None,
                     torch.zeros((1, 1), dtype=torch.float32, device=dev))
    kept = torch.full((rows, B), -1, dtype=torch.int32, device=dev)
    nk = torch.zeros(rows, dtype=torch.int32, device=dev)
    with t("kvc_select"):
        st = kvc.kvc_select(dims_p, scores, pol, kept, B, nk)
    Ko = torch.zeros((rows, S, d), dtype=torch.bfloat16, device=dev)
    Vo = torch.zeros_like(Ko)
    po = torch.full((rows, S), -1, dtype=torch.int32, device=dev)
    nh0 = torch.zeros(rows, dtype=torch.int32, device=dev)
    with t("kvc_compact_rerotate:prompt"):
        kvc.kvc_compact_rerotate(dims_p, inp.K, inp.V, None, kept, B, nk, -1, w.rope_base,
                                 kvc.CompactOut(S, Ko, Vo, po, nh0))
    # controller per generated token, then each row's action (group broadcast, recent window bf16)
    with t("host:kvc_host_pask_control"):
        grp = np.array([kvc.kvc_layer_group(l, L, w.n_groups) for l in range(L)])
        costs = kvc.kvc_host_pask_costs(np.bincount(grp, minlength=w.n_groups), Hkv, d, w.low_bits)
        acts, ledger = kvc.kvc_host_pask_control(inp.a0, inp.amin, inp.prio, inp.critical, costs,
                                                 w.budget_fraction, inp.tags)
        act_rows = kvc.kvc_host_pask_row_actions(acts, L, Hkv, w.gen_recent)
    action = torch.from_numpy(act_rows.reshape(rows, Tg)).to(dev)
    kept_g = torch.arange(Tg, dtype=torch.int32, device=dev).expand(rows, Tg).contiguous()
    pos_g = (Tp + kept_g).contiguous()
    nk_g = torch.full((rows,), Tg, dtype=torch.int32, device=dev)
    Kq = torch.zeros((rows, S, d * w.low_bits // 8), dtype=torch.int8, device=dev)
    Vq = torch.zeros_like(Kq)
    Ks = torch.zeros((rows, S), dtype=torch.int16, device=dev)
    Vs = torch.zeros_like(Ks)
    pq = torch.full((rows, S), -1, dtype=torch.int32, device=dev)
    nh = torch.zeros(rows, dtype=torch.int32, device=dev)
    nl = torch.zeros(rows, dtype=torch.int32, device=dev)
    dims_g = kvc.make_dims(N, L, Hkv, Hq, d, Tg)
    with t("kvc_compact_rerotate:tiered"):
        kvc.kvc_compact_rerotate(dims_g, inp.K_gen, inp.V_gen, pos_g, kept_g, Tg, nk_g, -1, w.rope_base,
                                 kvc.CompactOut(S, Ko, Vo, po, nh, action, Kq, Vq, Ks, Vs, pq, nl, h_base=nh0,
                                                low_bits=w.low_bits))
    dims_d = kvc.make_dims(N, L, Hkv, Hq, d, S)
    wsd = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims_d, S, S)), dtype=torch.uint8, device=dev)
    o = torch.empty((N, L, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((N, L, Hq), dtype=torch.float32, device=dev)
    with t("kvc_decode_attn"):
        kvc.kvc_decode_attn(dims_d, inp.q_dec, Ko, Vo, nh, S, o, wsd, lse, None, 0, 0, Kq, Vq, Ks, Vs, nl, S,
                            w.low_bits)
    return dict(status=st, scores=scores, kept=kept, n_kept=nk, acts=acts, ledger=ledger, Ko=Ko, Vo=Vo,
                pos=po, n_h=nh, Kq=Kq, Vq=Vq, Ks=Ks, Vs=Vs, pos_q=pq, n_l=nl, o=o, lse=lse)


def _event_page_arrays(w, inp, dev):
    """Event pages of every trajectory (kvc_host_event_pages over its event
    lengths): int32 [N][P] first/length of all pages and the count of
    eligible ones (pages lying wholly before the pre-commit window: a prefix,
    pages being in token order). The batched page calls take one page count,
    so every trajectory must cut into the same number of pages."""
    cut = [kvc.kvc_host_event_pages(inp.events[n], w.page_size) for n in range(w.n_seq)]
    counts = {(f.size, int(np.count_nonzero(f + ln <= w.q_first_pre))) for f, ln in cut}
    if len(counts) != 1:
        raise ValueError(f"trajectories cut into different page counts {sorted(counts)}")
    P, n_elig = counts.pop()
    first = torch.from_numpy(np.stack([f for f, _ in cut])).to(dev)
    length = torch.from_numpy(np.stack([ln for _, ln in cut])).to(dev)
    return first, length, P, n_elig


def run_commit(w, inp, taus, timer=None):
    """The page-lifecycle workload at one commit: page deletion effects in the
    pre- and post-commit windows, lifecycle labels and candidate order (host),
    greedy joint retirement for every bound in `taus` (the first feeds the
    checkpoint), checkpoint page scores from the post-commit window, the
    retained page set, the compaction of keys, values and positions by that
    one page set, and decode attention at the next position over the
    compacted pool and over a paged view of the original storage.

    Uniform pages keep budget / page_size pages (kvc_select over the page
    scores) and compact by page list. Event pages (w.event_max > 0) are cut
    on the host, keep the longest prefix of the page ranking that fits the
    token budget (kvc_page_select), expand it into one token list per
    trajectory (kvc_page_tokens), compact by that list and decode the
    original storage through it as a block table of one-token pages."""
    t = timer or _null_timer
    N, L, Hkv, Hq, d, T, W, ps = (w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim,
                                  w.n_tokens, w.window, w.page_size)
    dev = inp.K.device
    events = bool(w.event_max)
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    ws = kvc.page_workspace(dims, W, w.q_first_post, dev)
    if events:
        with t("host:kvc_host_event_pages"):
            pf_all, pl_all, P, n_elig = _event_page_arrays(w, inp, dev)
        pf, pl = pf_all[:, :n_elig].contiguous(), pl_all[:, :n_elig].contiguous()
    else:
        pf_all = pl_all = pf = pl = None
        P, n_elig = w.n_pages_all, w.n_eligible
    Rm = torch.empty((N, n_elig), dtype=torch.float32, device=dev)
    Rp = torch.empty_like(Rm)
    with t("kvc_page_effect:pre"):
        kvc.kvc_page_effect(dims, w.layer, inp.K, inp.V, inp.Q_pre, W, w.q_first_pre, ps, n_elig, Rm, ws,
                            page_first=pf, page_len=pl)
    with t("kvc_page_effect:post"):
        kvc.kvc_page_effect(dims, w.layer, inp.K, inp.V, inp.Q_post, W, w.q_first_post, ps, n_elig, Rp, ws,
                            page_first=pf, page_len=pl)
    with t("host:kvc_host_commit_candidates"):
        Rm_h, Rp_h = Rm.cpu().numpy(), Rp.cpu().numpy()
        states, orders, n_orders = [], [], []
        for n in range(N):
            st, od, no = kvc.kvc_host_commit_candidates(Rm_h[n], Rp_h[n], w.tau_use, w.tau_dead, w.rho_use,
                                                         w.rho_dead, w.max_scan)
            states.append(st)
            orders.append(od)
            n_orders.append(no)
        order = torch.from_numpy(np.stack(orders)).to(dev)
    retire = []
    for k, tau in enumerate(taus):
        acc = torch.zeros((N, w.max_scan), dtype=torch.uint8, device=dev)
        jr = torch.zeros((N, w.max_scan), dtype=torch.float32, device=dev)
        with t("kvc_page_retire" if k == 0 else f"kvc_page_retire:{k}"):
            kvc.kvc_page_retire(dims, w.layer, inp.K, inp.V, inp.Q_post, W, w.q_first_post, ps, n_elig,
                                order, tau, acc, ws, jr, page_first=pf, page_len=pl)
        retire.append((acc, jr))
    acc = retire[0][0]
    # checkpoint: page scores from the post-commit window, best pages kept for every row
    scores = torch.empty((N, L, Hkv, T), dtype=torch.float32, device=dev)
    wss = kvc.workspace(kvc.KVC_OP_SCORE, dims, W, 0, dev)
    with t("kvc_score"):
        kvc.kvc_score(dims, inp.K, inp.Q_post, W, scores, wss)
    B = w.budget
    pscore = torch.empty((N, P), dtype=torch.float32, device=dev)
    with t("kvc_page_scores"):
        kvc.kvc_page_scores(dims, scores, ps, P, pscore, order, acc, page_first=pf_all, page_len=pl_all)
    rows = N * L * Hkv
    if events:
        kept = torch.full((N, min(P, B)), -1, dtype=torch.int32, device=dev)
        nk = torch.zeros(N, dtype=torch.int32, device=dev)
        n_tok = torch.zeros(N, dtype=torch.int32, device=dev)
        with t("kvc_page_select"):
            kvc.kvc_page_select(dims, pscore, ps, P, B, kept, nk, n_tok, page_first=pf_all, page_len=pl_all)
        tokens = torch.full((N, B), -1, dtype=torch.int32, device=dev)
        with t("kvc_page_tokens"):
            kvc.kvc_page_tokens(dims, ps, P, kept, nk, tokens, n_tok, page_first=pf_all, page_len=pl_all)
        kept_list, kept_stride, kept_page, n_list = tokens, B, 1, n_tok
    else:
        Bp = B // ps
        pol = kvc.Policy(0, 0, Bp, 1, 1, 0, 1, None, torch.zeros((1, 1), dtype=torch.float32, device=dev))
        kept = torch.full((N, Bp), -1, dtype=torch.int32, device=dev)
        nk = torch.zeros(N, dtype=torch.int32, device=dev)
        with t("kvc_select"):
            kvc.kvc_select(kvc.make_dims(N, 1, 1, 1, 64, P), pscore, pol, kept, Bp, nk)
        kept_list, kept_stride, kept_page, n_list = kept, Bp, ps, nk
    Ko = torch.zeros((rows, B, d), dtype=torch.bfloat16, device=dev)
    Vo = torch.zeros_like(Ko)
    po = torch.full((rows, B), -1, dtype=torch.int32, device=dev)
    nh = torch.zeros(rows, dtype=torch.int32, device=dev)
    with t("kvc_compact_rerotate"):
        kvc.kvc_compact_rerotate(dims, inp.K, inp.V, None, kept_list, kept_stride, n_list, -1, 1e6,
                                 kvc.CompactOut(B, Ko, Vo, po, nh, kept_page=kept_page))
    # decode at position T: over the compacted pool, and through a block table of the kept pages
    dims_c = kvc.make_dims(N, L, Hkv, Hq, d, B)
    o1 = torch.empty((N, L, Hq, d), dtype=torch.bfloat16, device=dev)
    o2 = torch.empty_like(o1)
    lse1 = torch.empty((N, L, Hq), dtype=torch.float32, device=dev)
    lse2 = torch.empty_like(lse1)
    ws1 = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims_c, B, 0)), dtype=torch.uint8, device=dev)
    with t("kvc_decode_attn:pool"):
        kvc.kvc_decode_attn(dims_c, inp.q_dec, Ko, Vo, nh, B, o1, ws1, lse1)
    ws2 = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims, kept_stride * kept_page, 0)),
                      dtype=torch.uint8, device=dev)
    # every row of a trajectory holds its kept tokens (uniform pages: exactly the budget)
    n_all = nh if events else torch.full((rows,), B, dtype=torch.int32, device=dev)
    with t("kvc_decode_attn:paged"):
        kvc.kvc_decode_attn(dims, inp.q_dec, inp.K, inp.V, n_all, T, o2, ws2, lse2, kept_list, kept_page,
                            kept_stride)
    out = dict(Rm=Rm, Rp=Rp, states=np.stack(states), order=np.stack(orders), n_order=np.array(n_orders),
               retire=retire, scores=scores, pscore=pscore, kept=kept, n_kept=nk, Ko=Ko, Vo=Vo, pos=po, n_h=nh,
               o1=o1, o2=o2, lse1=lse1, lse2=lse2)
    if events:
        out.update(page_first=pf_all, page_len=pl_all, n_eligible=n_elig, tokens=tokens, n_tokens=n_tok)
    return out


# PACE §3.1: the foresight bonus scale. Its floor sigma/2 must stay above every
# cumulative attention score a slot can reach, so that every referenced token
# outranks every unreferenced one; a running H2O score grows without bound over
# a session (the pages report scores near 25,000), hence the page's 1e5.
H2O_SIGMA = 1e5


def run_h2o(w, inp, cycles, timer=None, record=False, sigma=H2O_SIGMA, lam=0.35):
    """PACE-style decode with H2O eviction over a resident cache of B + E
    slots per row: each cycle the engine appends E new tokens (score 0, no
    tag, no reference), E decode steps add their attention to the slots'
    cumulative scores, then the rows are evicted back to B slots by cumulative
    score + foresight bonus (per-slot tags) and compacted; scores, tags and
    the reference store move with the slots. Positions are kept unless the
    workload bounds them (w.limit = L > 0, PACE §3.2): after each eviction the
    host rule (kvc_host_pace_renumber, headroom E) decides whether this
    compaction renumbers the resident rows to 0..B-1, re-deriving the keys
    from the reference store, and the sequence's shift advances so new tokens
    continue at B. Two slot pools alternate. With `record`, returns per cycle
    the scores before eviction, the kept lists, the renumber decisions and the
    resident state after compaction, plus the final pool."""
    t = timer or _null_timer
    N, L, Hkv, Hq, d = w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim
    rows, S, B, E = w.rows, w.slots, w.budget, w.interval
    dev = inp.K.device
    dims = kvc.make_dims(N, L, Hkv, Hq, d, S)

    def pool():
        return dict(K=torch.empty((rows, S, d), dtype=torch.bfloat16, device=dev), V=torch.empty((rows, S, d),
                    dtype=torch.bfloat16, device=dev), pos=torch.empty((rows, S), dtype=torch.int32, device=dev),
                    acc=torch.empty((rows, S), dtype=torch.float32, device=dev),
                    tags=torch.empty((rows, S), dtype=torch.uint8, device=dev),
                    Kr=torch.zeros((rows, S, d), dtype=torch.bfloat16, device=dev),
                    pr=torch.full((rows, S), -1, dtype=torch.int32, device=dev))
    cur, nxt = pool(), pool()
    for k, src in (("K", inp.K), ("V", inp.V), ("pos", inp.pos), ("acc", inp.acc), ("tags", inp.tags)):
        cur[k].copy_(src)
    vals = [0.0] + [kvc.kvc_foresight_bonus(sigma, lam, s) for s in inp.steps_ahead]
    bonus = torch.tensor(vals, dtype=torch.float32, device=dev).reshape(-1, 1)
    nh = [torch.full((rows,), B + e + 1, dtype=torch.int32, device=dev) for e in range(E)]
    new_pos = int(inp.pos[:, B:].min().item())   # logical position of the first appended token
    shift = 0
    ar = torch.arange(E, dtype=torch.int32, device=dev)
    o = torch.empty((N, L, Hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, kvc.kvc_decode_h2o_workspace_bytes(dims, S)), dtype=torch.uint8, device=dev)
    kept = torch.full((rows, B), -1, dtype=torch.int32, device=dev)
    nk = torch.zeros(rows, dtype=torch.int32, device=dev)
    rec = []
    for c in range(cycles):
        with t("append"):
            cur["K"][:, B:] = inp.K_new[c]
            cur["V"][:, B:] = inp.V_new[c]
            cur["pos"][:, B:] = new_pos + c * E - shift + ar
            cur["acc"][:, B:] = 0.0
            cur["tags"][:, B:] = 0
            cur["pr"][:, B:] = -1
        for e in range(E):
            with t("kvc_decode_attn_h2o"):
                kvc.kvc_decode_attn_h2o(dims, inp.q[c, e], cur["K"], cur["V"], nh[e], S, cur["acc"], o, ws)
        if record:
            rec.append({"acc": cur["acc"].clone(), "pos": cur["pos"].clone(), "tags": cur["tags"].clone()})
        pol = kvc.Policy(w.n_sink, w.n_recent, B, len(vals), 1, 0, L, cur["tags"], bonus, None, tag_rows=1)
        with t("kvc_select"):
            kvc.kvc_select(dims, cur["acc"], pol, kept, B, nk)
        out = kvc.CompactOut(S, nxt["K"], nxt["V"], nxt["pos"], None, K_ref=cur["Kr"], p_ref=cur["pr"],
                             K_ref_out=nxt["Kr"], p_ref_out=nxt["pr"], score_in=cur["acc"],
                             score_out=nxt["acc"], tag_in=cur["tags"], tag_out=nxt["tags"])
        renumber = False
        if w.limit:
            renumber, shift = kvc.kvc_host_pace_renumber(new_pos + (c + 1) * E, shift, B, w.limit, E, B + E)
        with t("kvc_compact_rerotate"):
            kvc.kvc_compact_rerotate(dims, cur["K"], cur["V"], cur["pos"], kept, B, nk, 0 if renumber else -1,
                                     w.rope_base, out)
        if record:
            rec[-1].update(kept=kept.clone(), n_kept=nk.clone(), renumber=renumber,
                           post={k: nxt[k][:, :B].clone() for k in ("K", "V", "pos", "acc", "tags", "Kr", "pr")})
        cur, nxt = nxt, cur
    return {"cycles": rec, "final": cur, "o": o}


def run_commit_multi(w, inp, timer=None, record=False):
    """Successive commits of the CommitKV lifecycle (§3.2-3.4) for every
    trajectory. Per commit c:

    1. the engine appends turn c to the resident cache (t_pre tokens);
    2. pre-commit deletion effects R^- of every page before the pre-commit
       window, at the deciding layer (kvc_page_effect);
    3. the turn's pages, pending their post-commit measurement, are protected
       by decreasing R^- under B_N = floor(eta B), at most 16 pages
       (kvc_host_commit_protect, Eq. 12);
    4. checkpoint: window scores of the pre-commit queries, page scores with
       the pages retired at the previous commit excluded, top pages to B
       tokens with the protected pages floored (Eq. 13), compaction of keys,
       values and positions by the one page set (Eq. 4);
    5. the engine appends the observation and the post-commit window;
    6. post-commit effects R^+ of the retained pages that carry an R^-,
       lifecycle labels and candidate order (kvc_host_commit_candidates), and
       greedy joint retirement (kvc_page_retire, Eq. 11), whose accepted
       pages the next checkpoint excludes.
    With `record`, returns the per-commit host arrays the parity tests use."""
    t = timer or _null_timer
    N, L, Hkv, Hq, d, W, ps = w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.window, w.page_size
    B, Ta, Tb = w.budget, w.t_pre, w.t_post
    dev = inp.K0.device
    Pa, Pb, n_keep = Ta // ps, Tb // ps, B // ps
    n_el = (Ta - W) // ps                         # pages wholly before the pre-commit window
    first_turn_page = Tb // ps
    dims_a = kvc.make_dims(N, L, Hkv, Hq, d, Ta)
    dims_b = kvc.make_dims(N, L, Hkv, Hq, d, Tb)
    dims_p = kvc.make_dims(N, 1, 1, 1, 64, Pa)
    ws_a = kvc.page_workspace(dims_a, W, Ta - W, dev)
    ws_b = kvc.page_workspace(dims_b, W, Tb - W, dev)
    ws_s = kvc.workspace(kvc.KVC_OP_SCORE, dims_a, W, 0, dev)
    Ka = torch.empty((N, L, Hkv, Ta, d), dtype=torch.bfloat16, device=dev)
    Va = torch.empty_like(Ka)
    pa = torch.empty((N, L, Hkv, Ta), dtype=torch.int32, device=dev)
    Kb = inp.K0.clone()
    Vb = inp.V0.clone()
    pb = torch.arange(Tb, dtype=torch.int32, device=dev).expand(N, L, Hkv, Tb).contiguous()
    nh = torch.zeros(N * L * Hkv, dtype=torch.int32, device=dev)
    Rm = torch.empty((N, n_el), dtype=torch.float32, device=dev)
    Rp = torch.empty((N, n_keep), dtype=torch.float32, device=dev)
    scores = torch.empty((N, L, Hkv, Ta), dtype=torch.float32, device=dev)
    pscore = torch.empty((N, Pa), dtype=torch.float32, device=dev)
    # a floor table may protect any page, so selection gets a full-length list
    kept_sel = torch.full((N, Pa), -1, dtype=torch.int32, device=dev)
    kept = kept_sel[:, :n_keep]
    nk = torch.zeros(N, dtype=torch.int32, device=dev)
    floor = torch.tensor([[0], [1]], dtype=torch.uint8, device=dev)
    zero_bonus = torch.zeros((2, 1), dtype=torch.float32, device=dev)
    order = torch.full((N, w.max_scan), -1, dtype=torch.int32, device=dev)   # cache_b page indices
    accepted = torch.zeros((N, w.max_scan), dtype=torch.uint8, device=dev)
    next_pos = Tb
    rec = []
    for c in range(w.commits):
        with t("append"):
            Ka[:, :, :, :Tb] = Kb
            Va[:, :, :, :Tb] = Vb
            pa[:, :, :, :Tb] = pb
            Ka[:, :, :, Tb:] = inp.K_call[c]
            Va[:, :, :, Tb:] = inp.V_call[c]
            pa[:, :, :, Tb:] = torch.arange(next_pos, next_pos + w.n_call, dtype=torch.int32, device=dev)
        next_pos += w.n_call
        with t("kvc_page_effect:pre"):
            kvc.kvc_page_effect(dims_a, w.layer, Ka, Va, inp.Q_pre[c], W, Ta - W, ps, n_el, Rm, ws_a)
        with t("host:kvc_host_commit_protect"):
            Rm_h = Rm.cpu().numpy()
            tags = np.zeros((N, Pa), np.uint8)
            for n in range(N):
                pend = np.arange(first_turn_page, n_el)
                prot, _ = kvc.kvc_host_commit_protect(Rm_h[n, pend], np.full(pend.size, ps, np.int32), B, w.eta,
                                                      w.max_protect)
                tags[n, pend[prot.astype(bool)]] = 1
            tags_d = torch.from_numpy(tags).to(dev)
        with t("kvc_score"):
            kvc.kvc_score(dims_a, Ka, inp.Q_pre[c], W, scores, ws_s)
        with t("kvc_page_scores"):
            kvc.kvc_page_scores(dims_a, scores, ps, Pa, pscore, order if c else None, accepted if c else None)
        pol = kvc.Policy(0, 0, n_keep, 2, 1, 0, 1, tags_d, zero_bonus, floor)
        with t("kvc_select"):
            kvc.kvc_select(dims_p, pscore, pol, kept_sel, Pa, nk)
        with t("kvc_compact_rerotate"):
            kvc.kvc_compact_rerotate(dims_a, Ka, Va, pa, kept_sel, Pa, nk, -1, 1e6,
                                     kvc.CompactOut(Tb, Kb, Vb, pb, nh, kept_page=ps))
        with t("append"):
            Kb[:, :, :, B:] = inp.K_obs[c]
            Vb[:, :, :, B:] = inp.V_obs[c]
            pb[:, :, :, B:] = torch.arange(next_pos, next_pos + w.n_obs + W, dtype=torch.int32, device=dev)
        next_pos += w.n_obs + W
        with t("kvc_page_effect:post"):
            kvc.kvc_page_effect(dims_b, w.layer, Kb, Vb, inp.Q_post[c], W, Tb - W, ps, n_keep, Rp, ws_b)
        with t("host:kvc_host_commit_candidates"):
            Rp_h, kept_h = Rp.cpu().numpy(), kept.cpu().numpy()
            ord_h = np.full((N, w.max_scan), -1, np.int32)
            ncand = np.zeros(N, np.int32)
            events = []
            for n in range(N):
                ev = np.flatnonzero(kept_h[n] < n_el)            # retained pages with an R^-
                events.append(ev)
                if ev.size == 0:
                    continue
                _, od, no = kvc.kvc_host_commit_candidates(Rm_h[n, kept_h[n, ev]], Rp_h[n, ev], w.tau_use,
                                                           w.tau_dead, w.rho_use, w.rho_dead, w.max_scan)
                ord_h[n, :no] = ev[od[:no]]
                ncand[n] = no
            order = torch.from_numpy(ord_h).to(dev)
        accepted = torch.zeros((N, w.max_scan), dtype=torch.uint8, device=dev)
        with t("kvc_page_retire"):
            kvc.kvc_page_retire(dims_b, w.layer, Kb, Vb, inp.Q_post[c], W, Tb - W, ps, n_keep, order,
                                w.tau_joint, accepted, ws_b)
        if record:
            rec.append(dict(Rm=Rm_h.copy(), tags=tags, pscore=pscore.cpu().numpy(), kept=kept_h.copy(),
                            n_kept=nk.cpu().numpy(), Rp=Rp_h.copy(), events=events, order=ord_h.copy(),
                            n_order=ncand.copy(), accepted=accepted.cpu().numpy(), pos=pb.cpu().numpy()))
    return dict(commits=rec, K=Kb, V=Vb, pos=pb)
