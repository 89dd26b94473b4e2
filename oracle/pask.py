"""PASK online structural control (test infrastructure).

PASK §3.5 and Algorithm 2: every generated token has a structural tag z_t;
a constant-time lookup in the frozen table gives, per layer group c, a base
action a0_c, a floor a-_c and the frozen upgrade priorities. Actions are
ordered by protection, R (release) < L (low precision) < H (bf16). Then

    a_t   = max(a0, a-)                               (Eq. 11)
    B_t   = [R_t - Gamma]_+                           (Eq. 11)
    Demote: apply the eligible adjacent demotion (never below the floor) with
            the smallest stored priority until M(a_t) <= B_t or only floors
            remain (floors take precedence over the budget).
    Promote (critical tags only): apply adjacent promotions in descending
            priority while the total cost still fits B_t.
    R_{t+1} = R_t - M(a_t) + b,  b = B_D * C_full,  R_1 = b.

Payload costs follow PASK Appendix B.3 (Eq. 13-14), with the low-precision
tier at 8 bits instead of 4: n_c = 2 * sum_{l in c} H_kv * d,
k_c = 2 * sum_{l in c} H_kv, m(R) = 0, m(H) = 16 n_c, m(L) = 8 n_c + 16 k_c
(one FP16 scale per token, KV head and K/V).

Readings where the page is silent: the reserve table Gamma is 0 (the fallback
controller of Appendix A.4 uses Gamma = 0); the priority of demoting H->L is
the stored priority of the upgrade L->H it undoes (and R<-L that of R->L);
priority ties go to the lower group index (a fixed serialized tie order,
Appendix A.4); promotion stops at the first step that does not fit.

Parity status: pinned by invariants (floors never violated, the ledger's
closed form R_t = t*b - sum_{i<t} M(a_i) from Appendix B.6, the all-high
fallback), by hand-built steps whose outcome the order of §3.5 fixes (which
group is demoted first, which priority a demotion carries, promotion in
descending priority stopping at the first step that does not fit, ties to
the lower group), and by a search over every order of the groups' step
chains that picks the smallest (demotion) or largest (promotion) priorities
first. The synthetic tag chain and table it runs on in the benchmark are
"parity unpinned" beyond those.
"""
import numpy as np

R_ACT, L_ACT, H_ACT = 0, 1, 2


def group_costs(layers_per_group, n_kv_heads, head_dim, low_bits=8):
    """Per-group (m(R), m(L), m(H)) in bits, PASK Eq. 13-14."""
    out = []
    for nl in layers_per_group:
        n_c = 2 * nl * n_kv_heads * head_dim
        k_c = 2 * nl * n_kv_heads
        out.append((0, low_bits * n_c + 16 * k_c, 16 * n_c))
    return np.array(out, dtype=np.float64)


def cost(actions, costs):
    return float(sum(costs[c][a] for c, a in enumerate(actions)))


def control_token(a0, amin, prio_up, critical, R_t, costs, gamma=0.0):
    """One step of Algorithm 2.

    a0, amin: [C] actions; prio_up: [C][2] stored priorities of the upgrades
    R->L (index 0) and L->H (index 1); critical: bool. Returns (a_t, M(a_t)).
    """
    C = len(a0)
    a = [max(int(a0[c]), int(amin[c])) for c in range(C)]
    B_t = max(R_t - gamma, 0.0)
    while cost(a, costs) > B_t:
        best = None
        for c in range(C):
            if a[c] > amin[c]:
                p = prio_up[c][a[c] - 1]       # priority of the upgrade this demotion undoes
                if best is None or p < best[0]:
                    best = (p, c)
        if best is None:
            break
        a[best[1]] -= 1
    if critical:
        while True:
            best = None
            for c in range(C):
                if a[c] < H_ACT:
                    p = prio_up[c][a[c]]
                    if best is None or p > best[0]:
                        best = (p, c)
            if best is None:
                break
            c = best[1]
            delta = costs[c][a[c] + 1] - costs[c][a[c]]
            if cost(a, costs) + delta > B_t:
                break
            a[c] += 1
    return a, cost(a, costs)


def control_sequence(tags, table_a0, table_amin, table_prio, table_crit, costs, B_D, gamma=0.0):
    """Run Algorithm 2 over one sequence of generated-token tags.

    tags: [n] ints; table_a0/table_amin: [n_tags][C]; table_prio: [n_tags][C][2];
    table_crit: [n_tags]. Returns (actions [n][C] int, ledger R_t [n+1]).
    """
    costs = np.asarray(costs, np.float64)
    b = B_D * float(costs[:, H_ACT].sum())
    R = b
    acts = np.zeros((len(tags), costs.shape[0]), np.int64)
    ledger = [R]
    for t, z in enumerate(tags):
        a, M = control_token(table_a0[z], table_amin[z], table_prio[z],
                             bool(table_crit[z]), R, costs, gamma)
        acts[t] = a
        R = R - M + b
        ledger.append(R)
    return acts, np.array(ledger)


def row_actions(actions, n_layers, n_kv_heads, recent):
    """Per-row physical actions of the generated tokens. PASK §3.2: the
    layers of a group share its action but keep their own KV tensors, recent
    tokens remain high precision and scheduled releases happen after they
    leave the window (Appendix B.3 accounts for that window apart from the
    scheduled payload, so the ledger still charges the scheduled action).

    actions: [n_seq][n_tok][n_groups] scheduled actions (control_sequence).
    Returns [n_seq][n_layers][n_kv_heads][n_tok]: H for the last ``recent``
    tokens, else the action of the layer's group (oracle.policy.layer_group).
    """
    acts = np.asarray(actions)
    n_seq, n_tok, _ = acts.shape
    out = np.empty((n_seq, n_layers, n_kv_heads, n_tok), np.uint8)
    for n in range(n_seq):
        for l in range(n_layers):
            row = row_action(acts[n], l, n_layers, recent)
            for h in range(n_kv_heads):
                out[n, l, h] = row
    return out


def row_action(actions_n, layer, n_layers, recent):
    """row_actions for one sequence's [n_tok][n_groups] schedule and one layer."""
    from oracle.policy import layer_group
    acts = np.asarray(actions_n)
    n_tok, n_groups = acts.shape
    g = layer_group(layer, n_layers, n_groups)
    return np.array([H_ACT if t >= n_tok - recent else acts[t, g] for t in range(n_tok)], np.uint8)
